// chain_verify.hip -- chain verification of speculative sampling on gfx950.
//
// What is computed ("10.6 投机解码" §10.6.1 steps 1-5; "KV Cache 优化（四）" §4-§6): for
// each sequence, the tempered, top-p-filtered laws p_k (target) and q_k (draft), the
// acceptance test u < min(1, p_k(d_k)/q_k(d_k)) from left to right, the first rejection,
// the residual draw from max(0, p_k - q_k) or the bonus draw from p_{gamma+1}, and the
// committed-length pointer. See include/spec_verify.h for the exact contract.
//
// Structure
//  1. chain_row_kernel -- one wave per (sequence b, position k) item, k = 1..gamma_b+1.
//     The wave streams the target row and (for k <= gamma_b) the draft row of the item
//     together from HBM once, with 16-byte loads, 8 vectors per row in flight per lane:
//       - per-lane online max / sum of exp2((l - m) * log2(e)/T) (one rescale per trip);
//       - with top-p: the index of every 8-logit vector whose max is within kCaptureK*T of
//         the wave's running max is kept in LDS (a superset of the final window
//         m - kCaptureK*T); the end phase reads those few vectors again;
//       - greedy rows (T = 0): max with the lowest index only.
//     The end phase (wave reductions only) gives m, Z, the nucleus threshold t* (binary
//     search over bf16 keys on fixed-point masses of the captured elements; an exact
//     16-pass search over the whole row if the window did not hold the nucleus), p_k(d_k),
//     q_k(d_k), the acceptance decision, and a sorted nucleus list (<= kNucMax tokens) for
//     the resolve step.
//  2. chain_resolve_kernel -- one 256-thread workgroup per sequence: first rejection by a
//     ballot over the items' decisions, then the residual or bonus draw -- from the nucleus
//     lists when both are kept (no logits touched), else by one pass over the row pair with
//     per-tile sums, a tile scan and an in-tile scan (ascending token id) -- and the outputs.
#include <math.h>

#include "row_ops.h"
#include "spec_device.h"
#include "specv_internal.h"

namespace specv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Top-p capture window: logits within kCaptureK * T of the row max (weight >= e^-7 of the
// largest). Rows whose nucleus reaches further down take the exact multi-pass search.
constexpr float kCaptureK = 7.0f;
constexpr int kCapV = 1024;   // captured 8-logit vector indices per row
constexpr int kHist = 512;    // key offsets below the row max resolved by the window search
constexpr int kResolveThreads = 256;
constexpr int kMaxTiles = 1024;  // 64-vector tiles per row in the resolve pass (V <= 2^19)
constexpr double kFix = 17592186044416.0;  // 2^44: fixed-point scale of masses
// A trip whose weights, taken against the lane's previous maximum, may exceed 2^100 is
// recomputed against its own maximum (first trip of a row, or a large jump at small T).
constexpr float kTripBig = 1.2676506e30f;  // 2^100

struct ChainParams {
  const uint16_t* target;
  const uint16_t* draft;
  const int32_t* cu;
  const int32_t* tokens;
  const float* temp;
  const float* topp;
  const uint32_t* sid;
  int32_t* committed;
  int32_t* out_tokens;
  int32_t* num_acc;
  int32_t* flags_out;
  float* probe_rows;
  float* probe_seq;
  const float* ovr;
  RowRec* rec;
  NucEntry* nuc;  // [n_items][2][kNucMax]
  int32_t B, V, stride, nvec, max_gamma, n_draft, lead;
  uint32_t seed_lo, seed_hi;
};

// Indices of the captured vectors; the vectors themselves (about 1% of the row) are read
// again in the end phase.
struct CapBuf {
  int32_t vidx[kCapV];
};

// Threshold search state: fixed-point mass per key offset below the row max (integer
// additions, so the sums do not depend on the order of the atomics), and the staging area
// of a nucleus list.
struct SelBuf {
  unsigned long long hist[kHist];
  uint32_t sidx[kWave];
  float sw[kWave];
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t fixw(float w) {
  return (uint64_t)((double)w * kFix);
}

// Parameters checked on their bit patterns (NaN fails every test). T: >= 0 (or -0), not NaN;
// +inf is allowed (a flat law).
__device__ __forceinline__ bool temperature_ok(float T) {
  const uint32_t b = __float_as_uint(T);
  return (b & 0x80000000u) ? (b == 0x80000000u) : (b <= 0x7F800000u);
}
// top_p: 0 < P <= 1.
__device__ __forceinline__ bool top_p_ok(float P) {
  const uint32_t b = __float_as_uint(P);
  return b != 0u && b <= 0x3F800000u;
}

// Sequence parameters shared by the two kernels.
struct SeqInfo {
  int32_t g;       // gamma_b
  int32_t t0;      // first target row
  int32_t d0;      // first draft row
  int32_t L;       // committed length on entry
  uint32_t id;     // Philox stream id
  float T, P;
  bool bad_param;
};

__device__ __forceinline__ SeqInfo seq_info(const ChainParams& P, int b) {
  SeqInfo s;
  const int c0 = P.cu[b], c1 = P.cu[b + 1];
  s.g = c1 - c0;
  s.t0 = c0 + b;
  s.d0 = c0;
  s.L = P.committed[b];
  s.id = P.sid ? P.sid[b] : (uint32_t)b;
  s.T = P.temp[b];
  s.P = P.topp ? P.topp[b] : 1.0f;
  s.bad_param = !(s.g >= 0 && s.g <= P.max_gamma && c0 >= 0 && c1 <= P.n_draft) ||
                !temperature_ok(s.T) || !top_p_ok(s.P) ||
                (s.T != 0.0f && s.g > 0 && P.draft == nullptr);
  if (s.T == 0.0f) s.T = 0.0f;  // -0 is greedy too
  return s;
}

// ----------------------------------------------------------------------------------------
// Row statistics (T > 0)
// ----------------------------------------------------------------------------------------

struct LaneAcc {
  float m = -INFINITY;   // running max of this lane's logits
  float s = 0.0f;        // sum of exp2((l - m) * c) over this lane's logits
  float wm = -INFINITY;  // running max of the whole wave (capture threshold)
  int cnt = 0;           // captured vectors (wave-uniform)
};

// Weight of one logit relative to a reference: the same expression everywhere, so that
// masses and probabilities computed in different places agree bit for bit.
__device__ __forceinline__ float weight(float l, float c, float nref) {
  return __builtin_amdgcn_exp2f(fmaf(l, c, nref));
}

// One trip (kU vectors of one row) into the lane's running (m, s). The weights are taken
// against the lane's previous maximum; only when the trip raises it (rare after the first
// trips) is the trip's partial sum re-referenced, or recomputed when it may have overflowed.
template <bool CAPTURE>
__device__ __forceinline__ void consume_trip(const uint4 d[kU], int v0, int lane, float c,
                                             float capw, LaneAcc& a, CapBuf* cap) {
  const float ref = (a.m == -INFINITY) ? 0.0f : a.m;
  const float nref = -ref * c;
  float vm[kU];
  float st = 0.0f;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float x[8];
    unpack8(d[u], x);
    vm[u] = max8(x);
#pragma unroll
    for (int e = 0; e < 8; ++e) st += weight(x[e], c, nref);
  }
  static_assert(kU == 4, "trip max below assumes four vectors per trip");
  const float tm = vmax3(vmax3(vm[0], vm[1], vm[2]), vm[3], vm[3]);
  if (tm > a.m) {
    if (st < kTripBig) {
      st *= __builtin_amdgcn_exp2f((ref - tm) * c);
    } else {
      st = 0.0f;
      const float nt = -tm * c;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float x[8];
        unpack8(d[u], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) st += weight(x[e], c, nt);
      }
    }
    a.s *= __builtin_amdgcn_exp2f((a.m - tm) * c);  // 0 while a.m = -inf (a.s = 0 then)
    a.m = tm;
  }
  a.s += st;
  if (CAPTURE) {
    a.wm = fmaxf(a.wm, wave_max(tm));
    const float thr = a.wm - capw;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool want = vm[u] >= thr;
      const uint64_t mask = __ballot(want);
      if (mask) {
        const int slot = a.cnt + (int)lanes_below(mask);
        if (want && slot < kCapV) cap->vidx[slot] = v0 + u * kWave + lane;
        a.cnt += __popcll(mask);
      }
    }
  }
}

// Wave-wide (m, Z) of a row from the lanes' running (m, s).
__device__ __forceinline__ void finish_mz(const LaneAcc& a, float c, float& M, float& Z) {
  M = wave_max(a.m);
  const float ref = (M == -INFINITY) ? 0.0f : M;
  const float s = (a.m == -INFINITY) ? 0.0f : a.s * __builtin_amdgcn_exp2f((a.m - ref) * c);
  Z = wave_sum(s);
}

struct TopP {
  float t;     // threshold logit (-inf: keep all)
  float zs;    // normaliser over the kept set
  int nuc;     // kept count if the list was written, else -1
  bool slow;   // exact multi-pass search ran
};

// Appends the flagged lanes' (idx, w) to the staging list in LDS, in lane order. Returns the
// new length (a length above kWave means the list overflowed and is incomplete).
__device__ __forceinline__ int stage_append(bool in, uint32_t idx, float w, int n, SelBuf* sb) {
  const uint64_t mask = __ballot(in);
  const int slot = n + (int)lanes_below(mask);
  if (in && slot < kWave) {
    sb->sidx[slot] = idx;
    sb->sw[slot] = w;
  }
  return n + __popcll(mask);
}

// Writes the staged list (n <= kNucMax entries) to the workspace sorted by token id.
__device__ __forceinline__ void write_sorted_list(NucEntry* out, int n, const SelBuf* sb,
                                                  int lane) {
  const uint32_t idx = lane < n ? sb->sidx[lane] : 0xFFFFFFFFu;
  const float w = lane < n ? sb->sw[lane] : 0.0f;
  int rank = 0;
  for (int j = 0; j < n; ++j) rank += (__shfl(idx, j, kWave) < idx) ? 1 : 0;
  if (lane < n) out[rank] = NucEntry{(int32_t)idx, w};
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)v, o, kWave);
    const uint32_t hi = __shfl_up((uint32_t)(v >> 32), o, kWave);
    if (lane >= o) v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// First bucket (in increasing index = decreasing logit) at which base + the cumulative mass
// reaches thr; -1 if the buckets never get there. *cum receives the cumulative mass at that
// bucket (or base + the total). nb is a multiple of 64; each lane scans nb/64 buckets.
__device__ int hist_crossing(const unsigned long long* h, int nb, uint64_t thr, uint64_t base,
                             uint64_t* cum, int lane) {
  const int per = nb / kWave;
  uint64_t mine = 0;
  for (int j = 0; j < per; ++j) mine += h[lane * per + j];
  const uint64_t incl = base + wave_incl_scan_u64(mine, lane);
  const uint64_t hit = __ballot(incl >= thr);
  if (!hit) {
    *cum = __shfl(incl, kWave - 1, kWave);
    return -1;
  }
  const int src = __ffsll((long long)hit) - 1;
  int o = -1;
  uint64_t c = 0;
  if (lane == src) {
    c = incl - mine;
    for (int j = 0; j < per; ++j) {
      c += h[lane * per + j];
      if (c >= thr) {
        o = lane * per + j;
        break;
      }
    }
  }
  o = __shfl(o, src, kWave);
  const uint32_t lo = __shfl((uint32_t)c, src, kWave), hi = __shfl((uint32_t)(c >> 32), src, kWave);
  *cum = ((uint64_t)hi << 32) | lo;
  return o;
}

// Nucleus list of a row once t is known: every logit >= t, from the given vectors.
template <typename VecAt>
__device__ int collect_list(VecAt vec_at, int nv, int V, float t, float c, float nref,
                            SelBuf* sb, int lane) {
  int n = 0;
  for (int i0 = 0; i0 < nv && n <= kNucMax; i0 += kWave) {
    const int i = i0 + lane;
    float x[8];
    int vi = 0;
    if (i < nv) {
      vi = vec_at(i);
      unpack8(vec_at.load(vi), x);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = i < nv && (vi * 8 + e < V) && x[e] >= t;
      n = stage_append(in, (uint32_t)(vi * 8 + e), in ? weight(x[e], c, nref) : 0.0f, n, sb);
    }
  }
  return n;
}

struct AllVecs {
  const uint4* row;
  __device__ int operator()(int i) const { return i; }
  __device__ uint4 load(int vi) const { return row[vi]; }
};
struct CapVecs {
  const uint4* row;
  const CapBuf* cap;
  __device__ int operator()(int i) const { return cap->vidx[i]; }
  __device__ uint4 load(int vi) const { return row[vi]; }
};

__device__ void finish_list(TopP& r, int n, NucEntry* list, SelBuf* sb, int lane) {
  __syncthreads();
  if (n > kNucMax) {
    r.nuc = -1;
  } else {
    r.nuc = n;
    write_sorted_list(list, n, sb, lane);
  }
  __syncthreads();
}

// Exact threshold search over the whole row: the largest bf16 key t with
// mass(key >= t) >= thrP, by a 256-bucket fixed-point histogram of the key offset's high byte
// and then of its low byte inside the chosen bucket (two passes), plus one pass for the
// nucleus list. Used when the capture window missed the nucleus.
__device__ TopP topp_full_row(const uint4* __restrict__ row, int nvec, int V, float c,
                              float M, uint64_t thrP, NucEntry* list, SelBuf* sb, int lane) {
  const float nref = -M * c;
  const uint32_t kM = key_of(M);
  TopP r;
  r.slow = true;
  uint64_t cum = 0, base = 0;
  int hi_b = -1, o_star = -1;
  for (int pass = 0; pass < 2; ++pass) {
    for (int j = lane; j < kHist; j += kWave) sb->hist[j] = 0ull;
    __syncthreads();
    for (int v = lane; v < nvec; v += kWave) {
      float x[8];
      unpack8(row[v], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (v * 8 + e >= V) continue;
        const uint32_t o = kM - key_of(x[e]);
        if (pass == 1 && (int)(o >> 8) != hi_b) continue;
        const uint64_t fw = fixw(weight(x[e], c, nref));
        if (fw) atomicAdd(&sb->hist[pass == 0 ? (o >> 8) : (o & 255u)], (unsigned long long)fw);
      }
    }
    __syncthreads();
    if (pass == 0) {
      hi_b = hist_crossing(sb->hist, 256, thrP, 0, &cum, lane);
      if (hi_b < 0) break;  // rounding left the whole row just below P: keep everything
      base = cum - sb->hist[hi_b];
    } else {
      o_star = hi_b * 256 + hist_crossing(sb->hist, 256, thrP, base, &cum, lane);
    }
    __syncthreads();
  }
  if (hi_b < 0) {
    r.t = -INFINITY;
  } else {
    r.t = value_of_key(kM - (uint32_t)o_star);
  }
  r.zs = (float)((double)cum / kFix);
  const int n = collect_list(AllVecs{row}, nvec, V, r.t, c, nref, sb, lane);
  finish_list(r, n, list, sb, lane);
  return r;
}

// Threshold search on the captured window: fixed-point masses of the captured logits in a
// histogram over key offsets below the row max; the first offset at which the running mass
// reaches P * Z is the threshold. Falls back to the whole row when the window overflowed or
// does not reach mass P within kHist offsets.
__device__ TopP topp_select(const uint4* __restrict__ row, int nvec, int V, float c, float P,
                            float M, float Z, int cnt, const CapBuf* cap, SelBuf* sb,
                            NucEntry* list, int lane) {
  const float capw = kCaptureK * (kLog2e / c);  // kCaptureK * T in logit units
  const float theta = M - capw;
  const float nref = -M * c;
  const uint64_t thrP = (uint64_t)((double)P * (double)Z * kFix);
  const uint32_t kM = key_of(M);
  const int nv = min(cnt, kCapV);
  for (int j = lane; j < kHist; j += kWave) sb->hist[j] = 0ull;
  __syncthreads();
  for (int i0 = 0; i0 < nv; i0 += kWave) {
    const int i = i0 + lane;
    if (i >= nv) break;
    const int vi = cap->vidx[i];
    float x[8];
    unpack8(row[vi], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (vi * 8 + e >= V || !(x[e] >= theta)) continue;
      const uint32_t o = kM - key_of(x[e]);
      if (o < (uint32_t)kHist)
        atomicAdd(&sb->hist[o], (unsigned long long)fixw(weight(x[e], c, nref)));
    }
  }
  __syncthreads();
  uint64_t zs = 0;
  const int o_star = (cnt <= kCapV) ? hist_crossing(sb->hist, kHist, thrP, 0, &zs, lane) : -1;
  __syncthreads();
  if (o_star < 0) return topp_full_row(row, nvec, V, c, M, thrP, list, sb, lane);
  TopP r;
  r.slow = false;
  r.t = value_of_key(kM - (uint32_t)o_star);
  r.zs = (float)((double)zs / kFix);
  const int n = collect_list(CapVecs{row, cap}, nv, V, r.t, c, nref, sb, lane);
  finish_list(r, n, list, sb, lane);
  return r;
}

// ----------------------------------------------------------------------------------------
// Kernel 1: one wave per (sequence, position) item.
// ----------------------------------------------------------------------------------------
// TOPP: the batch carries a top-p array, so capture buffers live in (dynamic) LDS.
template <bool TOPP>
__global__ __launch_bounds__(kWave) void chain_row_kernel(ChainParams P) {
  extern __shared__ uint4 smem_dyn[];
  CapBuf* cap = reinterpret_cast<CapBuf*>(smem_dyn);
  SelBuf* sb = reinterpret_cast<SelBuf*>(cap + 2);
  const int lane = lane_id();
  const int per = P.max_gamma + 1;
  const int b = blockIdx.x / per;
  const int k = blockIdx.x % per + 1;  // 1-based position
  const SeqInfo s = seq_info(P, b);
  if (s.bad_param || k > s.g + 1) return;
  const int trow = s.t0 + k - 1;
  const bool pair = k <= s.g;
  const int drow = s.d0 + k - 1;
  RowRec* rec = P.rec + trow;
  NucEntry* lists = P.nuc + (size_t)trow * 2 * kNucMax;
  const uint4* rp = reinterpret_cast<const uint4*>(P.target + (size_t)trow * P.stride);
  int flags = 0;
  int d = -1;
  if (pair) {
    d = P.tokens[drow];
    if (d < 0 || d >= P.V) flags |= SPEC_FLAG_BAD_TOKEN;
  }

  if (s.T == 0.0f) {  // greedy: argmax of the target row; q is not read
    const int am = row_argmax(rp, P.nvec, P.V, lane);
    if (lane == 0) {
      const int acc = (pair && !(flags & SPEC_FLAG_BAD_TOKEN) && d == am) ? 1 : 0;
      RowRec r;
      r.m[0] = r.m[1] = 0.0f;
      r.z[0] = r.z[1] = 1.0f;
      r.t[0] = r.t[1] = -INFINITY;
      r.pd = (pair && d == am) ? 1.0f : 0.0f;
      r.qd = NAN;
      r.argmax = am;
      r.accept = acc;
      r.flags = flags;
      r.nuc[0] = r.nuc[1] = -1;
      r.valid = 1;
      r.pad[0] = r.pad[1] = 0;
      *rec = r;
      if (pair && P.probe_rows) {
        P.probe_rows[(size_t)drow * 3 + 0] = r.pd;
        P.probe_rows[(size_t)drow * 3 + 1] = NAN;
        P.probe_rows[(size_t)drow * 3 + 2] = (float)acc;
      }
    }
    return;
  }

  const float c = kLog2e / s.T;
  const bool topp = TOPP && s.P < 1.0f;
  const float capw = kCaptureK * s.T;
  const uint4* rq = pair ? reinterpret_cast<const uint4*>(P.draft + (size_t)drow * P.stride)
                         : nullptr;
  LaneAcc ap, aq;
  // Double-buffered: the next trip's loads are in flight while this trip is consumed.
  constexpr int kStep = kU * kWave;
  uint4 p0[kU], q0[kU], p1[kU], q1[kU];
  load_trip(rp, 0, P.nvec, lane, p0);
  if (pair) load_trip(rq, 0, P.nvec, lane, q0);
  auto consume = [&](uint4* dp, uint4* dq, int v0) {
    mask_tail(dp, v0, P.nvec, P.V, lane);
    if (topp) consume_trip<true>(dp, v0, lane, c, capw, ap, &cap[0]);
    else consume_trip<false>(dp, v0, lane, c, capw, ap, nullptr);
    if (pair) {
      mask_tail(dq, v0, P.nvec, P.V, lane);
      if (topp) consume_trip<true>(dq, v0, lane, c, capw, aq, &cap[1]);
      else consume_trip<false>(dq, v0, lane, c, capw, aq, nullptr);
    }
  };
  for (int v0 = 0; v0 < P.nvec; v0 += 2 * kStep) {
    const int v1 = v0 + kStep;
    if (v1 < P.nvec) {
      load_trip(rp, v1, P.nvec, lane, p1);
      if (pair) load_trip(rq, v1, P.nvec, lane, q1);
    }
    consume(p0, q0, v0);
    if (v1 >= P.nvec) break;
    const int v2 = v1 + kStep;
    if (v2 < P.nvec) {
      load_trip(rp, v2, P.nvec, lane, p0);
      if (pair) load_trip(rq, v2, P.nvec, lane, q0);
    }
    consume(p1, q1, v1);
  }
  __syncthreads();
  float Mp, Zp, Mq = 0.0f, Zq = 1.0f;
  finish_mz(ap, c, Mp, Zp);
  if (pair) finish_mz(aq, c, Mq, Zq);
  TopP tp{-INFINITY, Zp, -1, false}, tq{-INFINITY, Zq, -1, false};
  if (topp) {
    tp = topp_select(rp, P.nvec, P.V, c, s.P, Mp, Zp, ap.cnt, &cap[0], sb, lists, lane);
    if (pair)
      tq = topp_select(rq, P.nvec, P.V, c, s.P, Mq, Zq, aq.cnt, &cap[1], sb, lists + kNucMax,
                       lane);
    if (tp.slow || tq.slow) flags |= SPEC_FLAG_TOPP_SLOW;
  }
  float pd = NAN, qd = NAN, a = NAN;
  int acc = 0;
  if (pair && !(flags & SPEC_FLAG_BAD_TOKEN)) {
    const uint16_t* tr = P.target + (size_t)trow * P.stride;
    const uint16_t* dr = P.draft + (size_t)drow * P.stride;
    const float lp = __uint_as_float((uint32_t)tr[d] << 16);
    const float lq = __uint_as_float((uint32_t)dr[d] << 16);
    pd = (lp >= tp.t) ? weight(lp, c, -Mp * c) / tp.zs : 0.0f;
    qd = (lq >= tq.t) ? weight(lq, c, -Mq * c) / tq.zs : 0.0f;
    if (qd > 0.0f) {
      a = fminf(1.0f, pd / qd);
    } else {
      a = pd > 0.0f ? 1.0f : 0.0f;
      flags |= SPEC_FLAG_Q_ZERO;
    }
    const float u = P.ovr ? P.ovr[(size_t)trow * 2]
                          : uniform24(P.seed_lo, P.seed_hi, s.id, (uint32_t)(s.L + k),
                                      SPEC_PURPOSE_ACCEPT);
    acc = (u < a) ? 1 : 0;
  }
  if (lane == 0) {
    RowRec r;
    r.m[0] = Mp;
    r.m[1] = Mq;
    r.z[0] = tp.zs;
    r.z[1] = tq.zs;
    r.t[0] = tp.t;
    r.t[1] = tq.t;
    r.pd = pd;
    r.qd = qd;
    r.argmax = -1;
    r.accept = acc;
    r.flags = flags;
    r.nuc[0] = topp ? tp.nuc : -1;
    r.nuc[1] = (topp && pair) ? tq.nuc : -1;
    r.valid = 1;
    r.pad[0] = r.pad[1] = 0;
    *rec = r;
    if (pair && P.probe_rows) {
      P.probe_rows[(size_t)drow * 3 + 0] = pd;
      P.probe_rows[(size_t)drow * 3 + 1] = qd;
      P.probe_rows[(size_t)drow * 3 + 2] = a;
    }
  }
}

// ----------------------------------------------------------------------------------------
// Kernel 2: per-sequence resolve.
// ----------------------------------------------------------------------------------------

struct Draw {
  int token;
  float total;  // mass of the weights drawn from (R for a residual, ~1 for p itself)
  float wtok;   // weight of the drawn token
};

// One wave: inverse-CDF draw over a nucleus list sorted by token id (<= 64 entries).
// residual: weights max(0, p - q) with q looked up in q's list; else p.
__device__ Draw draw_from_lists(const NucEntry* pl, int np, float zp, const NucEntry* ql,
                                int nq, float zq, bool residual, float u, int lane) {
  int idx = 0x7FFFFFFF;
  float w = 0.0f;
  if (lane < np) {
    const NucEntry e = pl[lane];
    idx = e.idx;
    w = e.w / zp;
  }
  if (residual) {
    const NucEntry eq = lane < nq ? ql[lane] : NucEntry{-1, 0.0f};
    float wq = 0.0f;
    for (int j = 0; j < nq; ++j) {
      const int qi = __shfl(eq.idx, j, kWave);
      const float qw = __shfl(eq.w, j, kWave);
      if (qi == idx) wq = qw / zq;
    }
    w = fmaxf(0.0f, w - wq);
  }
  const float incl = wave_incl_scan(w, lane);
  const float total = __shfl(incl, kWave - 1, kWave);
  const float x = u * total;
  const uint64_t hit = __ballot(lane < np && incl > x);
  int src;
  if (hit) {
    src = __ffsll((long long)hit) - 1;
  } else {  // rounding left u*total at or past the end: the last token with weight
    const uint64_t pos = __ballot(lane < np && w > 0.0f);
    src = pos ? 63 - __clzll((long long)pos) : 0;
  }
  Draw d;
  d.token = __shfl(idx, src, kWave);
  d.wtok = __shfl(w, src, kWave);
  d.total = total;
  return d;
}

struct RowLaw {
  const uint4* row;
  float c, nref, t, z;
};

__device__ __forceinline__ void law_weights(const RowLaw& L, const uint4& d, float w[8]) {
  float x[8];
  unpack8(d, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = (x[e] >= L.t) ? weight(x[e], L.c, L.nref) / L.z : 0.0f;
}

// Weights of vector v: p, or max(0, p - q). Logits past V weigh 0.
__device__ __forceinline__ void vec_weights(const RowLaw& Lp, const RowLaw& Lq, bool residual,
                                            int v, int nvec, int V, float w[8]) {
  if (v >= nvec) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = 0.0f;
    return;
  }
  law_weights(Lp, Lp.row[v], w);
  if (residual) {
    float wq[8];
    law_weights(Lq, Lq.row[v], wq);
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = fmaxf(0.0f, w[e] - wq[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (v * 8 + e >= V) w[e] = 0.0f;
}

// All threads of the workgroup: inverse-CDF draw over a whole row (pair) in token order.
// Pass 1 stores per-tile sums (a tile = 64 vectors = 512 logits, one coalesced wave load);
// wave 0 scans the tile sums, then re-reads the chosen tile and scans it.
__device__ Draw draw_from_rows(const RowLaw& Lp, const RowLaw& Lq, bool residual, int nvec,
                               int V, float u, float* tile_sum, int* sh_i, float* sh_f) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int nw = kResolveThreads / kWave;
  const int ntiles = (nvec + kWave - 1) / kWave;
  int last = -1;  // last token with positive weight seen by this lane
  for (int g = wid; g < ntiles; g += nw) {
    const int v = g * kWave + lane;
    float w[8];
    vec_weights(Lp, Lq, residual, v, nvec, V, w);
    float ls = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ls += w[e];
      if (w[e] > 0.0f) last = v * 8 + e;
    }
    const float ts = wave_sum(ls);
    if (lane == 0) tile_sum[g] = ts;
  }
  last = wave_max_i(last);
  if (lane == 0) sh_i[wid] = last;
  __syncthreads();
  Draw d;
  if (wid == 0) {
    int lst = -1;
    for (int i = 0; i < nw; ++i) lst = max(lst, sh_i[i]);
    const int per = (ntiles + kWave - 1) / kWave;
    const int g0 = lane * per, g1 = min(ntiles, g0 + per);
    float mine = 0.0f;
    for (int g = g0; g < g1; ++g) mine += tile_sum[g];
    const float incl = wave_incl_scan(mine, lane);
    const float total = __shfl(incl, kWave - 1, kWave);
    const float x = u * total;
    const float excl = incl - mine;
    // the tile holding x: first lane whose range ends past x, then its tiles in order
    int gstar = -1;
    float base = 0.0f;
    const uint64_t hit = __ballot(incl > x && g1 > g0);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      if (lane == src) {
        float cum = excl;
        for (int g = g0; g < g1; ++g) {
          if (cum + tile_sum[g] > x) {
            gstar = g;
            break;
          }
          cum += tile_sum[g];
        }
        if (gstar < 0) {  // rounding: take this lane's last tile with mass
          for (int g = g1 - 1; g >= g0; --g)
            if (tile_sum[g] > 0.0f) {
              gstar = g;
              break;
            }
          cum = x;  // forces the in-tile fallback below
        }
        base = cum;
      }
      gstar = __shfl(gstar, src, kWave);
      base = __shfl(base, src, kWave);
    }
    int token = lst < 0 ? 0 : lst;
    float wtok = 0.0f;
    if (gstar >= 0) {
      const int v = gstar * kWave + lane;
      float w[8];
      vec_weights(Lp, Lq, residual, v, nvec, V, w);
      float ls = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ls += w[e];
      const float li = wave_incl_scan(ls, lane);
      const float le = base + (li - ls);
      const uint64_t lh = __ballot(le + ls > x && ls > 0.0f);
      int tok = -1;
      float wt = 0.0f;
      if (lh) {
        const int src = __ffsll((long long)lh) - 1;
        if (lane == src) {
          float cum = le;
          for (int e = 0; e < 8; ++e) {
            cum += w[e];
            if (w[e] > 0.0f && cum > x) {
              tok = v * 8 + e;
              wt = w[e];
              break;
            }
          }
          if (tok < 0) {
            for (int e = 7; e >= 0; --e)
              if (w[e] > 0.0f) {
                tok = v * 8 + e;
                wt = w[e];
                break;
              }
          }
        }
        tok = __shfl(tok, src, kWave);
        wt = __shfl(wt, src, kWave);
      } else {  // rounding inside the tile: its last token with weight
        int lp = -1;
        float lw = 0.0f;
        for (int e = 0; e < 8; ++e)
          if (w[e] > 0.0f) {
            lp = v * 8 + e;
            lw = w[e];
          }
        const int best = wave_max_i(lp);
        const uint64_t own = __ballot(lp == best && best >= 0);
        if (own) {
          const int src = __ffsll((long long)own) - 1;
          tok = best;
          wt = __shfl(lw, src, kWave);
        }
      }
      if (tok >= 0) {
        token = tok;
        wtok = wt;
      }
    } else if (lst >= 0) {  // u*total at or past the end: the last token with weight
      const int v = lst / 8;
      float w[8];
      vec_weights(Lp, Lq, residual, v, nvec, V, w);
      wtok = w[lst & 7];
    }
    if (lane == 0) {
      sh_i[0] = token;
      sh_f[0] = total;
      sh_f[1] = wtok;
    }
  }
  __syncthreads();
  d.token = sh_i[0];
  d.total = sh_f[0];
  d.wtok = sh_f[1];
  __syncthreads();
  return d;
}

__global__ __launch_bounds__(kResolveThreads) void chain_resolve_kernel(ChainParams P) {
  __shared__ float tile_sum[kMaxTiles];
  __shared__ int sh_i[8];
  __shared__ float sh_f[8];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const SeqInfo s = seq_info(P, b);
  __syncthreads();  // every thread has read committed_len[b] before thread 0 rewrites it
  // gamma_b and cu_gamma in range: the draft tokens of the sequence can be read
  const int c0 = P.cu[b], c1 = P.cu[b + 1];
  const bool cu_ok = c1 - c0 >= 0 && c1 - c0 <= P.max_gamma && c0 >= 0 && c1 <= P.n_draft;
  const bool in_g = cu_ok && lane < s.g;
  int tok = 0, acc = 1, rflags = 0;
  if (in_g) tok = P.tokens[s.d0 + lane];
  const bool bad_tok = __ballot(in_g && (tok < 0 || tok >= P.V)) != 0;
  if (s.bad_param || bad_tok) {  // no progress: nothing emitted, pointer unchanged
    if (tid == 0) {
      P.num_acc[b] = 0;
      if (P.flags_out)
        P.flags_out[b] = (bad_tok ? SPEC_FLAG_BAD_TOKEN : 0) |
                         (s.bad_param ? SPEC_FLAG_BAD_PARAM : 0);
      if (P.probe_seq) {
        P.probe_seq[2 * b] = NAN;
        P.probe_seq[2 * b + 1] = NAN;
      }
    }
    return;
  }
  // decisions and first rejection (gamma_b <= 64: one wave ballot)
  if (in_g) {
    const RowRec& r = P.rec[s.t0 + lane];
    acc = r.accept;
    rflags = r.flags;
  }
  const uint64_t rej = __ballot(in_g && acc == 0);
  const int n_acc = rej ? __ffsll((long long)rej) - 1 : s.g;
  const int kstar = n_acc + 1;
  int flags = 0;
  {
    int f = (lane < min(kstar, s.g)) ? rflags : 0;
    for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, kWave);
    flags = f & (SPEC_FLAG_Q_ZERO | SPEC_FLAG_TOPP_SLOW);
  }
  const int trow = s.t0 + kstar - 1;
  const RowRec r = P.rec[trow];
  flags |= r.flags & SPEC_FLAG_TOPP_SLOW;
  int y;
  float R = NAN, py;
  if (s.T == 0.0f) {
    y = r.argmax;
    py = 1.0f;
  } else {
    const bool residual = kstar <= s.g;
    const float u = P.ovr ? P.ovr[(size_t)trow * 2 + 1]
                          : uniform24(P.seed_lo, P.seed_hi, s.id, (uint32_t)(s.L + kstar),
                                      residual ? SPEC_PURPOSE_RESIDUAL : SPEC_PURPOSE_BONUS);
    const float c = kLog2e / s.T;
    const NucEntry* lists = P.nuc + (size_t)trow * 2 * kNucMax;
    RowLaw Lp{reinterpret_cast<const uint4*>(P.target + (size_t)trow * P.stride), c,
              -r.m[0] * c, r.t[0], r.z[0]};
    RowLaw Lq{residual ? reinterpret_cast<const uint4*>(P.draft + (size_t)(s.d0 + kstar - 1) *
                                                        P.stride)
                       : nullptr,
              c, -r.m[1] * c, r.t[1], r.z[1]};
    Draw d;
    const bool lists_p = r.nuc[0] >= 0, lists_pq = lists_p && r.nuc[1] >= 0;
    if (residual) {
      if (lists_pq) {
        if (wid == 0) {
          d = draw_from_lists(lists, r.nuc[0], r.z[0], lists + kNucMax, r.nuc[1], r.z[1], true,
                              u, lane);
          if (lane == 0) {
            sh_i[0] = d.token;
            sh_f[0] = d.total;
            sh_f[1] = d.wtok;
          }
        }
        __syncthreads();
        d = Draw{sh_i[0], sh_f[0], sh_f[1]};
        __syncthreads();
      } else {
        d = draw_from_rows(Lp, Lq, true, P.nvec, P.V, u, tile_sum, sh_i, sh_f);
      }
      R = d.total;
      if (!(d.total > 0.0f)) flags |= SPEC_FLAG_RESID_FALLBACK;
    }
    if (!residual || !(d.total > 0.0f)) {
      if (lists_p) {
        if (wid == 0) {
          d = draw_from_lists(lists, r.nuc[0], r.z[0], nullptr, 0, 1.0f, false, u, lane);
          if (lane == 0) {
            sh_i[0] = d.token;
            sh_f[0] = d.total;
            sh_f[1] = d.wtok;
          }
        }
        __syncthreads();
        d = Draw{sh_i[0], sh_f[0], sh_f[1]};
      } else {
        d = draw_from_rows(Lp, Lq, false, P.nvec, P.V, u, tile_sum, sh_i, sh_f);
      }
      y = d.token;
      py = d.wtok;
    } else {
      y = d.token;
      py = d.wtok / d.total;
    }
  }
  if (wid == 0) {
    if (lane < n_acc) P.out_tokens[s.t0 + lane] = tok;
    if (lane == 0) {
      P.out_tokens[s.t0 + n_acc] = y;
      P.num_acc[b] = n_acc;
      P.committed[b] = s.L + P.lead + n_acc;
      if (P.flags_out) P.flags_out[b] = flags;
      if (P.probe_seq) {
        P.probe_seq[2 * b] = R;
        P.probe_seq[2 * b + 1] = py;
      }
    }
  }
}

}  // namespace

size_t chain_workspace_bytes(int32_t batch, int32_t total_draft_rows, int32_t vocab) {
  (void)vocab;
  const size_t items = (size_t)total_draft_rows + (size_t)batch;
  return align256(items * sizeof(RowRec)) + align256(items * 2 * kNucMax * sizeof(NucEntry));
}

hipError_t launch_chain(const spec_chain_args& a, void* ws, hipStream_t st) {
  ChainParams P;
  P.target = a.target_logits;
  P.draft = a.draft_logits;
  P.cu = a.cu_gamma;
  P.tokens = a.draft_tokens;
  P.temp = a.temperature;
  P.topp = a.top_p;
  P.sid = a.seq_id;
  P.committed = a.committed_len;
  P.out_tokens = a.out_tokens;
  P.num_acc = a.num_accepted;
  P.flags_out = a.seq_flags;
  P.probe_rows = a.probe_rows;
  P.probe_seq = a.probe_seq;
  P.ovr = a.uniform_override;
  const size_t items = (size_t)a.total_draft_rows + (size_t)a.batch;
  P.rec = reinterpret_cast<RowRec*>(ws);
  P.nuc = reinterpret_cast<NucEntry*>(reinterpret_cast<char*>(ws) +
                                      align256(items * sizeof(RowRec)));
  P.B = a.batch;
  P.V = a.vocab;
  P.stride = a.row_stride;
  P.nvec = (a.vocab + 7) / 8;
  P.max_gamma = a.max_gamma;
  P.n_draft = a.total_draft_rows;
  P.lead = a.lead_slots;
  P.seed_lo = (uint32_t)(a.seed & 0xFFFFFFFFu);
  P.seed_hi = (uint32_t)(a.seed >> 32);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(a.profile_events);
  hipError_t e = hipSuccess;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  const unsigned grid = (unsigned)a.batch * (unsigned)(a.max_gamma + 1);
  if (a.top_p)
    hipLaunchKernelGGL(chain_row_kernel<true>, dim3(grid), dim3(kWave),
                       2 * sizeof(CapBuf) + sizeof(SelBuf), st, P);
  else
    hipLaunchKernelGGL(chain_row_kernel<false>, dim3(grid), dim3(kWave), 0, st, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  hipLaunchKernelGGL(chain_resolve_kernel, dim3((unsigned)a.batch), dim3(kResolveThreads), 0,
                     st, P);
  return hipGetLastError();
}

}  // namespace specv
