// chain_verify.hip -- chain verification of speculative sampling on gfx950.
//
// What is computed ("10.6 投机解码" §10.6.1 steps 1-5; "KV Cache 优化（四）" §4-§6): for
// each sequence, the tempered, top-p-filtered laws p_k (target) and q_k (draft), the
// acceptance test u < min(1, p_k(d_k)/q_k(d_k)) from left to right, the first rejection,
// the residual draw from max(0, p_k - q_k) or the bonus draw from p_{gamma+1}, and the
// committed-length pointer. See include/spec_verify.h for the exact contract.
//
// Structure
//  1. row_stats_kernel -- one workgroup of kRowWgWaves waves per logits row: the target row
//     p_k or the draft row q_k of draft position k = 1..gamma_b, and the bonus row
//     p_{gamma_b+1}. The waves claim the row's trips from an LDS counter (nontemporal 16-byte
//     loads; one trip in flight per wave while capturing, two otherwise), so the row
//     streams from HBM once as one wide sequential read, and the hardware hands rows to CUs
//     as they free up:
//       - per trip (4 KB of the row): its max and its sum of exp2((l - max) * log2(e)/T),
//         each reduced over the wave in a fixed order and kept by trip index, so that the
//         row's (m, Z), combined in trip order, does not depend on which wave took a trip;
//       - with top-p: every 8-logit vector whose max is within kCaptureK*T of the best known
//         lower bound of the row max (the waves share theirs through LDS) is copied to LDS
//         (a superset of the final window m - kCaptureK*T; past kCapN vectors only their
//         indexes are kept, in the workspace), so the end phase touches no HBM;
//       - greedy rows (T = 0): max with the lowest index only.
//     After a workgroup barrier the end phase gives m, Z, the nucleus threshold t*
//     (fixed-point mass histogram over bf16 keys of the captured logits; an exact multi-pass
//     search over the whole row if the window did not hold the nucleus), the draft token's
//     weight, and the nucleus list in token order (<= kNucMax tokens) for the residual draw,
//     filtered from the window logits the histogram pass recorded.
//  2. chain_resolve_kernel -- one workgroup per sequence: p_k(d_k), q_k(d_k) and the
//     acceptance decisions from the row statistics, the first rejection (one ballot), then
//     the residual or bonus draw -- from the nucleus lists when both are kept (their heads
//     are prefetched with the statistics), else by one pass over the row pair with per-tile
//     sums, a tile scan and an in-tile scan (ascending token id) -- and the outputs.
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
// With top-k the window is wider (the K-th largest logit often lies below 7 * T); rows whose
// window still holds fewer than K logits capture again from a lower bound of the K-th largest.
constexpr float kCaptureKTopK = 10.0f;
constexpr int kCapN = 1024;        // captured vectors per row held in LDS
constexpr int kCapG = 1024;        // further captured vector ids per row spilled to the workspace
constexpr int kDepth = 2;          // trips of loads in flight per wave in the row pass
// Rows with captures keep one trip in flight per wave: the capture registers then leave room
// for three workgroups per CU (six waves per SIMD), and the third workgroup's stream covers
// the end phases of the other two.
constexpr int kDepthCap = 1;
constexpr int kRowWgWaves = 8;     // waves of a row-pass workgroup (one row per workgroup)
constexpr int kRowThreads = kRowWgWaves * kWave;
constexpr int kCand = 1024;        // window logits kept as candidates for the nucleus list
constexpr int kHist = 512;         // key offsets below the row max resolved by the window search
// Resolve workgroup shapes (threads, row-pair tiles in flight per wave in the resolve pass):
// one 1024-thread workgroup per CU while the batch fits the CUs, 256-thread workgroups
// beyond (four or more per CU), so that the latency-bound decisions and scans of some
// sequences overlap the row traffic of others.
constexpr int kResolveWide = 1024, kTilesWide = 4;
constexpr int kResolveNarrow = 256, kTilesNarrow = 5;
constexpr int kResolveMaxWaves = kResolveWide / kWave;
constexpr int kNumCus = 256;  // compute units of the chip: one wide workgroup each
constexpr int kMaxTiles = 1024;  // 64-vector tiles per row in the resolve pass (V <= 2^19)
constexpr int kPreRows = 8;      // draft positions whose list heads the resolve prefetches
constexpr int kPre = 64;         // list entries prefetched per row
constexpr double kFix = 17592186044416.0;  // 2^44: fixed-point scale of masses
// Trips of a row at most (V <= 2^19 logits, kU vectors of 8 logits per lane per trip).
constexpr int kMaxTrips = (1 << 19) / (8 * kU * kWave);

struct ChainParams {
  const uint16_t* target;
  const uint16_t* draft;
  const int32_t* cu;
  const int32_t* tokens;
  const float* temp;
  const float* topp;
  const int32_t* topk;
  const int32_t* eos;
  const int32_t* cap;
  const uint32_t* sid;
  int32_t* committed;
  int32_t* out_tokens;
  int32_t* num_acc;
  int32_t* num_emit;
  int32_t* flags_out;
  float* probe_rows;
  float* probe_seq;
  const float* ovr;
  RowStat* stat;    // [n_draft][2]
  NucEntry* nuc;    // [n_draft][2][kNucMax]
  uint16_t* spill;  // [n_draft][2][kCapG]
  int32_t B, V, stride, nvec, max_gamma, n_draft, lead;
  uint32_t seed_lo, seed_hi;
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// floor(w * 2^44) for 0 <= w < 2^19 (a weight relative to the row max is <= 1): the exact
// fixed-point value, by integer shifts of the mantissa.
__device__ __forceinline__ uint64_t fixw(float w) {
  const uint32_t b = __float_as_uint(w);
  const int e = (int)(b >> 23) - 127;  // w = m * 2^(e - 23), m = 24-bit mantissa
  if (e < -44) return 0;               // below the fixed-point resolution (zero included)
  const uint64_t m = (uint64_t)((b & 0x7FFFFFu) | 0x800000u);
  const int sh = e + 44 - 23;
  return sh >= 0 ? (m << sh) : (m >> -sh);
}

// Logit e (0..7) of a vector: one of its two 64-bit halves, shifted (a word picked by index
// would be lowered to a scratch array).
__device__ __forceinline__ float logit_at(const uint4& d, int e) {
  const uint64_t lo = ((uint64_t)d.y << 32) | d.x, hi = ((uint64_t)d.w << 32) | d.z;
  const uint64_t h = (e & 4) ? hi : lo;
  return bf_lo((uint32_t)(h >> ((e & 3) * 16)));
}

__device__ __forceinline__ int wave_incl_scan_i(int v, int) { return wave_incl_scan_dpp(v); }

// Parameters checked on their bit patterns (NaN fails every test). T: +0 or -0 (greedy), or
// 2^-126 <= T <= 2^126, so that the scale log2(e)/T is a finite normal value (a scale of 0
// would turn the -inf padding of a row's last vector into NaN).
__device__ __forceinline__ bool temperature_ok(float T) {
  const uint32_t b = __float_as_uint(T);
  return (b & 0x7FFFFFFFu) == 0u || (b >= 0x00800000u && b <= 0x7E800000u);
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
  int32_t K;       // top-k (<= 0 or >= V: off)
  int32_t eos;     // EOS id (< 0: none)
  int32_t cap;     // emission cap (<= 0: none)
  bool filter;     // a top-k or top-p cut applies to this sequence's laws
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
  s.K = P.topk ? P.topk[b] : 0;
  s.eos = P.eos ? P.eos[b] : -1;
  s.cap = P.cap ? P.cap[b] : 0;
  s.bad_param = !(s.g >= 0 && s.g <= P.max_gamma && c0 >= 0 && c1 <= P.n_draft) ||
                !temperature_ok(s.T) || !top_p_ok(s.P);
  if (s.T == 0.0f) s.T = 0.0f;  // -0 is greedy too
  s.filter = s.T != 0.0f && (s.P < 1.0f || (s.K >= 1 && s.K < P.V));
  return s;
}

// ----------------------------------------------------------------------------------------
// Row statistics (T > 0)
// ----------------------------------------------------------------------------------------

struct LaneAcc {
  float m = -INFINITY;   // max of the logits this lane has consumed
  float wm = -INFINITY;  // capture reference: a lower bound of the row max known to the wave
};

// Weight of one logit relative to a reference: the same expression everywhere, so that
// masses and probabilities computed in different places agree bit for bit.
__device__ __forceinline__ float weight(float l, float c, float nref) {
  return __builtin_amdgcn_exp2f(fmaf(l, c, nref));
}

// LDS of one row's workgroup.
struct RowLds {
  uint4 data[kCapN];               // captured vectors, in claim order
  float tmax[kMaxTrips];           // each trip's max
  float tsum[kMaxTrips];           // each trip's sum of weights against its max
  unsigned long long hist[kHist];  // fixed-point masses by key offset below the row max
  uint32_t hcnt[kHist];            // logits by key offset below the row max (top-k)
  NucEntry kept[kNucMax];          // nucleus entries before they are put in token order
  int32_t ctok[kCand];             // the window's logits as the bins take them: token ...
  float cval[kCand];               // ... and logit (the nucleus list filters these)
  uint16_t idx[kCapN];             // vector index of each captured vector
  float wmax[kRowWgWaves];         // each wave's max so far, published for the others
  float lmax[kRowThreads];         // every lane's max at the end of the stream
  float pm[kRowWgWaves];           // per-wave max (value of the argmax for greedy rows)
  int pa[kRowWgWaves];             // per-wave argmax (greedy rows)
  int trip;                        // trips of the row claimed by the waves
  int ncap;                        // capture slots claimed: LDS slots, then spill slots
  int nkept;                       // nucleus entries claimed
  int ncand;                       // window logits claimed (past kCand: only counted)
};

// Claims slots for the trip's flagged vectors (one LDS atomic per wave) and writes them:
// slots below kCapN hold the vector and its index in LDS, the next kCapG only the index in
// the row's workspace spill list; claims past both are only counted (the end phase then
// searches the whole row).
__device__ __forceinline__ void capture_trip(RowLds* L, uint16_t* spill, const uint4 d[kU],
                                             const float vm[kU], float thr, int v0, int lane) {
  uint64_t bm[kU];
  int n[kU], tot = 0;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    bm[u] = __ballot(vm[u] >= thr);
    n[u] = __popcll(bm[u]);
    tot += n[u];
  }
  if (tot == 0) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(&L->ncap, tot);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (vm[u] >= thr) {
      const int pos = base + (int)lanes_below(bm[u]);
      const int vid = v0 + u * kWave + lane;
      if (pos < kCapN) {
        L->data[pos] = d[u];
        L->idx[pos] = (uint16_t)vid;
      } else if (pos < kCapN + kCapG) {
        spill[pos - kCapN] = (uint16_t)vid;
      }
    }
    base += n[u];
  }
}

// One trip (kU vectors of the row): its max M_t and its sum of weights against M_t, each
// reduced over the wave in a fixed order, kept in LDS by trip index. The row's (M, Z) is
// combined from these records in trip order, so it does not depend on which wave claimed
// which trip: repeated calls give identical bits. With CAPTURE, the vectors whose max is
// within capw of the best lower bound of the row max the wave knows (its own max so far, and
// the maxima the other waves published in LDS) are captured: a superset of the final window.
template <bool CAPTURE>
__device__ __forceinline__ void consume_trip(const uint4 d[kU], int v0, int lane, float c,
                                             float capw, LaneAcc& a, RowLds* L,
                                             uint16_t* spill) {
  // the other waves' published maxima, read now and used after the trip's arithmetic
  float wg = -INFINITY;
  if (CAPTURE) {
#pragma unroll
    for (int i = 0; i < kRowWgWaves; ++i)
      wg = fmaxf(wg, __hip_atomic_load(&L->wmax[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  }
  float vm[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float x[8];
    unpack8(d[u], x);
    vm[u] = max8(x);
  }
  static_assert(kU == 4, "trip max below assumes four vectors per trip");
  const float tm = vmax3(vmax3(vm[0], vm[1], vm[2]), vm[3], vm[3]);
  const float mt = wave_max_dpp(tm);
  const float nref = mt == -INFINITY ? 0.0f : -mt * c;  // a trip of -inf logits weighs 0
  float st = 0.0f;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float x[8];
    unpack8(d[u], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) st += weight(x[e], c, nref);
  }
  const float zt = wave_sum_dpp(st);
  if (lane == 0) {
    const int t = v0 / (kU * kWave);
    L->tmax[t] = mt;
    L->tsum[t] = zt;
  }
  a.m = vmax3(a.m, tm, tm);
  if (CAPTURE) {
    a.wm = vmax3(a.wm, mt, wg);
    // kept finite, so a vector of -inf logits (past the row end included) is never captured
    const float thr = vmax3(a.wm - capw, -3.4028235e38f, -3.4028235e38f);
    capture_trip(L, spill, d, vm, thr, v0, lane);
    if (lane == 0)
      __hip_atomic_store(&L->wmax[threadIdx.x / kWave], a.wm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// (M, Z) of the row from its ntrips trip records: lane l takes trips l, l + 64, ... in order,
// then fixed-order wave reductions. Every wave computes the same values the same way.
__device__ __forceinline__ void row_mz(const RowLds* L, int ntrips, float c, int lane, float& M,
                                       float& Z) {
  float m = -INFINITY;
  for (int t = lane; t < ntrips; t += kWave) m = vmax3(m, L->tmax[t], L->tmax[t]);
  M = wave_max_dpp(m);
  const float nref = M == -INFINITY ? 0.0f : -M * c;
  float z = 0.0f;
  for (int t = lane; t < ntrips; t += kWave) {
    const float mt = L->tmax[t];
    if (mt != -INFINITY) z += L->tsum[t] * weight(mt, c, nref);
  }
  Z = wave_sum_dpp(z);
}

struct TopP {
  float t;     // threshold logit (-inf: keep all)
  float zs;    // normaliser over the kept set
  int nuc;     // kept count if the list was written, else -1
  bool slow;   // exact multi-pass search ran
};

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int) {
  return wave_incl_scan_dpp_u64(v);
}

// The first bin, in increasing bin index (= decreasing logit), at which base + the running
// sum of v reaches thr, over the wave's bins (PER per lane, bin = lane * PER + j); -1 if it
// never does. *cum receives the running sum at that bin (or base + the total). Every lane
// returns the same values.
template <int PER>
__device__ int lane_bins_crossing(const uint64_t v[PER], uint64_t base, uint64_t thr,
                                  uint64_t* cum, int lane) {
  uint64_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) mine += v[j];
  const uint64_t incl = base + wave_incl_scan_u64(mine, lane);
  const uint64_t hit = __ballot(incl >= thr);
  if (!hit) {
    *cum = __shfl(incl, kWave - 1, kWave);
    return -1;
  }
  const int src = __ffsll((long long)hit) - 1;
  int o = -1;
  uint64_t c = incl - mine;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (o < 0) {
      c += v[j];
      if (c >= thr) o = lane * PER + j;
    }
  }
  o = __shfl(o, src, kWave);
  const uint32_t lo = __shfl((uint32_t)c, src, kWave), hi = __shfl((uint32_t)(c >> 32), src, kWave);
  *cum = ((uint64_t)hi << 32) | lo;
  return o;
}

// Sum over the wave of the lane's bins at or below bin index o.
template <int PER>
__device__ __forceinline__ uint64_t bins_upto(const uint64_t v[PER], int o, int lane) {
  uint64_t s = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (lane * PER + j <= o) s += v[j];
  return wave_sum_u64(s);
}

// The cut of a row's law: t = the logit of key offset o below the row max (o < 0: keep
// every token), zs = the fixed-point mass of the kept set.
struct Cut {
  int o;
  uint64_t zs;
};

// Top-k, then top-p, over per-bin counts and fixed-point masses held by the wave's lanes:
// with top-k, the first bin at which the running count reaches K (the K-th largest logit,
// repeats counted) and the mass up to it; then, with top-p, the first bin at which the
// running mass reaches P times that mass (P times the row's mass without top-k). o < 0: a
// crossing was not reached within the bins.
template <int PER>
__device__ Cut bins_cut(const uint64_t cnt[PER], const uint64_t ms[PER], bool use_k, int K,
                        bool use_p, float P, float Z, int lane) {
  Cut r{-1, 0};
  uint64_t cum = 0;
  if (use_k) {
    r.o = lane_bins_crossing<PER>(cnt, 0, (uint64_t)K, &cum, lane);
    if (r.o < 0) return r;
    r.zs = bins_upto<PER>(ms, r.o, lane);
  }
  if (!use_p) return r;
  const uint64_t thr = use_k ? (uint64_t)((double)P * (double)r.zs)
                             : (uint64_t)((double)P * (double)Z * kFix);
  r.o = lane_bins_crossing<PER>(ms, 0, thr, &cum, lane);
  r.zs = cum;
  return r;
}

// Sources of a row's vectors for the end phase, each read through one address space (a getter
// that picked LDS or global memory per index would compile to generic flat loads, which wait
// on the vector memory path even for LDS): the captured vectors held in LDS (slots below
// kCapN), the spilled ones (indexes in the workspace, vectors read again from the row), and
// the whole row.
struct CapLds {
  const RowLds* L;
  __device__ void operator()(int j, int& vi, uint4& dv) const {
    vi = L->idx[j];
    dv = L->data[j];
  }
};
struct CapSpill {
  const uint16_t* spill;
  const uint4* row;
  __device__ void operator()(int j, int& vi, uint4& dv) const {
    vi = spill[j - kCapN];
    dv = row[vi];
  }
};
struct RowSrc {
  const uint4* row;
  __device__ void operator()(int j, int& vi, uint4& dv) const {
    vi = j;
    dv = row[j];
  }
};

// Nucleus list of a row once t is known: every kept logit (>= t, token < V) of the source
// vectors, claimed into LDS by a wave-aggregated atomic (collect_range, once per source
// range), then written to the workspace in token order (collect_finish: each entry's position
// is the number of kept tokens below it). Returns the kept count; above kNucMax the list is
// not written.
template <typename Src>
__device__ __forceinline__ void collect_range(Src src, int j_begin, int j_end, int V, float t,
                                              float c, float nref, RowLds* L, int tid) {
  const int lane = tid % kWave;
  for (int j0 = j_begin + tid - lane; j0 < j_end; j0 += kRowThreads) {
    const int j = j0 + lane;
    float x[8];
    int vi = 0;
    uint32_t keep = 0;
    uint4 dv{0u, 0u, 0u, 0u};
    if (j < j_end) {
      src(j, vi, dv);
      unpack8(dv, x);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (vi * 8 + e < V && x[e] >= t) keep |= 1u << e;
    }
    const int cnt = __popc(keep);
    const int incl = wave_incl_scan_i(cnt, lane);
    const int tot = __shfl(incl, kWave - 1, kWave);
    if (tot == 0) continue;
    int base = 0;
    if (lane == 0) base = atomicAdd(&L->nkept, tot);
    int pos = __builtin_amdgcn_readfirstlane(base) + incl - cnt;
    // the kept logits in increasing e, one round per kept logit of the busiest lane
    while (keep) {
      const int e = __builtin_ctz(keep);
      keep &= keep - 1;
      if (pos < kNucMax) L->kept[pos] = NucEntry{vi * 8 + e, weight(logit_at(dv, e), c, nref)};
      ++pos;
    }
  }
}
// The nucleus entries from the window's candidates: every logit >= t of the row lies in the
// window and in the bins (t is the value of a non-empty bin), so filtering the candidates
// gives the same kept set as a pass over the captured vectors.
__device__ __forceinline__ void collect_cands(RowLds* L, int nc, float t, float c, float nref,
                                              int tid) {
  const int lane = tid % kWave;
  for (int j0 = tid - lane; j0 < nc; j0 += kRowThreads) {
    const int j = j0 + lane;
    const bool keep = j < nc && L->cval[j] >= t;
    const uint64_t bm = __ballot(keep);
    if (!bm) continue;
    int base = 0;
    if (lane == 0) base = atomicAdd(&L->nkept, __popcll(bm));
    base = __builtin_amdgcn_readfirstlane(base);
    if (keep) {
      const int pos = base + (int)lanes_below(bm);
      if (pos < kNucMax) L->kept[pos] = NucEntry{L->ctok[j], weight(L->cval[j], c, nref)};
    }
  }
}

__device__ int collect_finish(RowLds* L, NucEntry* list, int tid) {
  __syncthreads();
  const int K = L->nkept;
  if (K <= kNucMax) {
    for (int i = tid; i < K; i += kRowThreads) {
      const NucEntry e = L->kept[i];
      int r = 0;
      for (int k = 0; k < K; ++k) r += L->kept[k].idx < e.idx;
      list[r] = e;
    }
  }
  return K;
}

// Exact search over the whole row, by a radix over the key offset below the row max (its
// high byte, then its low byte inside the chosen bucket; two passes): the first offset at
// which the running count (by_count) or fixed-point mass of the tokens at or above it
// reaches thr. *mass_at receives the running mass there (the row's whole mass if thr is not
// reached; the return value is then -1). Every thread returns the same values.
// The whole-row search does not use the captured vectors, so their LDS holds kRadixCopies
// copies of each radix histogram, bin-major (bin * kRadixCopies + copy: the copies of a bin
// sit in different banks). A lane adds into copy lane % kRadixCopies: on flat rows most
// logits share a few bins, and the copies divide the conflicts of one atomic by that much.
constexpr int kRadixCopies = 4;
static_assert(256 * kRadixCopies * (sizeof(unsigned long long) + sizeof(uint32_t)) <=
                  sizeof(uint4) * kCapN,
              "radix histogram copies fit the capture buffer");

__device__ int radix_cut(const uint4* __restrict__ row, int nvec, int V, float c, float nref,
                         uint32_t kM, bool by_count, uint64_t thr, uint64_t* mass_at,
                         RowLds* L, int tid) {
  const int lane = tid % kWave;
  constexpr int PER = 256 / kWave;
  unsigned long long* hist = reinterpret_cast<unsigned long long*>(L->data);
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(hist + 256 * kRadixCopies);
  const int copy = lane % kRadixCopies;
  int hi = -1;
  uint64_t base_c = 0, base_m = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int j = tid; j < 256 * kRadixCopies; j += kRowThreads) {
      hist[j] = 0ull;
      hcnt[j] = 0u;
    }
    __syncthreads();
    for (int v = tid; v < nvec; v += kRowThreads) {
      float x[8];
      unpack8(row[v], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (v * 8 + e >= V) continue;
        const uint32_t o = kM - key_of(x[e]);
        if (pass == 1 && (int)(o >> 8) != hi) continue;
        const uint32_t bin = pass == 0 ? (o >> 8) : (o & 255u);
        atomicAdd(&hcnt[bin * kRadixCopies + copy], 1u);
        const uint64_t fw = fixw(weight(x[e], c, nref));
        if (fw) atomicAdd(&hist[bin * kRadixCopies + copy], (unsigned long long)fw);
      }
    }
    __syncthreads();
    uint64_t cnt[PER], ms[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int b = lane * PER + j;
      cnt[j] = 0;
      ms[j] = 0;
#pragma unroll
      for (int k = 0; k < kRadixCopies; ++k) {
        cnt[j] += hcnt[b * kRadixCopies + k];
        ms[j] += hist[b * kRadixCopies + k];
      }
    }
    __syncthreads();  // the bins are cleared again only after every wave has read them
    uint64_t cum = 0;
    const int o = lane_bins_crossing<PER>(by_count ? cnt : ms, by_count ? base_c : base_m, thr,
                                          &cum, lane);
    if (o < 0) {
      *mass_at = base_m + (by_count ? bins_upto<PER>(ms, 255, lane) : cum - base_m);
      return -1;
    }
    if (pass == 0) {
      hi = o;
      base_c += bins_upto<PER>(cnt, o - 1, lane);
      base_m += bins_upto<PER>(ms, o - 1, lane);
    } else {
      *mass_at = base_m + bins_upto<PER>(ms, o, lane);
      return hi * 256 + o;
    }
  }
  return -1;
}

// Exact top-k / top-p cut over the whole row (radix_cut for the K-th largest logit, then for
// the top-p crossing), plus one pass for the nucleus list. Used when the captures missed the
// cut or overflowed. A top-p crossing that rounding leaves unreached keeps the top-k set
// (every token without top-k).
__device__ TopP topp_full_row(const uint4* __restrict__ row, int nvec, int V, float c, float M,
                              bool use_k, int K, bool use_p, float P, float Z, RowLds* L,
                              NucEntry* list, int tid) {
  const float nref = -M * c;
  const uint32_t kM = key_of(M);
  TopP r;
  r.slow = true;
  int o = -1;
  uint64_t zs = 0;
  if (use_k) o = radix_cut(row, nvec, V, c, nref, kM, true, (uint64_t)K, &zs, L, tid);
  if (use_p) {
    const uint64_t thr = use_k ? (uint64_t)((double)P * (double)zs)
                               : (uint64_t)((double)P * (double)Z * kFix);
    uint64_t zp = 0;
    const int op = radix_cut(row, nvec, V, c, nref, kM, false, thr, &zp, L, tid);
    if (op >= 0 || !use_k) {
      o = op;
      zs = zp;
    }
  }
  r.t = o < 0 ? -INFINITY : value_of_key(kM - (uint32_t)o);
  r.zs = (float)((double)zs / kFix);
  collect_range(RowSrc{row}, 0, nvec, V, r.t, c, nref, L, tid);
  const int n = collect_finish(L, list, tid);
  r.nuc = n <= kNucMax ? n : -1;
  return r;
}

// The cut on the captured vectors, which hold every logit >= theta of the row: fixed-point
// masses (and, with top-k, counts) of those logits by key offset below the row max, in LDS
// bins cleared beforehand; top-k and then top-p cross those bins, found by every wave from
// the same integer sums (so the same answer, with no barrier to hand it out). o < 0: a
// crossing is not reached within the kHist offsets (or the logits >= theta).
__device__ __forceinline__ Cut capture_cut(const uint4* __restrict__ row, int V, float c,
                                           float theta, float M, bool use_k, int K, bool use_p,
                                           float P, float Z, RowLds* L, const uint16_t* spill,
                                           int tid) {
  const int lane = tid % kWave;
  const float nref = -M * c;
  const uint32_t kM = key_of(M);
  const int ntot = L->ncap;
  // The logits of the vector that fall in the bins first, as a mask; then only those: a wave
  // takes as many rounds as its busiest lane has such logits (usually one or two of eight).
  auto hist_vec = [&](int vi, const uint4& dv) {
    float x[8];
    unpack8(dv, x);
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (vi * 8 + e < V && x[e] >= theta && kM - key_of(x[e]) < (uint32_t)kHist) m |= 1u << e;
    while (m) {
      const int e = __builtin_ctz(m);
      const float xe = logit_at(dv, e);
      m &= m - 1;
      const uint32_t o = kM - key_of(xe);
      if (use_k) atomicAdd(&L->hcnt[o], 1u);
      atomicAdd(&L->hist[o], (unsigned long long)fixw(weight(xe, c, nref)));
      // the logit is also a candidate for the nucleus list: one claim per wave and round
      const uint64_t act = __ballot(1);
      const int r = (int)lanes_below(act);
      int base = 0;
      if (r == 0) base = atomicAdd(&L->ncand, __popcll(act));
      const int pos = __builtin_amdgcn_readfirstlane(base) + r;
      if (pos < kCand) {
        L->ctok[pos] = vi * 8 + e;
        L->cval[pos] = xe;
      }
    }
  };
  for (int j = tid; j < min(ntot, kCapN); j += kRowThreads) hist_vec(L->idx[j], L->data[j]);
  for (int j = kCapN + tid; j < ntot; j += kRowThreads) {
    const int vi = spill[j - kCapN];
    hist_vec(vi, row[vi]);
  }
  __syncthreads();
  constexpr int PER = kHist / kWave;
  uint64_t cnt[PER], ms[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    cnt[j] = use_k ? L->hcnt[lane * PER + j] : 0u;
    ms[j] = L->hist[lane * PER + j];
  }
  return bins_cut<PER>(cnt, ms, use_k, K, use_p, P, Z, lane);
}

// The K-th largest of the workgroup's lane maxima (K <= kRowThreads): K distinct logits of
// the row are at or above it, so it is a lower bound of the row's K-th largest logit.
__device__ float lane_max_kth(RowLds* L, int K, int tid) {
  const int lane = tid % kWave, w = tid / kWave;
  const float v = L->lmax[tid];
  int n = 0;
  for (int i = 0; i < kRowThreads; ++i) n += L->lmax[i] >= v;
  const float best = wave_max_dpp(n >= K ? v : -INFINITY);
  if (lane == 0) L->pm[w] = best;  // the waves' partials are no longer needed
  __syncthreads();
  float r = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRowWgWaves; ++i) r = fmaxf(r, L->pm[i]);
  return r;
}

// A second capture of the row: every vector whose max is >= vk, in the same LDS slots and
// spill list (cleared first, as are the bins). The row is read in trips of the stream's
// layout (vector v0 + u * kWave + lane in slot u), wave w taking trips w, w + 8, ...; a
// trip's kU loads are issued together, from clamped indexes so that each stays one
// unconditional 16-byte load, and the vectors past the row weigh as -inf.
__device__ void recapture(const uint4* __restrict__ row, int nvec, int V, float vk, RowLds* L,
                          uint16_t* spill, int tid) {
  const int lane = tid % kWave, w = tid / kWave;
  __syncthreads();  // every thread is done with the first capture and its bins
  if (tid == 0) {
    L->ncap = 0;
    L->ncand = 0;
  }
  for (int i = tid; i < kHist; i += kRowThreads) {
    L->hist[i] = 0ull;
    L->hcnt[i] = 0u;
  }
  __syncthreads();
  constexpr int kTripVecs = kU * kWave;
  // a finite threshold: vectors past the row (all -inf) are never captured, even if vk is -inf
  const float thr = vmax3(vk, -3.4028235e38f, -3.4028235e38f);
  for (int v0 = w * kTripVecs; v0 < nvec; v0 += kRowWgWaves * kTripVecs) {
    uint4 d[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) d[u] = row[min(v0 + u * kWave + lane, nvec - 1)];
    float vm[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * kWave + lane;
      float x[8];
      unpack8(d[u], x);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (v * 8 + e >= V) x[e] = -INFINITY;  // v >= nvec: every logit, as v * 8 >= V
      vm[u] = max8(x);
    }
    capture_trip(L, spill, d, vm, thr, v0, lane);
  }
  __syncthreads();
}

// Threshold search for a row with a top-k and/or top-p cut: on the captured window; with
// top-k and too few logits in the window, on a second capture from a lower bound of the
// K-th largest logit; else (captures overflowed, or a crossing past the bins) over the whole
// row.
__device__ __forceinline__ TopP topp_select(const uint4* __restrict__ row, int nvec, int V,
                                            float c, bool use_k, int K, bool use_p, float P,
                                            float capw, float M, float Z, RowLds* L,
                                            uint16_t* spill, NucEntry* list, int tid) {
  const float nref = -M * c;
  const uint32_t kM = key_of(M);
  bool held = L->ncap <= kCapN + kCapG, again = false;
  if (held) {
    Cut cut = capture_cut(row, V, c, M - capw, M, use_k, K, use_p, P, Z, L, spill, tid);
    if (cut.o < 0 && use_k && K <= kRowThreads) {
      again = true;
      const float vk = lane_max_kth(L, K, tid);
      recapture(row, nvec, V, vk, L, spill, tid);
      held = L->ncap <= kCapN + kCapG;
      if (held) cut = capture_cut(row, V, c, vk, M, use_k, K, use_p, P, Z, L, spill, tid);
    }
    if (held && cut.o >= 0) {
      TopP r;
      r.slow = again;  // a second read of the row
      r.t = value_of_key(kM - (uint32_t)cut.o);
      r.zs = (float)((double)cut.zs / kFix);
      const int nc = L->ncand;
      if (nc <= kCand) {
        collect_cands(L, nc, r.t, c, nref, tid);
      } else {
        collect_range(CapLds{L}, 0, min(L->ncap, kCapN), V, r.t, c, nref, L, tid);
        collect_range(CapSpill{spill, row}, kCapN, L->ncap, V, r.t, c, nref, L, tid);
      }
      const int n = collect_finish(L, list, tid);
      r.nuc = n <= kNucMax ? n : -1;
      return r;
    }
    __syncthreads();  // every wave has read the bins before the whole-row search reuses them
  }
  return topp_full_row(row, nvec, V, c, M, use_k, K, use_p, P, Z, L, list, tid);
}

// ----------------------------------------------------------------------------------------
// Kernel 1: one workgroup of kRowWgWaves waves per logits row. The waves take the row's
// trips in turn (wave w: trips w, w + kRowWgWaves, ...), so a row streams as one wide
// sequential read and the hardware hands out rows to CUs as they free up (which evens out
// the speed differences between CUs and XCDs that a fixed row-to-CU split would expose).
// Sequence b owns row ids b*(2G+1) .. b*(2G+1)+2G (G = max_gamma): id 2(k-1) is the target
// row p_k of draft position k, id 2(k-1)+1 its draft row q_k, and the last one the bonus row
// p_{gamma_b+1} (needed only after a full accept, but read with the rest: one workgroup
// cannot pull a row from HBM fast enough to do it later without stalling the resolve step).
// TOPP: the batch carries a top-p or top-k array (the captures and the cut are compiled in).
// The row streams use nontemporal loads: the stream reads every row once (a top-k row
// captured a second time reads it once more, in the end phase).
// ----------------------------------------------------------------------------------------
template <bool TOPP>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(6)))
void row_stats_kernel(ChainParams P) {
  __shared__ RowLds L;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int per = 2 * P.max_gamma + 1;
  const int row_id = blockIdx.x;
  if (row_id >= P.B * per) return;
  const int b = row_id / per, j = row_id % per;
  const bool bonus = j == 2 * P.max_gamma;
  const int r = bonus ? 0 : (j & 1);
  const SeqInfo s = seq_info(P, b);
  if (s.bad_param) return;
  const int k = bonus ? s.g + 1 : (j >> 1) + 1;  // 1-based position
  if (!bonus && k > s.g) return;
  if (r == 1 && s.T == 0.0f) return;  // greedy: q is not read
  const int drow = s.d0 + k - 1;       // draft row (draft positions only)
  const size_t slot = bonus ? 2 * (size_t)P.n_draft + (size_t)b : (size_t)drow * 2 + r;
  RowStat* st = P.stat + slot;
  NucEntry* list = P.nuc + slot * kNucMax;
  int d = -1;  // the draft token (none for the bonus row)
  if (!bonus) {
    d = P.tokens[drow];
    if (d < 0 || d >= P.V) {  // the resolve step flags the sequence; nothing to compute
      if (tid == 0) *st = RowStat{0.0f, 1.0f, -INFINITY, 0.0f, 0, -1, 0, 1};
      return;
    }
    if (r == 1 && P.draft == nullptr) {  // no draft rows: q is the point mass at d
      if (tid == 0) {
        list[0] = NucEntry{d, 1.0f};
        *st = RowStat{0.0f, 1.0f, -INFINITY, 1.0f, d, 1, 0, 1};
      }
      return;
    }
  }
  const uint16_t* base = r == 0 ? P.target + (size_t)(s.t0 + k - 1) * P.stride
                                : P.draft + (size_t)drow * P.stride;
  const uint4* rp = reinterpret_cast<const uint4*>(base);

  const bool filt = TOPP && s.filter;
  if (tid == 0) {
    L.trip = 0;
    L.ncap = 0;
    L.nkept = 0;
    L.ncand = 0;
  }
  if (tid < kRowWgWaves) L.wmax[tid] = -INFINITY;
  if (filt)
    for (int i = tid; i < kHist; i += kRowThreads) {
      L.hist[i] = 0ull;
      L.hcnt[i] = 0u;
    }
  __syncthreads();

  if (s.T == 0.0f) {  // greedy: argmax of the target row, lowest index on ties
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    stream_row_claimed<kDepth>(rp, P.nvec, lane, &L.trip, [&](uint4* dd, int v0, bool) {
      argmax_trip(dd, v0, P.nvec, P.V, lane, bv, bi);
    });
    wave_argmax(bv, bi);
    if (lane == 0) {
      L.pm[w] = bv;
      L.pa[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {  // starts from wave 0's (bv, bi)
      for (int i = 1; i < kRowWgWaves; ++i)
        if (L.pm[i] > bv || (L.pm[i] == bv && L.pa[i] < bi)) {
          bv = L.pm[i];
          bi = L.pa[i];
        }
      const int am = bi == 0x7FFFFFFF ? 0 : bi;
      *st = RowStat{0.0f, 1.0f, -INFINITY, d == am ? 1.0f : 0.0f, am, -1, 0, 1};
    }
    return;
  }

  const uint32_t ld_bits = (tid == 0 && d >= 0) ? base[d] : 0u;  // the draft token's logit
  const float c = kLog2e / s.T;
  const bool use_k = s.K >= 1 && s.K < P.V;
  const float capw = (use_k ? kCaptureKTopK : kCaptureK) * s.T;
  uint16_t* spill = P.spill + slot * kCapG;
  LaneAcc acc;
  if (filt)
    stream_row_claimed<kDepthCap>(rp, P.nvec, lane, &L.trip, [&](uint4* dd, int v0, bool ml) {
      if (ml) mask_tail(dd, v0, P.nvec, P.V, lane);
      consume_trip<true>(dd, v0, lane, c, capw, acc, &L, spill);
    });
  else
    stream_row_claimed<kDepth>(rp, P.nvec, lane, &L.trip, [&](uint4* dd, int v0, bool ml) {
      if (ml) mask_tail(dd, v0, P.nvec, P.V, lane);
      consume_trip<false>(dd, v0, lane, c, capw, acc, &L, nullptr);
    });
  if (filt) L.lmax[tid] = acc.m;
  __syncthreads();
  float M, Z;
  row_mz(&L, (P.nvec + kU * kWave - 1) / (kU * kWave), c, lane, M, Z);
  TopP tp{-INFINITY, Z, -1, false};
  if (filt)
    tp = topp_select(rp, P.nvec, P.V, c, use_k, s.K, s.P < 1.0f, s.P, capw, M, Z, &L, spill,
                     list, tid);
  if (tid == 0) {
    const float ld = __uint_as_float(ld_bits << 16);
    const float wd = (d >= 0 && ld >= tp.t) ? weight(ld, c, -M * c) : 0.0f;
    *st = RowStat{M, tp.zs, tp.t, wd, -1, filt ? tp.nuc : -1,
                  tp.slow ? SPEC_FLAG_TOPP_SLOW : 0, 1};
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

// Weight of token id in a sorted nucleus list held in LDS (0 if absent): a scan of a short
// list (independent broadcast reads), else a binary search.
__device__ __forceinline__ float list_weight(const NucEntry* q, int nq, int id) {
  if (nq <= kWave) {
    float r = 0.0f;
    for (int i = 0; i < nq; ++i) {
      const NucEntry e = q[i];
      r = e.idx == id ? e.w : r;
    }
    return r;
  }
  int lo = 0, hi = nq;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (q[mid].idx < id) lo = mid + 1;
    else hi = mid;
  }
  return (lo < nq && q[lo].idx == id) ? q[lo].w : 0.0f;
}

constexpr int kPerLane = kNucMax / kWave;  // list entries per lane in a list draw

// One wave: inverse-CDF draw over a nucleus list sorted by token id (<= kNucMax entries;
// entry j sits in lane j % 64, slot j / 64, so token order is slot-major, then lane order).
// residual: weights max(0, p - q) with q looked up in q's list -- held in registers and
// scanned with lane reads when it has at most 64 entries, else searched in memory; else p.
__device__ __forceinline__ Draw draw_from_lists(const NucEntry* pl, int np, float zp,
                                                const NucEntry* ql, int nq, float zq,
                                                bool residual, float u, int lane) {
  const bool qregs = residual && nq <= kWave;
  int qidx = 0x7FFFFFFF;
  float qw = 0.0f;
  if (qregs && lane < nq) {
    const NucEntry e = ql[lane];
    qidx = e.idx;
    qw = e.w;
  }
  int idx[kPerLane];
  float w[kPerLane];
#pragma unroll
  for (int s = 0; s < kPerLane; ++s) {
    const int j = s * kWave + lane;
    idx[s] = 0x7FFFFFFF;
    w[s] = 0.0f;
    if (s * kWave < np) {  // wave-uniform: the lane reads below stay in converged code
      if (j < np) {
        const NucEntry en = pl[j];
        idx[s] = en.idx;
        w[s] = en.w / zp;
      }
      if (residual) {
        float wq = 0.0f;
        if (qregs) {
          for (int i = 0; i < nq; ++i) {
            const int qi = __builtin_amdgcn_readlane(qidx, i);
            const float qv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qw), i));
            wq = qi == idx[s] ? qv : wq;
          }
        } else if (j < np) {
          wq = list_weight(ql, nq, idx[s]);
        }
        w[s] = fmaxf(0.0f, w[s] - wq / zq);
      }
    }
  }
  // slot totals (uniform), then the slot holding x and the lane inside it
  float incl[kPerLane], tot[kPerLane];
  float total = 0.0f;
#pragma unroll
  for (int s = 0; s < kPerLane; ++s) {
    incl[s] = wave_incl_scan_dpp_f(w[s]);
    tot[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl[s]), 63));
    total += tot[s];
  }
  const float x = u * total;
  int tok = -1;
  float wt = 0.0f;
  float base = 0.0f;
  bool found = false;
#pragma unroll
  for (int s = 0; s < kPerLane; ++s) {
    if (!found) {
      const uint64_t hit = __ballot(base + incl[s] > x && w[s] > 0.0f);
      if (hit) {
        const int src = __ffsll((long long)hit) - 1;
        tok = __builtin_amdgcn_readlane(idx[s], src);
        wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[s]), src));
        found = true;
      }
      base += tot[s];
    }
  }
  if (!found) {  // rounding left u*total at or past the end: the last entry with weight
#pragma unroll
    for (int s = kPerLane - 1; s >= 0; --s) {
      const uint64_t pos = __ballot(w[s] > 0.0f);
      if (!found && pos) {
        const int src = 63 - __clzll((long long)pos);
        tok = __builtin_amdgcn_readlane(idx[s], src);
        wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[s]), src));
        found = true;
      }
    }
  }
  Draw d;
  d.token = tok;
  d.wtok = wt;
  d.total = total;
  if (d.token < 0) {  // an empty list (no weight anywhere): token 0
    d.token = 0;
    d.wtok = 0.0f;
  }
  return d;
}

// A row's filtered law: probability exp2(l*c + nref) / z for l >= t, else 0 (z = the law's
// normaliser Z against the same reference).
struct RowLaw {
  const uint4* row;
  float c, nref, t, z;
  int point = -1;  // >= 0: the law is the point mass at this token (row is not read; z = 1)
};

// Whole-row draws work on weights in units of p's normaliser: p's weight is exp2(l*c + nref)
// (Z_p times its probability) and the residual's is max(0, p_w - rq * q_w) with
// rq = Z_p / Z_q (Z_p times max(0, p - q)). An inverse-CDF draw is the same under a common
// scale, so only the reported masses are multiplied by 1 / Z_p at the end; the residual
// costs one fused multiply-add per logit instead of two products and a difference.
__device__ __forceinline__ void law_weights(const RowLaw& L, const uint4& d, float w[8]) {
  float x[8];
  unpack8(d, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = (x[e] >= L.t) ? weight(x[e], L.c, L.nref) : 0.0f;
}

// Weights of vector v from its loaded p (and q) data, in units of p's normaliser: p, or
// max(0, p - q). Vectors past the row and logits past V weigh 0.
__device__ __forceinline__ void data_weights(const RowLaw& Lp, const RowLaw& Lq, bool residual,
                                             float rq, int v, int nvec, int V, const uint4& dp,
                                             const uint4& dq, float w[8]) {
  if (v >= nvec) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = 0.0f;
    return;
  }
  law_weights(Lp, dp, w);
  if (residual) {
    float wq[8];
    if (Lq.point >= 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wq[e] = (v * 8 + e == Lq.point) ? 1.0f : 0.0f;
    } else {
      law_weights(Lq, dq, wq);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = fmaxf(0.0f, fmaf(-rq, wq[e], w[e]));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (v * 8 + e >= V) w[e] = 0.0f;
}
__device__ __forceinline__ void vec_weights(const RowLaw& Lp, const RowLaw& Lq, bool residual,
                                            float rq, int v, int nvec, int V, float w[8]) {
  // clamped, unconditional 16-byte loads; data_weights gives 0 past the row
  const int vc = min(v, nvec - 1);
  const uint4 dp = Lp.row[vc];
  uint4 dq{0u, 0u, 0u, 0u};
  if (residual && Lq.point < 0) dq = Lq.row[vc];
  data_weights(Lp, Lq, residual, rq, v, nvec, V, dp, dq, w);
}

// Phase 2 of a row draw, once tile_sum holds every tile's sum and each lane knows the last
// positive-weight vector it saw: wave 0 scans the tile sums, then re-reads the chosen tile
// and scans it. When u * total lands at or past the end (rounding), the draw is the row's
// last token with positive weight, found in the last such vector.
template <int NT>
__device__ __forceinline__ Draw draw_scan(const RowLaw Lp, const RowLaw Lq, bool residual,
                                          float rq, int nvec, int V, float u, int last,
                                          float* tile_sum,
                                          int* sh_i, float* sh_f) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int nw = NT / kWave;
  const int ntiles = (nvec + kWave - 1) / kWave;
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
    int token = -1;
    float wtok = 0.0f;
    if (gstar >= 0) {
      const int v = gstar * kWave + lane;
      float w[8];
      vec_weights(Lp, Lq, residual, rq, v, nvec, V, w);
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
      token = tok;
      wtok = wt;
    }
    if (token < 0 && lst >= 0) {  // u*total at or past the end: the last token with weight
      float w[8];
      vec_weights(Lp, Lq, residual, rq, lst, nvec, V, w);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (w[e] > 0.0f) {
          token = lst * 8 + e;
          wtok = w[e];
        }
    }
    if (lane == 0) {
      sh_i[0] = token < 0 ? 0 : token;
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

// All threads of the workgroup: inverse-CDF draw over a whole row (pair) in token order.
// Pass 1 stores per-tile sums (a tile = 64 vectors = 512 logits, one coalesced wave load;
// each wave keeps TI tiles of p and of q in flight); draw_scan finishes.
// Per-tile sums of a row (pair): each wave takes TI tiles at a time (a tile = 64 vectors =
// 512 logits, one coalesced wave load per row); tile g -> tile_sum[g]. Returns the last
// vector with positive weight this lane saw (-1: none). A vector past the row loads the row's last
// vector instead (its weight is zero), so that every load is one unconditional 16-byte load:
// a load under a per-lane condition compiles to four predicated 4-byte loads.
// Vector v with its logits at or past V set to -inf (v >= nvec: all of them), whose weights
// are then 0 under a law without a cut.
__device__ __forceinline__ uint4 mask_past_v(uint4 d, int v, int V) {
  uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (v * 8 + e >= V) {
      if (e & 1) w[e >> 1] = (w[e >> 1] & 0x0000FFFFu) | 0xFF800000u;
      else w[e >> 1] = (w[e >> 1] & 0xFFFF0000u) | 0x0000FF80u;
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// tile_sums for laws without a cut (t = -inf on p, and on q when RES): the weights are the
// same expression as data_weights gives, bit for bit (every finite or -inf logit passes the
// cut, and a -inf logit weighs exactly 0), with the row's end masked to -inf in the lanes
// that hold it instead of per-logit bound checks. Returns the last vector with positive
// weight this lane saw (-1: none).
template <int NT, int TI, bool RES>
__device__ __forceinline__ int tile_sums_nocut(const RowLaw& Lp, const RowLaw& Lq, float rq,
                                               int nvec, int V, float* tile_sum) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int nw = NT / kWave;
  const int ntiles = (nvec + kWave - 1) / kWave;
  int lastv = -1;
  for (int g0 = wid * TI; g0 < ntiles; g0 += nw * TI) {
    uint4 dp[TI], dq[TI];
#pragma unroll
    for (int t = 0; t < TI; ++t) dp[t] = Lp.row[min((g0 + t) * kWave + lane, nvec - 1)];
    if (RES) {
#pragma unroll
      for (int t = 0; t < TI; ++t) dq[t] = Lq.row[min((g0 + t) * kWave + lane, nvec - 1)];
    }
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      const int v = (g0 + t) * kWave + lane;
      uint4 a = dp[t], b = RES ? dq[t] : dp[t];
      if (v >= nvec - 1) {  // the row's last vector, or past the row
        a = mask_past_v(a, v, V);
        if (RES) b = mask_past_v(b, v, V);
      }
      float xp[8], xq[8];
      unpack8(a, xp);
      if (RES) unpack8(b, xq);
      float ls = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float w = weight(xp[e], Lp.c, Lp.nref);
        if (RES) w = fmaxf(0.0f, fmaf(-rq, weight(xq[e], Lq.c, Lq.nref), w));
        ls += w;
      }
      if (ls > 0.0f) lastv = v;
      const float ts = wave_sum_dpp(ls);
      if (lane == 0 && g0 + t < ntiles) tile_sum[g0 + t] = ts;
    }
  }
  return lastv;
}

template <int NT, int TI>
__device__ __forceinline__ int tile_sums(const RowLaw& Lp, const RowLaw& Lq, bool residual,
                                         float rq, int nvec, int V, float* tile_sum) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int nw = NT / kWave;
  const int ntiles = (nvec + kWave - 1) / kWave;
  const bool with_q = residual && Lq.point < 0;
  if (Lp.t == -INFINITY && (!residual || (with_q && Lq.t == -INFINITY))) {
    if (residual) return tile_sums_nocut<NT, TI, true>(Lp, Lq, rq, nvec, V, tile_sum);
    return tile_sums_nocut<NT, TI, false>(Lp, Lq, rq, nvec, V, tile_sum);
  }
  int lastv = -1;  // last vector with positive weight seen by this lane
  for (int g0 = wid * TI; g0 < ntiles; g0 += nw * TI) {
    uint4 dp[TI], dq[TI];
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      dp[t] = Lp.row[min((g0 + t) * kWave + lane, nvec - 1)];
      dq[t] = uint4{0u, 0u, 0u, 0u};
    }
    if (with_q) {
#pragma unroll
      for (int t = 0; t < TI; ++t) dq[t] = Lq.row[min((g0 + t) * kWave + lane, nvec - 1)];
    }
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      const int v0 = (g0 + t) * kWave + lane;
      const int v = v0 < nvec ? v0 : nvec;  // data_weights gives 0 past the row
      float w[8];
      data_weights(Lp, Lq, residual, rq, v, nvec, V, dp[t], dq[t], w);
      float ls = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ls += w[e];
      if (ls > 0.0f) lastv = v;  // the weights are >= 0: a positive sum has a positive weight
      const float ts = wave_sum_dpp(ls);
      if (lane == 0 && g0 + t < ntiles) tile_sum[g0 + t] = ts;
    }
  }
  return lastv;
}

template <int NT, int TI>
__device__ __forceinline__ Draw draw_from_rows(const RowLaw Lp, const RowLaw Lq, bool residual,
                                               int nvec, int V, float u, float* tile_sum,
                                               int* sh_i, float* sh_f) {
  const float rq = residual ? Lp.z / Lq.z : 0.0f;
  const int last = tile_sums<NT, TI>(Lp, Lq, residual, rq, nvec, V, tile_sum);
  Draw d = draw_scan<NT>(Lp, Lq, residual, rq, nvec, V, u, last, tile_sum, sh_i, sh_f);
  const float iz = 1.0f / Lp.z;  // back from units of Z_p to probabilities
  d.total *= iz;
  d.wtok *= iz;
  return d;
}

// Per-sequence decision state the resolve step shares through LDS.
struct SeqDecision {
  int tok[kWave];  // the draft tokens d_1..d_gamma, as the decision loaded them
  int n_acc;
  int drawn;  // the round ends with a residual or bonus token (no early stop)
  int flags;
  int bad;  // SPEC_FLAG_BAD_TOKEN / SPEC_FLAG_BAD_PARAM bits: no progress
  RowStat sp, sq;  // statistics of the rows at the first rejection (if any)
};

// One wave: a list draw, published to the workgroup through LDS.
__device__ __forceinline__ Draw wg_list_draw(const NucEntry* pl, int np, float zp,
                                             const NucEntry* ql, int nq, float zq,
                                             bool residual, float u, int* sh_i, float* sh_f) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  if (tid < kWave) {
    const Draw d = draw_from_lists(pl, np, zp, ql, nq, zq, residual, u, lane);
    if (lane == 0) {
      sh_i[0] = d.token;
      sh_f[0] = d.total;
      sh_f[1] = d.wtok;
    }
  }
  __syncthreads();
  const Draw d{sh_i[0], sh_f[0], sh_f[1]};
  __syncthreads();
  return d;
}

// Index of the bonus row's statistics (and list, spill area) after the draft rows' ones.
__device__ __forceinline__ size_t bonus_slot(const ChainParams& P, int b) {
  return 2 * (size_t)P.n_draft + (size_t)b;
}

// The round's decision for sequence b, by one wave (lane = its lane id): the acceptance tests
// from the row statistics, the first rejection, the early stop, the flags; the statistics of
// the rows at the first rejection. Written to sd, and the probes if the call asks for them.
__device__ __forceinline__ void decide_wave(const ChainParams& P, const SeqInfo& s, bool cu_ok,
                                            bool stochastic, SeqDecision& sd, int lane) {
  const bool in_g = cu_ok && lane < s.g;
  int tok = 0;
  RowStat sp{}, sq{};
  if (in_g) {
    tok = P.tokens[s.d0 + lane];
    sp = P.stat[(size_t)(s.d0 + lane) * 2];
    if (stochastic) sq = P.stat[(size_t)(s.d0 + lane) * 2 + 1];
  }
  sd.tok[lane] = tok;
  const bool bad_tok = __ballot(in_g && (tok < 0 || tok >= P.V)) != 0;
  int acc = 1, rflags = 0;
  if (in_g && !s.bad_param && !bad_tok) {
    float pd, qd, a;
    if (s.T == 0.0f) {  // greedy: accept iff the draft is the target argmax
      acc = tok == sp.argmax ? 1 : 0;
      pd = (float)acc;
      qd = NAN;
      a = (float)acc;
    } else {
      pd = sp.wd / sp.z;
      qd = sq.wd / sq.z;
      if (qd > 0.0f) {
        a = fminf(1.0f, pd / qd);
      } else {
        a = pd > 0.0f ? 1.0f : 0.0f;
        rflags |= SPEC_FLAG_Q_ZERO;
      }
      const float u = P.ovr ? P.ovr[(size_t)(s.t0 + lane) * 2]
                            : uniform24(P.seed_lo, P.seed_hi, s.id,
                                        (uint32_t)(s.L + lane + 1), SPEC_PURPOSE_ACCEPT);
      acc = (u < a) ? 1 : 0;
      rflags |= (sp.flags | sq.flags) & SPEC_FLAG_TOPP_SLOW;
    }
    if (P.probe_rows) {
      P.probe_rows[(size_t)(s.d0 + lane) * 3 + 0] = pd;
      P.probe_rows[(size_t)(s.d0 + lane) * 3 + 1] = qd;
      P.probe_rows[(size_t)(s.d0 + lane) * 3 + 2] = a;
    }
  }
  const uint64_t rej = __ballot(in_g && acc == 0);
  int n_acc = rej ? __ffsll((long long)rej) - 1 : s.g;
  // Early stop ("KV Cache 优化（四）" §5): emission ends after an accepted draft equal to
  // the EOS id, or once the cap's worth of accepted drafts is out; the round then ends
  // there, with no later test and no residual or bonus draw.
  const uint64_t eos_at = __ballot(in_g && s.eos >= 0 && tok == s.eos && lane < n_acc);
  int stop = eos_at ? __ffsll((long long)eos_at) : 0x7FFFFFFF;  // 1-based position
  int stop_flag = SPEC_FLAG_EOS;
  if (s.cap > 0 && s.cap < stop) {
    stop = s.cap;
    stop_flag = SPEC_FLAG_LEN_CAP;
  }
  const bool early = stop <= n_acc;
  if (early) n_acc = stop;
  int f = (lane < (early ? n_acc : min(n_acc + 1, s.g))) ? rflags : 0;  // tested positions
  for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, kWave);
  if (lane == 0) {
    sd.n_acc = n_acc;
    sd.drawn = early ? 0 : 1;
    sd.flags = f | (early ? stop_flag : 0);
    sd.bad = (bad_tok ? SPEC_FLAG_BAD_TOKEN : 0) | (s.bad_param ? SPEC_FLAG_BAD_PARAM : 0);
  }
  if (in_g && lane == n_acc) {  // the first rejected position
    sd.sp = sp;
    sd.sq = sq;
  }
}

template <int NT, int TI>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4)))
void chain_resolve_kernel(ChainParams P) {
  __shared__ float tile_sum[kMaxTiles];  // inverse-CDF draw over a row (pair)
  __shared__ int sh_i[kResolveMaxWaves];
  __shared__ float sh_f[2];
  __shared__ NucEntry s_lp[kNucMax], s_lq[kNucMax];
  __shared__ NucEntry s_pre[kPreRows][2][kPre];
  __shared__ NucEntry s_preb[kPre];
  __shared__ SeqDecision sd;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const SeqInfo s = seq_info(P, b);
  __syncthreads();  // every thread has read committed_len[b] before thread 0 rewrites it
  // gamma_b and cu_gamma in range: the draft tokens and statistics of the sequence exist
  const int c0 = P.cu[b], c1 = P.cu[b + 1];
  const bool cu_ok = c1 - c0 >= 0 && c1 - c0 <= P.max_gamma && c0 >= 0 && c1 <= P.n_draft;
  const bool stochastic = !s.bad_param && s.T != 0.0f;
  // The heads of the candidate rows' nucleus lists, fetched together with the statistics:
  // where the first rejection falls is not known yet, and the draw usually needs no more.
  // Every load of this phase is issued before any result is used (the list entries into
  // registers, from in-range slots only -- rows past gamma_b read the bonus list -- then the
  // decision's loads in wave 0), so that the phase costs one memory round trip.
  constexpr int kPreEach = (kPreRows * 2 * kPre + NT - 1) / NT;
  const bool prefetch = cu_ok && stochastic && (P.topp || P.topk);
  NucEntry pre[kPreEach], preb{};
  if (prefetch) {
#pragma unroll
    for (int r = 0; r < kPreEach; ++r) {
      const int i = tid + r * NT;
      const int kk = i / (2 * kPre), rr = (i / kPre) & 1, j = i % kPre;
      const size_t slot = kk < s.g ? (size_t)(s.d0 + kk) * 2 + rr : bonus_slot(P, b);
      pre[r] = P.nuc[slot * kNucMax + j];
    }
    preb = P.nuc[bonus_slot(P, b) * kNucMax + (tid & (kPre - 1))];
  }
  RowStat sbon{};
  if (!s.bad_param) sbon = P.stat[bonus_slot(P, b)];
  if (wid == 0) decide_wave(P, s, cu_ok, stochastic, sd, lane);
  if (prefetch) {
#pragma unroll
    for (int r = 0; r < kPreEach; ++r) {
      const int i = tid + r * NT;
      const int kk = i / (2 * kPre), rr = (i / kPre) & 1, j = i % kPre;
      if (i < kPreRows * 2 * kPre && kk < s.g) s_pre[kk][rr][j] = pre[r];
    }
    if (tid < kPre) s_preb[tid] = preb;
  }
  __syncthreads();
  const int n_acc = sd.n_acc;
  int flags = sd.flags;
  if (sd.bad) {  // no progress: nothing emitted, pointer unchanged
    if (tid == 0) {
      P.num_acc[b] = 0;
      if (P.num_emit) P.num_emit[b] = 0;
      if (P.flags_out) P.flags_out[b] = sd.bad;
      if (P.probe_seq) {
        P.probe_seq[2 * b] = NAN;
        P.probe_seq[2 * b + 1] = NAN;
      }
    }
    return;
  }
  if (!sd.drawn) {  // stopped inside the accepted drafts: they are the round's output
    if (wid == 0) {
      if (lane < n_acc) P.out_tokens[s.t0 + lane] = sd.tok[lane];
      if (lane == 0) {
        P.num_acc[b] = n_acc;
        if (P.num_emit) P.num_emit[b] = n_acc;
        P.committed[b] = s.L + P.lead + n_acc;
        if (P.flags_out) P.flags_out[b] = flags;
        if (P.probe_seq) {
          P.probe_seq[2 * b] = NAN;
          P.probe_seq[2 * b + 1] = NAN;
        }
      }
    }
    return;
  }
  const int kstar = n_acc + 1;
  const int trow = s.t0 + kstar - 1;
  const bool residual = kstar <= s.g;
  const uint4* prow = reinterpret_cast<const uint4*>(P.target + (size_t)trow * P.stride);
  const float c = s.T == 0.0f ? 0.0f : kLog2e / s.T;
  int y;
  float R = NAN, py;
  if (!residual) {  // every draft accepted: the bonus token from p_{gamma+1}
    if (s.T == 0.0f) {
      y = sbon.argmax;
      py = 1.0f;
    } else {
      const float u = P.ovr ? P.ovr[(size_t)trow * 2 + 1]
                            : uniform24(P.seed_lo, P.seed_hi, s.id, (uint32_t)(s.L + kstar),
                                        SPEC_PURPOSE_BONUS);
      flags |= sbon.flags & SPEC_FLAG_TOPP_SLOW;
      Draw d;
      if (sbon.nuc >= 0) {
        const NucEntry* lb = s_preb;
        if (sbon.nuc > kPre) {
          const NucEntry* gl = P.nuc + bonus_slot(P, b) * kNucMax;
          for (int j = tid; j < sbon.nuc; j += NT) s_lp[j] = gl[j];
          __syncthreads();
          lb = s_lp;
        }
        d = wg_list_draw(lb, sbon.nuc, sbon.z, nullptr, 0, 1.0f, false, u, sh_i, sh_f);
      } else {
        const RowLaw Lp{prow, c, -sbon.m * c, sbon.t, sbon.z};
        d = draw_from_rows<NT, TI>(Lp, Lp, false, P.nvec, P.V, u, tile_sum, sh_i, sh_f);
      }
      y = d.token;
      py = d.wtok;
    }
  } else if (s.T == 0.0f) {
    y = sd.sp.argmax;
    py = 1.0f;
  } else {  // first rejection at kstar: the residual max(0, p - q), or p if it has no mass
    const RowStat sp = sd.sp, sq = sd.sq;
    const float u = P.ovr ? P.ovr[(size_t)trow * 2 + 1]
                          : uniform24(P.seed_lo, P.seed_hi, s.id, (uint32_t)(s.L + kstar),
                                      SPEC_PURPOSE_RESIDUAL);
    const RowLaw Lp{prow, c, -sp.m * c, sp.t, sp.z};
    // no draft rows: the draft law is the point mass at the draft token
    const RowLaw Lq = P.draft ? RowLaw{reinterpret_cast<const uint4*>(
                                           P.draft + (size_t)(s.d0 + kstar - 1) * P.stride),
                                       c, -sq.m * c, sq.t, sq.z}
                              : RowLaw{nullptr, c, 0.0f, -INFINITY, 1.0f,
                                       sd.tok[kstar - 1]};
    Draw d;
    const bool lists_p = sp.nuc >= 0, lists_pq = lists_p && sq.nuc >= 0;
    const NucEntry* lp = s_lp;
    const NucEntry* lq = s_lq;
    if (lists_p) {
      if (kstar - 1 < kPreRows && sp.nuc <= kPre && sq.nuc <= kPre) {
        lp = s_pre[kstar - 1][0];
        lq = s_pre[kstar - 1][1];
      } else {
        const NucEntry* gl = P.nuc + (size_t)(s.d0 + kstar - 1) * 2 * kNucMax;
        for (int j = tid; j < sp.nuc; j += NT) s_lp[j] = gl[j];
        if (lists_pq)
          for (int j = tid; j < sq.nuc; j += NT) s_lq[j] = gl[kNucMax + j];
        __syncthreads();
      }
    }
    if (lists_pq) d = wg_list_draw(lp, sp.nuc, sp.z, lq, sq.nuc, sq.z, true, u, sh_i, sh_f);
    else d = draw_from_rows<NT, TI>(Lp, Lq, true, P.nvec, P.V, u, tile_sum, sh_i, sh_f);
    R = d.total;
    if (d.total > 0.0f) {
      y = d.token;
      py = d.wtok / d.total;
    } else {  // R = 0 means p = q: the draw from p has the same law
      flags |= SPEC_FLAG_RESID_FALLBACK;
      if (lists_p) d = wg_list_draw(lp, sp.nuc, sp.z, nullptr, 0, 1.0f, false, u, sh_i, sh_f);
      else d = draw_from_rows<NT, TI>(Lp, Lq, false, P.nvec, P.V, u, tile_sum, sh_i, sh_f);
      y = d.token;
      py = d.wtok;
    }
  }
  if (wid == 0) {
    if (lane < n_acc) P.out_tokens[s.t0 + lane] = sd.tok[lane];
    if (lane == 0) {
      if (s.eos >= 0 && y == s.eos) flags |= SPEC_FLAG_EOS;
      P.out_tokens[s.t0 + n_acc] = y;
      P.num_acc[b] = n_acc;
      if (P.num_emit) P.num_emit[b] = n_acc + 1;
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

// Row statistics, nucleus lists and spill lists for the 2 * total_draft_rows draft-position
// rows and the batch's bonus rows.
size_t chain_workspace_bytes(int32_t batch, int32_t total_draft_rows, int32_t vocab) {
  (void)vocab;
  const size_t rows = 2 * (size_t)total_draft_rows + (size_t)batch;
  const size_t n = align256(rows * sizeof(RowStat)) + align256(rows * kNucMax * sizeof(NucEntry)) +
                   align256(rows * kCapG * sizeof(uint16_t));
  return n > 256 ? n : 256;
}

hipError_t launch_chain(const spec_chain_args& a, void* ws, hipStream_t st, void* const* events) {
  ChainParams P;
  P.target = a.target_logits;
  P.draft = a.draft_logits;
  P.cu = a.cu_gamma;
  P.tokens = a.draft_tokens;
  P.temp = a.temperature;
  P.topp = a.top_p;
  P.topk = a.top_k;
  P.eos = a.eos_token;
  P.cap = a.max_emit;
  P.sid = a.seq_id;
  P.committed = a.committed_len;
  P.out_tokens = a.out_tokens;
  P.num_acc = a.num_accepted;
  P.num_emit = a.num_emitted;
  P.flags_out = a.seq_flags;
  P.probe_rows = a.probe_rows;
  P.probe_seq = a.probe_seq;
  P.ovr = a.uniform_override;
  const size_t rows = 2 * (size_t)a.total_draft_rows + (size_t)a.batch;
  P.stat = reinterpret_cast<RowStat*>(ws);
  char* w = reinterpret_cast<char*>(ws) + align256(rows * sizeof(RowStat));
  P.nuc = reinterpret_cast<NucEntry*>(w);
  P.spill = reinterpret_cast<uint16_t*>(w + align256(rows * kNucMax * sizeof(NucEntry)));
  P.B = a.batch;
  P.V = a.vocab;
  P.stride = a.row_stride;
  P.nvec = (a.vocab + 7) / 8;
  P.max_gamma = a.max_gamma;
  P.n_draft = a.total_draft_rows;
  P.lead = a.lead_slots;
  P.seed_lo = (uint32_t)(a.seed & 0xFFFFFFFFu);
  P.seed_hi = (uint32_t)(a.seed >> 32);
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
  hipError_t e = hipSuccess;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  // per sequence: two rows (target, draft) per draft position slot k <= max_gamma, then the
  // bonus row
  const unsigned nrows = (unsigned)a.batch * (2u * (unsigned)a.max_gamma + 1u);
  if (a.top_k || a.top_p)
    hipLaunchKernelGGL((row_stats_kernel<true>), dim3(nrows), dim3(kRowThreads), 0, st, P);
  else
    hipLaunchKernelGGL((row_stats_kernel<false>), dim3(nrows), dim3(kRowThreads), 0, st, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  if (a.batch > kNumCus)
    hipLaunchKernelGGL((chain_resolve_kernel<kResolveNarrow, kTilesNarrow>),
                       dim3((unsigned)a.batch), dim3(kResolveNarrow), 0, st, P);
  else
    hipLaunchKernelGGL((chain_resolve_kernel<kResolveWide, kTilesWide>), dim3((unsigned)a.batch),
                       dim3(kResolveWide), 0, st, P);
  return hipGetLastError();
}

}  // namespace specv
