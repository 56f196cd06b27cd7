// tree_draft.hip -- one tree-drafting step on gfx950 ("投机推理：小模型搭树，大模型一次验证",
// tree configuration and draft-step sections; "10.6 投机解码" §10.6.3, tree drafts and
// Table 10-17).
//
//  1. draft_topk_kernel -- every draft row of the step is split into S chunks, one
//     256-thread workgroup per chunk. The chunk streams from HBM once with 16-byte loads,
//     two trips of 2 KB per wave in flight. Every lane keeps a running maximum and sum of
//     exp(l - max) (the softmax normaliser); every wave keeps (logit, token) candidates in LDS
//     behind a threshold: first the K-th largest of its lanes' first-trip maxima (K logits lie
//     at or above it), then the K-th largest candidate held, so that a trip whose lanes all
//     stay below it costs one ballot. A wave's best K come from K rounds of a wave-wide
//     maximum over its candidates; the workgroup merges its waves' lists and writes one record
//     (max, sum, best K) per chunk.
//  2. tree_grow_kernel -- one workgroup per sequence merges each expanded node's S records
//     into the row's normaliser and its K best tokens, appends the children with their path
//     log-probabilities, positions and ancestor-mask rows, and ranks the new layer by path
//     log-probability to choose the next step's expanded nodes and their target rows.
//
// Every address of the tree arrays has one writer per launch, so no write of one thread is
// ordered against another's.
#include "row_ops.h"
#include "spec_device.h"
#include "specv_internal.h"

namespace specv {
namespace {

constexpr int kDraftWaves = 4;
constexpr int kDraftThreads = kDraftWaves * kWave;
constexpr int kTv = 2;                  // vectors per lane per trip
constexpr int kTripVec = kTv * kWave;   // a wave's trip: 128 vectors, 1024 logits
constexpr int kStageSlots = 2 * kWave;  // staged lane-trips per wave
constexpr int kFlushLanes = 32;         // staged lane-trips turned into candidates at once
constexpr int kCandCap = kFlushLanes * kTv * 8 + kTreeDraftMaxK;  // a compacted list + a group
constexpr int kGrowThreads = 256;
constexpr int kGrowWaves = kGrowThreads / kWave;
constexpr int kStageCap = kTreeDraftMaxSplits * kTreeDraftMaxK;  // a row's merged candidates
constexpr int kMaxHead = kTreeDraftMaxHead;
constexpr int kMaskWordsMax = 8;  // 256 nodes
constexpr int kTargetWgs = 1024;  // four 256-thread workgroups per CU
constexpr int kMinChunkVec = 1024;
constexpr float kLog2e = 1.4426950408889634f;

// A candidate packs the bf16 order key above the complement of the token id: the larger
// candidate has the larger logit, or the same logit and the lower id. 0 is no candidate (key 0
// is a NaN pattern, and logits are never NaN).
__device__ __forceinline__ uint64_t cand_of(uint32_t bits16, uint32_t idx) {
  return ((uint64_t)key_of_bits(bits16) << 32) | (uint32_t)~idx;
}
__device__ __forceinline__ int cand_token(uint64_t c) { return (int)~(uint32_t)c; }
__device__ __forceinline__ float cand_logit(uint64_t c) {
  return value_of_key((uint32_t)(c >> 32));
}

// One DPP step of a 64-bit maximum: lanes that the move does not write keep their own value.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_max_u64_step(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v,
                                                            CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(
      (int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  const uint64_t w = ((uint64_t)hi << 32) | lo;
  return w > v ? w : v;
}
// Wave maximum of a 64-bit value through the same DPP tree as wave_max_dpp, read back from
// lane 63.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64_step<0xB1>(v);
  v = dpp_max_u64_step<0x4E>(v);
  v = dpp_max_u64_step<0x141>(v);
  v = dpp_max_u64_step<0x140>(v);
  v = dpp_max_u64_step<0x142, 0xA>(v);
  v = dpp_max_u64_step<0x143, 0xC>(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// The K (<= 64) largest of the candidates src[0..n) in LDS (0 = empty slot), largest first:
// lane r receives the r-th in `mine` (0 past the end). Returns how many exist. K rounds, each
// a scan of the lane's entries and a wave maximum below the previous round's.
__device__ __forceinline__ int wave_select(const uint64_t* src, int n, int K, int lane,
                                           uint64_t& mine) {
  uint64_t prev = ~0ull;
  int found = 0;
  mine = 0;
  for (int r = 0; r < K; ++r) {
    uint64_t best = 0;
    for (int j = lane; j < n; j += kWave) {
      const uint64_t e = src[j];
      best = (e < prev && e > best) ? e : best;
    }
    best = wave_max_u64(best);
    if (best == 0) break;
    if (lane == r) mine = best;
    prev = best;
    ++found;
  }
  return found;
}

// Reduces a wave's candidate buffer to its K best, largest first, in place, and returns the
// new count; tau rises to the K-th best's logit when K are held.
__device__ __forceinline__ int compact(uint64_t* buf, int n, int K, float& tau, int lane) {
  uint64_t mine;
  const int f = wave_select(buf, n, K, lane, mine);
  if (lane < f) buf[lane] = mine;  // every read of the rounds above precedes this write
  if (f == K) tau = fmaxf(tau, cand_logit(readlane_u64(mine, K - 1)));
  return f;
}

// The K-th largest of the 64 lanes' values v, repeats counted (-inf if fewer than K lanes
// hold a finite value): at least K lanes hold a value at or above it.
__device__ __forceinline__ float lane_kth_max(float v, int K) {
  float last = -INFINITY;
  int taken = 0;
  while (taken < K) {
    const float m = wave_max_dpp(v);
    if (m == -INFINITY) return -INFINITY;
    taken += __popcll(__ballot(v == m));
    last = m;
    v = (v == m) ? -INFINITY : v;
  }
  return last;
}

struct DraftParams {
  const uint16_t* logits;
  uint8_t* part;
  int32_t V, stride, nvec, S, chunk, h, rec_bytes;
  int32_t kk[kMaxHead];
};

struct PartHead {
  float m;  // largest logit of the chunk (-inf if none)
  float s;  // sum over the chunk of exp(l - m)
  int32_t n;
  int32_t pad;
};

// Loads one trip (kTv vectors per lane, kWave vectors apart) of a chunk of nv vectors;
// vectors past the chunk read as -inf. The loads are nontemporal: every draft row is read once.
__device__ __forceinline__ void load_trip2(const uint4* __restrict__ base, int v0, int nv,
                                           int lane, uint4 (&d)[kTv]) {
  if (v0 + kTripVec <= nv) {
#pragma unroll
    for (int u = 0; u < kTv; ++u) d[u] = ld_row(base + v0 + u * kWave + lane);
  } else {
#pragma unroll
    for (int u = 0; u < kTv; ++u) {
      const int v = v0 + u * kWave + lane;
      d[u] = v < nv ? ld_row(base + v) : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
    }
  }
}

__global__ __launch_bounds__(kDraftThreads) void draft_topk_kernel(DraftParams P) {
  __shared__ uint64_t s_buf[kDraftWaves][kCandCap];
  __shared__ uint4 s_stage[kDraftWaves][kStageSlots][kTv];
  __shared__ int s_svec[kDraftWaves][kStageSlots];
  __shared__ float s_m[kDraftWaves], s_s[kDraftWaves];
  __shared__ int s_n[kDraftWaves];
  __shared__ float s_tau;  // the largest of the waves' thresholds: a bound for the whole chunk
  const int row = blockIdx.x / P.S;
  const int split = blockIdx.x - row * P.S;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int K = P.kk[row % P.h];
  const int c0 = split * P.chunk;
  const int nv = max(0, min(P.nvec, c0 + P.chunk) - c0);  // vectors of this chunk
  const int lim = min(P.V, (c0 + nv) * 8);                 // its token ids lie below lim
  uint64_t* buf = s_buf[wave];
  uint4 (*stage)[kTv] = s_stage[wave];
  int* svec = s_svec[wave];
  float m = -INFINITY, s = 0.f, tau = -INFINITY;
  int n = 0;   // candidates in buf
  int ns = 0;  // staged lane-trips
  bool first = true;
  const uint4* base = reinterpret_cast<const uint4*>(P.logits + (size_t)row * P.stride) + c0;
  if (tid == 0) s_tau = -INFINITY;
  __syncthreads();
  // Any wave's threshold bounds the chunk's K-th largest logit from below (that wave holds K
  // logits at or above it), so every wave filters with the largest one published.
  auto publish = [&]() {
    if (lane == 0)
      __hip_atomic_fetch_max(&s_tau, tau, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };

  // Turns the staged lane-trips into candidates, kFlushLanes at a time (one per lane): each
  // lane appends the logits of its lane-trip that reach the threshold.
  auto flush = [&]() {
    for (int g = 0; g < ns; g += kFlushLanes) {
      if (n + kFlushLanes * kTv * 8 > kCandCap) {  // then n <= K <= 64
        n = compact(buf, n, K, tau, lane);
        publish();
      }
      const int e = g + lane;
      uint32_t fl = 0;
      float x[kTv * 8] = {};
      int vb = 0;
      if (lane < kFlushLanes && e < ns) {
        vb = svec[e];
#pragma unroll
        for (int u = 0; u < kTv; ++u) unpack8(stage[e][u], x + 8 * u);
#pragma unroll
        for (int i = 0; i < kTv * 8; ++i) {
          const int idx = (vb + (i >> 3) * kWave) * 8 + (i & 7);
          fl |= (uint32_t)(x[i] >= tau && idx < lim) << i;
        }
      }
      const int cnt = __popc(fl);
      const int incl = wave_incl_scan_dpp(cnt);
      const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
      int off = n + incl - cnt;
      while (fl) {
        const int i = __builtin_ctz(fl);
        fl &= fl - 1;
        float val = x[0];
#pragma unroll
        for (int k = 1; k < kTv * 8; ++k) val = (i == k) ? x[k] : val;
        const int idx = (vb + (i >> 3) * kWave) * 8 + (i & 7);
        buf[off++] = cand_of(__float_as_uint(val) >> 16, (uint32_t)idx);
      }
      n += total;
    }
    ns = 0;
  };

  auto consume = [&](uint4 (&d)[kTv], int v0) {
    if (c0 + v0 + kTripVec >= P.nvec) {  // the trip may hold the row's last vector
      const int rem = P.V & 7;
#pragma unroll
      for (int u = 0; u < kTv; ++u) {
        if (rem != 0 && c0 + v0 + u * kWave + lane == P.nvec - 1) {
          uint32_t w[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (e >= rem) {
              if (e & 1) w[e >> 1] = (w[e >> 1] & 0x0000FFFFu) | 0xFF800000u;
              else w[e >> 1] = (w[e >> 1] & 0xFFFF0000u) | 0x0000FF80u;
            }
          }
          d[u] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
    float x[kTv * 8];
#pragma unroll
    for (int u = 0; u < kTv; ++u) unpack8(d[u], x + 8 * u);
    float tm = vmax3(x[0], x[1], x[2]);
#pragma unroll
    for (int i = 3; i + 1 < kTv * 8; i += 2) tm = vmax3(tm, x[i], x[i + 1]);
    tm = vmax3(tm, x[kTv * 8 - 1], x[kTv * 8 - 1]);
    if (tm > m) {
      s = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - tm) * kLog2e);
      m = tm;
    }
    if (m != -INFINITY) {
      const float nref = -m * kLog2e;
#pragma unroll
      for (int i = 0; i < kTv * 8; ++i) s += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, nref));
    }
    if (first) {  // seed the threshold: K lanes hold a logit at or above this bound
      tau = lane_kth_max(tm, K);
      first = false;
      publish();
    }
    tau = fmaxf(tau, __hip_atomic_load(&s_tau, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    // lanes whose trip maximum reaches the threshold stage their lane-trip
    const bool pass = tm >= tau;
    const uint64_t bal = __ballot(pass);
    if (bal == 0) return;  // wave-uniform
    if (pass) {
      const int sl = ns + (int)__builtin_amdgcn_mbcnt_hi(
                              (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
#pragma unroll
      for (int u = 0; u < kTv; ++u) stage[sl][u] = d[u];
      svec[sl] = c0 + v0 + lane;
    }
    ns += (int)__popcll(bal);
    if (ns > kStageSlots - kWave) flush();  // a trip stages at most kWave lane-trips
  };

  // this wave's trips t = wave, wave + 4, ...: two in flight, alternating buffers
  int t = wave;
  uint4 da[kTv], db[kTv];
  if (t * kTripVec < nv) load_trip2(base, t * kTripVec, nv, lane, da);
  while (t * kTripVec < nv) {
    const int t1 = t + kDraftWaves;
    if (t1 * kTripVec < nv) load_trip2(base, t1 * kTripVec, nv, lane, db);
    consume(da, t * kTripVec);
    if (t1 * kTripVec >= nv) break;
    const int t2 = t1 + kDraftWaves;
    if (t2 * kTripVec < nv) load_trip2(base, t2 * kTripVec, nv, lane, da);
    consume(db, t1 * kTripVec);
    t = t2;
  }
  if (ns > 0) flush();
  // the wave's normaliser relative to its own maximum
  const float mw = wave_max_dpp(m);
  const float sw = wave_sum_dpp(m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - mw) * kLog2e));
  if (lane == 0) {
    s_m[wave] = mw;
    s_s[wave] = sw;
    s_n[wave] = n;
  }
  __syncthreads();
  if (wave != 0) return;
  // wave 0 selects the chunk's K best from every wave's candidates
  uint64_t mine = 0;
  int f = 0;
  {
    uint64_t prev = ~0ull;
    for (int r = 0; r < K; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int w = 0; w < kDraftWaves; ++w) {
        const int nw = s_n[w];
        for (int j = lane; j < nw; j += kWave) {
          const uint64_t e = s_buf[w][j];
          best = (e < prev && e > best) ? e : best;
        }
      }
      best = wave_max_u64(best);
      if (best == 0) break;
      if (lane == r) mine = best;
      prev = best;
      ++f;
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDraftWaves; ++w) M = fmaxf(M, s_m[w]);
  float Z = 0.f;
#pragma unroll
  for (int w = 0; w < kDraftWaves; ++w)
    Z += s_m[w] == -INFINITY ? 0.f : s_s[w] * __builtin_amdgcn_exp2f((s_m[w] - M) * kLog2e);
  uint8_t* rec = P.part + (size_t)blockIdx.x * P.rec_bytes;
  if (lane == 0) {
    PartHead hd;
    hd.m = M;
    hd.s = Z;
    hd.n = f;
    hd.pad = 0;
    *reinterpret_cast<PartHead*>(rec) = hd;
  }
  if (lane < K) reinterpret_cast<uint64_t*>(rec + sizeof(PartHead))[lane] = lane < f ? mine : 0ull;
}

struct GrowParams {
  const uint8_t* part;
  const int32_t* root_token;
  const int32_t* pos_base;
  int32_t* parent;
  int32_t* node_token;
  int32_t* node_row;
  float* node_logp;
  int32_t* position_ids;
  uint32_t* mask;
  int32_t* expand_nodes;
  int32_t* seq_flags;
  int32_t step, ts, mw, es, h, S, rec_bytes;
  int32_t par_lo, par_hi, first_new, n_new, h_next, row_base_next;
  int32_t kk[kMaxHead];
  int32_t koff[kMaxHead];
};

// candidates per lane staged through registers in one round of loads (the rest, past
// kStageRegs * 64, one at a time)
constexpr int kStageRegs = 4;

__global__ __launch_bounds__(kGrowThreads) void tree_grow_kernel(GrowParams P) {
  __shared__ uint64_t s_stage[kGrowWaves][kStageCap];
  __shared__ uint32_t s_pmask[kGrowWaves][kMaskWordsMax];
  __shared__ int s_ctok[kTreeDraftMaxNodes], s_cpar[kTreeDraftMaxNodes];
  __shared__ int s_cpos[kTreeDraftMaxNodes];
  __shared__ float s_lp[kTreeDraftMaxNodes];
  __shared__ uint32_t s_cmask[kTreeDraftMaxNodes][kMaskWordsMax];
  __shared__ int s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const size_t nb = (size_t)b * P.ts;
  int32_t* par = P.parent + nb;
  int32_t* tok = P.node_token + nb;
  int32_t* nrow = P.node_row + nb;
  float* lp = P.node_logp + nb;
  int32_t* pos = P.position_ids + nb;
  uint32_t* mask = P.mask + nb * P.mw;
  int32_t* expn = P.expand_nodes + (size_t)b * P.es;
  const int new_hi = P.first_new + P.n_new;
  if (tid == 0) s_bad = 0;
  if (P.step == 0) {
    // every entry but this step's new nodes (written at the end) gets its initial value
    for (int i = tid; i < P.ts; i += kGrowThreads) {
      if (i >= P.first_new && i < new_hi) continue;
      const bool root = i == 0;
      par[i] = -1;
      tok[i] = root ? P.root_token[b] : -1;
      nrow[i] = root ? 0 : -1;
      lp[i] = root ? 0.f : -INFINITY;
      pos[i] = root ? (P.pos_base ? P.pos_base[b] : 0) : -1;
    }
    for (int k = tid; k < P.ts * P.mw; k += kGrowThreads) {
      const int i = k / P.mw;
      if (i >= P.first_new && i < new_hi) continue;
      mask[k] = (k == 0) ? 1u : 0u;
    }
  }
  __syncthreads();  // s_bad is set before any wave may raise it
  // Children of each expanded node, one wave per node, kept in LDS until every expanded node
  // has been checked. The node's chunk records are loaded together with the node itself.
  for (int j = wave; j < P.h; j += kGrowWaves) {
    const size_t row = (size_t)b * P.h + j;
    const uint8_t* rec0 = P.part + row * P.S * P.rec_bytes;
    const int K = P.kk[j];
    const int nc = P.S * K;  // the S chunk lists, K candidates each
    uint64_t* stage = s_stage[wave];
    auto cand = [&](int i) {
      const int li = i / K, r = i - li * K;
      return reinterpret_cast<const uint64_t*>(rec0 + (size_t)li * P.rec_bytes +
                                               sizeof(PartHead))[r];
    };
    const int pnode = P.step == 0 ? 0 : expn[j];
    const bool bad = pnode < P.par_lo || pnode >= P.par_hi;
    if (bad) {
      if (lane == 0) s_bad = 1;
      continue;
    }
    // the parent's path log-probability, position and mask row, the chunk heads and the
    // candidates all load together (the candidates into registers from clamped indexes),
    // one memory round trip after the parent's index
    float plp = 0.f;
    int ppos = P.pos_base ? P.pos_base[b] : 0;
    uint32_t pm = lane == 0 ? 1u : 0u;
    if (P.step != 0) {
      plp = lp[pnode];
      ppos = pos[pnode];
      pm = mask[(size_t)pnode * P.mw + min(lane, P.mw - 1)];
    }
    float m = -INFINITY, sm = 0.f;
    {
      const PartHead hd =
          *reinterpret_cast<const PartHead*>(rec0 + (size_t)min(lane, P.S - 1) * P.rec_bytes);
      if (lane < P.S) {
        m = hd.m;
        sm = hd.s;
      }
    }
    uint64_t cv[kStageRegs];
#pragma unroll
    for (int u = 0; u < kStageRegs; ++u) cv[u] = cand(min(lane + u * kWave, nc - 1));
#pragma unroll
    for (int u = 0; u < kStageRegs; ++u)
      if (lane + u * kWave < nc) stage[lane + u * kWave] = cv[u];
    for (int i = lane + kStageRegs * kWave; i < nc; i += kWave) stage[i] = cand(i);
    if (lane < P.mw) s_pmask[wave][lane] = pm;
    const float M = wave_max_dpp(m);
    const float Z = wave_sum_dpp(m == -INFINITY ? 0.f : sm * __builtin_amdgcn_exp2f((m - M) * kLog2e));
    const float lz = logf(Z);  // log of sum over the row of exp(l - M)
    uint64_t mine;
    const int f = wave_select(stage, nc, K, lane, mine);
    if (lane < f) {
      const int c = P.first_new + P.koff[j] + lane;
      const int t = c - P.first_new;
      s_ctok[t] = cand_token(mine);
      s_cpar[t] = pnode;
      s_cpos[t] = ppos + 1;
      s_lp[t] = plp + ((cand_logit(mine) - M) - lz);
      for (int w = 0; w < P.mw; ++w)
        s_cmask[t][w] = s_pmask[wave][w] | ((c >> 5) == w ? 1u << (c & 31) : 0u);
    }
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && P.seq_flags) P.seq_flags[b] |= SPEC_FLAG_BAD_TREE;
    return;
  }
  // the new nodes, and the new layer's rows: its h_next most probable nodes get the next
  // step's target rows
  for (int t = tid; t < P.n_new; t += kGrowThreads) {
    const int c = P.first_new + t;
    par[c] = s_cpar[t];
    tok[c] = s_ctok[t];
    lp[c] = s_lp[t];
    pos[c] = s_cpos[t];
    const float me = s_lp[t];
    int rank = 0;
    for (int u = 0; u < P.n_new; ++u) {
      const float o = s_lp[u];
      rank += (o > me) || (o == me && u < t);
    }
    const bool chosen = rank < P.h_next;
    nrow[c] = chosen ? P.row_base_next + rank : -1;
    if (chosen) expn[rank] = c;
  }
  for (int k = tid; k < P.n_new * P.mw; k += kGrowThreads) {
    const int t = k / P.mw, w = k - t * P.mw;
    mask[(size_t)(P.first_new + t) * P.mw + w] = s_cmask[t][w];
  }
}

}  // namespace

int tree_draft_splits(int32_t rows, int32_t vocab) {
  const int nvec = (vocab + 7) / 8;
  int s = (kTargetWgs + rows - 1) / max(rows, 1);
  const int cap = max(1, min(kTreeDraftMaxSplits, nvec / kMinChunkVec));
  return max(1, min(s, cap));
}

size_t tree_draft_record_bytes(int32_t kmax) {
  return sizeof(PartHead) + (size_t)kmax * sizeof(uint64_t);
}

hipError_t launch_tree_draft(const spec_tree_draft_args& a, const TreeDraftPlan& p, void* ws,
                             hipStream_t st) {
  DraftParams D;
  D.logits = a.draft_logits;
  D.part = reinterpret_cast<uint8_t*>(ws);
  D.V = a.vocab;
  D.stride = a.row_stride;
  D.nvec = (a.vocab + 7) / 8;
  D.S = p.splits;
  D.chunk = (D.nvec + p.splits - 1) / p.splits;
  D.h = p.h;
  D.rec_bytes = (int32_t)tree_draft_record_bytes(p.kmax);
  for (int j = 0; j < kMaxHead; ++j) D.kk[j] = j < p.h ? p.kk[j] : 0;
  const unsigned grid = (unsigned)(a.batch * p.h * p.splits);
  hipLaunchKernelGGL(draft_topk_kernel, dim3(grid), dim3(kDraftThreads), 0, st, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GrowParams G;
  G.part = D.part;
  G.root_token = a.root_token;
  G.pos_base = a.pos_base;
  G.parent = a.parent;
  G.node_token = a.node_token;
  G.node_row = a.node_row;
  G.node_logp = a.node_logp;
  G.position_ids = a.position_ids;
  G.mask = a.ancestor_mask;
  G.expand_nodes = a.expand_nodes;
  G.seq_flags = a.seq_flags;
  G.step = a.step;
  G.ts = a.tree_stride;
  G.mw = (a.tree_stride + 31) / 32;
  G.es = a.expand_stride;
  G.h = p.h;
  G.S = p.splits;
  G.rec_bytes = D.rec_bytes;
  G.par_lo = p.par_lo;
  G.par_hi = p.par_hi;
  G.first_new = p.first_new;
  G.n_new = p.n_new;
  G.h_next = p.h_next;
  G.row_base_next = p.row_base_next;
  for (int j = 0; j < kMaxHead; ++j) {
    G.kk[j] = j < p.h ? p.kk[j] : 0;
    G.koff[j] = j < p.h ? p.koff[j] : 0;
  }
  hipLaunchKernelGGL(tree_grow_kernel, dim3((unsigned)a.batch), dim3(kGrowThreads), 0, st, G);
  return hipGetLastError();
}

}  // namespace specv
