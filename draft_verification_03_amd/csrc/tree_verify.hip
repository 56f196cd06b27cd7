// tree_verify.hip -- greedy verification of a draft tree on gfx950
// ("投机推理：小模型搭树，大模型一次验证", validation and path-walk sections; the tree rows
// come from one target forward with a tree attention mask, "10.6 投机解码" §10.6.3).
//
//  1. tree_argmax_kernel -- one 8-wave workgroup per provided target row: the waves claim the
//     row's 4 KB trips from an LDS counter (two in flight per wave, nontemporal 16-byte loads:
//     every row is read once) and keep per-lane maxima
//     with the earliest index; wave, then workgroup reductions give the argmax (lowest id on
//     ties), written to the workspace.
//  2. tree_walk_kernel   -- one wave per sequence: checks the topology, then walks from the
//     root along the child whose token equals the target argmax of the current node (the
//     lowest node index among matching siblings), never combining matches of different
//     branches, and emits the path tokens plus the argmax at the stopping node when that
//     node has a row.
#include "row_ops.h"
#include "spec_device.h"
#include "specv_internal.h"

namespace specv {
namespace {

constexpr int kMaxNodes = 256;
constexpr int kMaxRows = 256;
constexpr int kArgWaves = 8;

struct TreeParams {
  const uint16_t* logits;
  const int32_t* parent;
  const int32_t* node_row;
  const int32_t* node_token;
  int32_t* path_nodes;
  int32_t* path_len;
  int32_t* out_tokens;
  int32_t* num_emitted;
  int32_t* seq_flags;
  int32_t* argmax;  // workspace [B][rows_per_seq]
  int32_t B, V, stride, nvec, N, R, max_depth, tree_stride;
};

__global__ __launch_bounds__(kArgWaves * kWave) void tree_argmax_kernel(TreeParams P) {
  __shared__ int s_trip;
  __shared__ float s_bv[kArgWaves];
  __shared__ int s_bi[kArgWaves];
  const int row = blockIdx.x;  // b * R + r
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  if (threadIdx.x == 0) s_trip = 0;
  __syncthreads();
  const uint4* rp = reinterpret_cast<const uint4*>(P.logits + (size_t)row * P.stride);
  // a wave's claims increase, so each lane meets its trips in token order and keeps the
  // earliest index of its maximum
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  stream_row_claimed<2>(rp, P.nvec, lane, &s_trip, [&](uint4* d, int v0, bool) {
    argmax_trip(d, v0, P.nvec, P.V, lane, bv, bi);
  });
  wave_argmax(bv, bi);
  if (lane == 0) {
    s_bv[wid] = bv;
    s_bi[wid] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgWaves; ++w)
      if (s_bv[w] > bv || (s_bv[w] == bv && s_bi[w] < bi)) {
        bv = s_bv[w];
        bi = s_bi[w];
      }
    P.argmax[row] = bi == 0x7FFFFFFF ? 0 : bi;
  }
}

__global__ __launch_bounds__(kWave) void tree_walk_kernel(TreeParams P) {
  __shared__ int32_t s_par[kMaxNodes], s_row[kMaxNodes], s_tok[kMaxNodes];
  __shared__ int32_t s_am[kMaxRows];
  const int b = blockIdx.x;
  const int lane = lane_id();
  const int32_t* par = P.parent + (size_t)b * P.tree_stride;
  const int32_t* nrow = P.node_row + (size_t)b * P.tree_stride;
  const int32_t* tok = P.node_token + (size_t)b * P.N;
  // every load first (clamped indexes; entries past N or R are dropped), so that the
  // tree and the row argmaxes arrive in one memory round trip
  constexpr int kNodesPerLane = kMaxNodes / kWave, kRowsPerLane = kMaxRows / kWave;
  int pv[kNodesPerLane], rv[kNodesPerLane], tv[kNodesPerLane], av[kRowsPerLane];
#pragma unroll
  for (int k = 0; k < kNodesPerLane; ++k) {
    const int i = min(lane + k * kWave, P.N - 1);
    pv[k] = par[i];
    rv[k] = nrow[i];
    tv[k] = tok[i];
  }
#pragma unroll
  for (int k = 0; k < kRowsPerLane; ++k)
    av[k] = P.argmax[(size_t)b * P.R + min(lane + k * kWave, P.R - 1)];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kNodesPerLane; ++k) {
    const int i = lane + k * kWave;
    if (i < P.N) {
      s_par[i] = pv[k];
      s_row[i] = rv[k];
      s_tok[i] = tv[k];
      bad |= (i == 0) ? (pv[k] != -1) : (pv[k] < 0 || pv[k] >= i);
      bad |= (rv[k] < -1 || rv[k] >= P.R);
    } else {
      s_par[i] = -2;  // never a parent
    }
  }
#pragma unroll
  for (int k = 0; k < kRowsPerLane; ++k)
    if (lane + k * kWave < P.R) s_am[lane + k * kWave] = av[k];
  bad = __ballot(bad) != 0;
  __syncthreads();
  int32_t* path = P.path_nodes + (size_t)b * P.max_depth;
  for (int j = lane; j < P.max_depth; j += kWave) path[j] = -1;
  if (bad) {
    if (lane == 0) {
      P.path_len[b] = 0;
      P.num_emitted[b] = 0;
      if (P.seq_flags) P.seq_flags[b] = SPEC_FLAG_BAD_TREE;
    }
    return;
  }
  int32_t* out = P.out_tokens + (size_t)b * (P.max_depth + 1);
  int v = 0, D = 0, extra = -1, flags = 0;
  for (;;) {  // at most max_depth + 1 steps: D grows by one per matched step
    const int r = s_row[v];
    if (r < 0) {
      flags |= SPEC_FLAG_NO_ROW;
      break;
    }
    const int t = s_am[r];
    int child = -1;
    if (D < P.max_depth) {
      for (int j = 0; j < kMaxNodes / kWave && child < 0; ++j) {
        const int i = j * kWave + lane;
        const uint64_t m = __ballot(s_par[i] == v && s_tok[i] == t);
        if (m) child = j * kWave + __ffsll((long long)m) - 1;
      }
    }
    if (child < 0) {
      extra = t;
      break;
    }
    if (lane == 0) {
      path[D] = child;
      out[D] = s_tok[child];
    }
    ++D;
    v = child;
  }
  if (lane == 0) {
    if (extra >= 0) out[D] = extra;
    P.path_len[b] = D;
    P.num_emitted[b] = D + (extra >= 0 ? 1 : 0);
    if (P.seq_flags) P.seq_flags[b] = flags;
  }
}

}  // namespace

size_t tree_workspace_bytes(int32_t batch, int32_t rows_per_seq) {
  return align256((size_t)batch * (size_t)rows_per_seq * sizeof(int32_t));
}

hipError_t launch_tree(const spec_tree_args& a, void* ws, hipStream_t st) {
  TreeParams P;
  P.logits = a.target_logits;
  P.parent = a.parent;
  P.node_row = a.node_row;
  P.node_token = a.node_token;
  P.path_nodes = a.path_nodes;
  P.path_len = a.path_len;
  P.out_tokens = a.out_tokens;
  P.num_emitted = a.num_emitted;
  P.seq_flags = a.seq_flags;
  P.argmax = reinterpret_cast<int32_t*>(ws);
  P.B = a.batch;
  P.V = a.vocab;
  P.stride = a.row_stride;
  P.nvec = (a.vocab + 7) / 8;
  P.N = a.num_nodes;
  P.R = a.rows_per_seq;
  P.max_depth = a.max_depth;
  P.tree_stride = a.tree_stride;
  hipLaunchKernelGGL(tree_argmax_kernel, dim3((unsigned)(a.batch * a.rows_per_seq)),
                     dim3(kArgWaves * kWave), 0, st, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tree_walk_kernel, dim3((unsigned)a.batch), dim3(kWave), 0, st, P);
  return hipGetLastError();
}

}  // namespace specv
