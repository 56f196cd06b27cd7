// kv_commit.hip -- commit of an accepted path's K/V and the committed-length pointer on
// gfx950 ("KV Cache 优化（四）：Speculative Decoding 投机解码" §6: reserved slots, one
// committed-length pointer with the same boundary in every layer, no copy of whole blocks;
// "10.6 投机解码" §10.6.3: after a rejection the cache length is cut back).
//
//  1. kv_copy_kernel -- S 256-thread workgroups per sequence (workgroup b * S + s), each
//     over a share of the sequence's 16-byte chunks (one chunk = 8 elements of one head's K
//     or V row in one layer; consecutive threads take consecutive chunks of a slot, so a wave
//     moves contiguous memory). A workgroup reads the committed length, path length and path
//     once into LDS and checks them (every slot the commit touches lies in [0, capacity)).
//     For its chunk a thread moves slot base + path[j-1] to slot base + j for j = 1..D in
//     increasing order -- in-order copying for any path. The steps go kGroup at a time: when
//     no source of a group is the destination of an earlier step of that group (always so for
//     a tree path, where path[j-1] >= j), the group's loads, for kBatch chunks at once, are
//     all issued before its stores; otherwise the group runs one load-store pair at a time.
//  2. kv_pointer_kernel -- one thread per sequence, after every copy has read the committed
//     length: committed_len = L + lead_slots + D, or flag SLOT_OOB (the same check).
#include "spec_device.h"
#include "specv_internal.h"

namespace specv {
namespace {

constexpr int kMaxLayers = 128;
constexpr int kThreads = 256;
constexpr int kMaxDepth = 64;
constexpr int kGroup = 4;  // path steps whose loads are in flight together
constexpr int kBatch = 4;  // chunks per thread whose loads are in flight together
constexpr int kChunksPerWg = kThreads * kBatch;
// 16-byte chunk as a native vector: an array of them stays in registers
typedef uint32_t chunk16 __attribute__((ext_vector_type(4)));

struct KvParams {
  uint16_t* k[kMaxLayers];
  uint16_t* v[kMaxLayers];
  const int32_t* path;
  const int32_t* plen;
  int32_t* committed;
  int32_t* flags;
  int64_t seq_stride, slot_stride, head_stride;
  int32_t B, NL, H, chunks, cap, lead, max_depth;
  int32_t split;  // copy workgroups per sequence
};

// The check of both kernels: every slot the commit touches lies in [0, capacity). path holds
// the sequence's max_depth entries (only the first D are read).
__device__ __forceinline__ bool seq_valid(const KvParams& P, int L, int D, const int32_t* path) {
  const int64_t base = (int64_t)L + P.lead - 1;
  bool ok = D >= 0 && D <= P.max_depth && base >= -1 && base + D < P.cap;
  for (int j = 0; ok && j < D; ++j) ok = path[j] >= 1 && base + path[j] < P.cap;
  return ok;
}

__global__ __launch_bounds__(kThreads) void kv_copy_kernel(KvParams P) {
  __shared__ int32_t s_path[kMaxDepth];
  __shared__ int s_L, s_D, s_ok;
  __shared__ uint8_t s_together[kMaxDepth / kGroup];
  const int b = blockIdx.x / P.split, part = blockIdx.x % P.split, tid = threadIdx.x;
  const int nch = P.NL * 2 * P.H * P.chunks;
  const int c0 = part * kChunksPerWg + tid;
  // chunk addresses, computed before the barrier so that the layer pointers load while the
  // sequence is read: a slot past the sequence's chunks repeats chunk c0 and stores nothing,
  // and a thread past them all (c0 >= nch) takes the last chunk's address and never uses it
  uint16_t* head[kBatch];
  bool has[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    int c = c0 + u * kThreads;
    has[u] = c < nch;
    if (!has[u]) c = min(c0, nch - 1);
    const int ch = c % P.chunks;
    c /= P.chunks;
    const int h = c % P.H;
    c /= P.H;
    uint16_t* cache = (c & 1) ? P.v[c >> 1] : P.k[c >> 1];
    head[u] = cache + (int64_t)b * P.seq_stride + (int64_t)h * P.head_stride + ch * 8;
  }
  if (tid == 0) {
    s_L = P.committed[b];
    s_D = P.plen[b];
  }
  if (tid < P.max_depth) s_path[tid] = P.path[(size_t)b * P.max_depth + tid];
  __syncthreads();
  if (tid == 0) {
    const int D = s_D;
    const bool ok = seq_valid(P, s_L, D, s_path);
    s_ok = ok;
    for (int j0 = 1; ok && j0 <= D; j0 += kGroup) {
      const int n = min(kGroup, D - j0 + 1);
      bool together = true;
      for (int g = 1; g < n; ++g)
        for (int e = 0; e < g; ++e) together &= s_path[j0 + g - 1] != j0 + e;
      s_together[(j0 - 1) / kGroup] = together;
    }
  }
  __syncthreads();
  const int D = s_D;
  if (!s_ok || D == 0) return;
  const int base = s_L + P.lead - 1;
  if (c0 >= nch) return;
  for (int j0 = 1; j0 <= D; j0 += kGroup) {
    const int n = min(kGroup, D - j0 + 1);
    int64_t so[kGroup], dof[kGroup];
    bool mv[kGroup];
    int first = -1;  // the group's first step that moves a slot
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int src = g < n ? base + s_path[j0 + g - 1] : 0, dst = base + j0 + g;
      mv[g] = g < n && src != dst;
      if (mv[g] && first < 0) first = g;
      so[g] = (int64_t)src * P.slot_stride;
      dof[g] = (int64_t)dst * P.slot_stride;
    }
    if (first < 0) continue;  // nothing moves in this group
    if (s_together[(j0 - 1) / kGroup]) {
      // every load is issued (a step that moves nothing re-reads the first moving step's
      // source), then the stores of the moving steps
      int64_t ld[kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) ld[g] = mv[g] ? so[g] : so[first];
      chunk16 val[kBatch][kGroup];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
#pragma unroll
        for (int g = 0; g < kGroup; ++g)
          val[u][g] = *reinterpret_cast<const chunk16*>(head[u] + ld[g]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
#pragma unroll
        for (int g = 0; g < kGroup; ++g)
          if (has[u] && mv[g]) *reinterpret_cast<chunk16*>(head[u] + dof[g]) = val[u][g];
    } else {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (!has[u]) continue;
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {  // mv[g] is false past the group's n steps
          if (!mv[g]) continue;
          const chunk16 val = *reinterpret_cast<const chunk16*>(head[u] + so[g]);
          *reinterpret_cast<chunk16*>(head[u] + dof[g]) = val;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void kv_pointer_kernel(KvParams P) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= P.B) return;
  const int L = P.committed[b], D = P.plen[b];
  // the path's first kGroup entries load together with L and D (a path row has max_depth)
  const int32_t* row = P.path + (size_t)b * P.max_depth;
  int32_t head[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) head[j] = j < P.max_depth ? row[j] : 0;
  const int64_t base = (int64_t)L + P.lead - 1;
  bool ok = D >= 0 && D <= P.max_depth && base >= -1 && base + D < P.cap;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) ok = ok && (j >= D || (head[j] >= 1 && base + head[j] < P.cap));
  if (ok && D > kGroup) ok = seq_valid(P, L, D, row);
  if (ok) {
    P.committed[b] = L + P.lead + D;
  } else if (P.flags) {
    P.flags[b] |= SPEC_FLAG_SLOT_OOB;
  }
}

}  // namespace

hipError_t launch_kv(const spec_kv_args& a, hipStream_t st) {
  KvParams P;
  for (int l = 0; l < kMaxLayers; ++l) {
    P.k[l] = l < a.num_layers ? a.k_cache[l] : nullptr;
    P.v[l] = l < a.num_layers ? a.v_cache[l] : nullptr;
  }
  P.path = a.path_nodes;
  P.plen = a.path_len;
  P.committed = a.committed_len;
  P.flags = a.seq_flags;
  P.seq_stride = a.seq_stride;
  P.slot_stride = a.slot_stride;
  P.head_stride = a.head_stride;
  P.B = a.batch;
  P.NL = a.num_layers;
  P.H = a.num_kv_heads;
  P.chunks = a.head_dim / 8;
  P.cap = a.slot_capacity;
  P.lead = a.lead_slots;
  P.max_depth = a.max_depth;
  if (a.batch <= 0) return hipSuccess;
  const int nch = a.num_layers * 2 * a.num_kv_heads * P.chunks;  // bounded by the host check
  P.split = (nch + kChunksPerWg - 1) / kChunksPerWg;
  hipLaunchKernelGGL(kv_copy_kernel, dim3((unsigned)((int64_t)a.batch * P.split)), dim3(kThreads),
                     0, st, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_pointer_kernel, dim3((unsigned)((a.batch + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace specv
