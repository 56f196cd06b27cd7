// kv_commit.hip -- commit of an accepted path's K/V and the committed-length pointer on
// gfx950 ("KV Cache 优化（四）：Speculative Decoding 投机解码" §6: reserved slots, one
// committed-length pointer with the same boundary in every layer, no copy of whole blocks;
// "10.6 投机解码" §10.6.3: after a rejection the cache length is cut back).
//
//  1. kv_copy_kernel    -- one thread per 16-byte chunk of one head's K or V row in one
//     layer of one sequence; for j = 1..D in increasing order it moves the chunk of slot
//     base + path[j-1] to slot base + j. Consecutive threads cover consecutive chunks of a
//     slot (2 KiB contiguous for 8 heads x 128 bf16), so each wave moves contiguous memory.
//     A thread handles its own chunk sequentially in j, which reproduces in-order copying
//     for any path (for a tree path, path[j-1] >= j, so no source is overwritten first).
//  2. kv_pointer_kernel -- one thread per sequence: committed_len += lead_slots + D, or
//     SPEC_FLAG_SLOT_OOB. It runs after every copy has read committed_len.
#include "spec_device.h"
#include "specv_internal.h"

namespace specv {
namespace {

constexpr int kMaxLayers = 128;
constexpr int kThreads = 256;

struct KvParams {
  uint16_t* k[kMaxLayers];
  uint16_t* v[kMaxLayers];
  const int32_t* path;
  const int32_t* plen;
  int32_t* committed;
  int32_t* flags;
  int64_t seq_stride, slot_stride, head_stride;
  int32_t B, NL, H, chunks, cap, lead, max_depth;
};

// Same predicate in both kernels: every slot the commit touches lies in [0, cap).
__device__ __forceinline__ bool seq_valid(const KvParams& P, int b, int& L, int& D) {
  L = P.committed[b];
  D = P.plen[b];
  if (D < 0 || D > P.max_depth) return false;
  const int base = L + P.lead - 1;
  if (base < -1 || base + D >= P.cap) return false;
  for (int j = 0; j < D; ++j) {
    const int node = P.path[(size_t)b * P.max_depth + j];
    if (node < 1 || base + node >= P.cap) return false;
  }
  return true;
}

__global__ __launch_bounds__(kThreads) void kv_copy_kernel(KvParams P, int64_t total) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  int64_t r = t;
  const int ch = (int)(r % P.chunks);
  r /= P.chunks;
  const int h = (int)(r % P.H);
  r /= P.H;
  const int kv = (int)(r % 2);
  r /= 2;
  const int l = (int)(r % P.NL);
  const int b = (int)(r / P.NL);
  int L, D;
  if (!seq_valid(P, b, L, D) || D == 0) return;
  const int base = L + P.lead - 1;
  uint16_t* cache = kv ? P.v[l] : P.k[l];
  uint16_t* head = cache + (int64_t)b * P.seq_stride + (int64_t)h * P.head_stride + ch * 8;
  const int32_t* path = P.path + (size_t)b * P.max_depth;
  for (int j = 1; j <= D; ++j) {
    const int src = base + path[j - 1], dst = base + j;
    if (src == dst) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(head + (int64_t)src * P.slot_stride);
    *reinterpret_cast<uint4*>(head + (int64_t)dst * P.slot_stride) = val;
  }
}

__global__ __launch_bounds__(kThreads) void kv_pointer_kernel(KvParams P) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= P.B) return;
  int L, D;
  if (seq_valid(P, b, L, D)) {
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
  const int64_t total = (int64_t)a.batch * a.num_layers * 2 * a.num_kv_heads * P.chunks;
  if (total > 0) {
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(kv_copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, P, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kv_pointer_kernel, dim3((unsigned)((a.batch + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace specv
