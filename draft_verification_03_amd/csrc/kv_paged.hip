// kv_paged.hip -- paged KV commit, pointer update and block release on gfx950 ("10.6 投机解码"
// §10.6.3: after a rejection the cache length is cut back and a paged cache releases the
// blocks it no longer needs; "KV Cache 优化（四）：Speculative Decoding 投机解码" §6: one
// committed-length pointer, the same boundary in every layer).
//
//  1. paged_copy_kernel    -- one thread per 16-byte chunk of one head's K or V row in one
//     layer of one sequence; for j = 1..D in increasing order it moves the chunk of logical
//     slot base + path[j-1] to logical slot base + j, each slot found through the sequence's
//     block table. A thread handles its own chunk in j order, which reproduces in-order
//     copying (a tree path has path[j-1] >= j, so no source is overwritten first).
//  2. paged_release_kernel -- one 1024-thread workgroup over tiles of whole table rows: one
//     thread per sequence checks it (the same predicate), writes its new committed length and
//     notes its first block past that length; then the tile's table entries, taken in
//     row-major order (8 consecutive per thread), are flagged and scanned, and a released
//     entry's place in the free list is the number of released entries before it -- so the
//     ids land in (sequence, logical block) order whatever the launch timing. It runs after
//     every copy has read the tables.
#include "spec_device.h"
#include "specv_internal.h"

namespace specv {
namespace {

constexpr int kMaxLayers = 128;
constexpr int kThreads = 256;
constexpr int kRelThreads = 1024;
constexpr int kRelWaves = kRelThreads / kWave;
constexpr int kRun = 8;           // table entries per thread per chunk
constexpr int kRelEntries = kRelThreads * kRun;  // table entries per tile (whole rows)
constexpr int kRelRows = kRelEntries;            // rows per tile at most

struct PagedParams {
  uint16_t* k[kMaxLayers];
  uint16_t* v[kMaxLayers];
  int32_t* bt;
  const int32_t* path;
  const int32_t* plen;
  int32_t* committed;
  int32_t* free_list;
  int32_t* free_count;
  int32_t* flags;
  int64_t block_stride, slot_stride, head_stride;
  int32_t B, NL, H, chunks, bs, max_blocks, num_blocks, free_cap, lead, max_depth;
};

// A slot's physical block, or -1 when the slot lies outside the table or its block is not a
// valid block id.
__device__ __forceinline__ int block_of(const PagedParams& P, const int32_t* bt, int slot) {
  if (slot < 0 || slot >= P.max_blocks * P.bs) return -1;
  const int pb = bt[slot / P.bs];
  return (pb >= 0 && pb < P.num_blocks) ? pb : -1;
}

// Same predicate in both kernels: every slot a copy touches is mapped, every path node is a
// node, and the new committed length fits the table.
__device__ __forceinline__ bool seq_valid(const PagedParams& P, int b, int& L, int& D) {
  L = P.committed[b];
  D = P.plen[b];
  if (D < 0 || D > P.max_depth) return false;
  const int base = L + P.lead - 1;
  if (base < -1) return false;
  const int64_t new_len = (int64_t)L + P.lead + D;
  if ((new_len + P.bs - 1) / P.bs > P.max_blocks) return false;
  const int32_t* bt = P.bt + (size_t)b * P.max_blocks;
  const int32_t* path = P.path + (size_t)b * P.max_depth;
  for (int j = 1; j <= D; ++j) {
    const int node = path[j - 1];
    if (node < 1) return false;
    const int src = base + node, dst = base + j;
    if (src == dst) continue;
    if (block_of(P, bt, src) < 0 || block_of(P, bt, dst) < 0) return false;
  }
  return true;
}

__global__ __launch_bounds__(kThreads) void paged_copy_kernel(PagedParams P, int64_t total) {
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
  const int32_t* bt = P.bt + (size_t)b * P.max_blocks;
  const int32_t* path = P.path + (size_t)b * P.max_depth;
  uint16_t* head = (kv ? P.v[l] : P.k[l]) + (int64_t)h * P.head_stride + ch * 8;
  auto at = [&](int slot) {
    return head + (int64_t)block_of(P, bt, slot) * P.block_stride +
           (int64_t)(slot % P.bs) * P.slot_stride;
  };
  for (int j = 1; j <= D; ++j) {
    const int src = base + path[j - 1], dst = base + j;
    if (src == dst) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(at(src));
    *reinterpret_cast<uint4*>(at(dst)) = val;
  }
}

__global__ __launch_bounds__(kRelThreads) void paged_release_kernel(PagedParams P) {
  __shared__ int s_need[kRelRows];  // first released logical block of each row (-1: invalid)
  __shared__ int s_wave[kRelWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int fc0 = min(max(*P.free_count, 0), P.free_cap);
  const int mb = P.max_blocks;
  const int rows = max(1, min(kRelRows, kRelEntries / mb));  // whole rows per tile
  int carry = 0;  // blocks released before this chunk (uniform)
  for (int b0 = 0; b0 < P.B; b0 += rows) {
    const int nr = min(rows, P.B - b0);
    // one thread per sequence: validity, new length and the first block past it
    for (int i = tid; i < nr; i += kRelThreads) {
      const int b = b0 + i;
      int L, D;
      const bool ok = seq_valid(P, b, L, D);
      s_need[i] = ok ? (int)(((int64_t)L + P.lead + D + P.bs - 1) / P.bs) : -1;
      if (ok) {
        P.committed[b] = L + P.lead + D;  // every read of committed[b] is above
      } else if (P.flags) {
        P.flags[b] |= SPEC_FLAG_SLOT_OOB;
      }
    }
    __syncthreads();
    // the tile's table entries in row-major order, kRun consecutive per thread: the free
    // list position of a released entry is the count of released entries before it
    const int64_t e0 = (int64_t)b0 * mb, ne = (int64_t)nr * mb;
    for (int64_t c0 = 0; c0 < ne; c0 += (int64_t)kRelThreads * kRun) {
      int pb[kRun];
      int cnt = 0;
#pragma unroll
      for (int r = 0; r < kRun; ++r) {
        const int64_t e = c0 + (int64_t)tid * kRun + r;  // entry of the tile
        pb[r] = -1;
        if (e < ne) {
          const int i = (int)(e / mb), lb = (int)(e - (int64_t)i * mb);
          const int need = s_need[i];
          const int v = P.bt[e0 + e];
          if (need >= 0 && lb >= need && v >= 0) pb[r] = v;
        }
        cnt += pb[r] >= 0;
      }
      const int incl = wave_incl_scan_dpp(cnt);
      if (lane == kWave - 1) s_wave[wave] = incl;
      __syncthreads();
      int before = 0, total = 0;
      for (int w = 0; w < kRelWaves; ++w) {
        const int tw = s_wave[w];
        before += w < wave ? tw : 0;
        total += tw;
      }
      int at = fc0 + carry + before + incl - cnt;
#pragma unroll
      for (int r = 0; r < kRun; ++r) {
        if (pb[r] >= 0) {
          if (at < P.free_cap) P.free_list[at] = pb[r];
          ++at;
          P.bt[e0 + c0 + (int64_t)tid * kRun + r] = -1;
        }
      }
      carry += total;
      __syncthreads();  // s_wave is read by every thread before the next chunk writes it
    }
  }
  if (tid == 0) *P.free_count = min(fc0 + carry, P.free_cap);
}

}  // namespace

hipError_t launch_kv_paged(const spec_paged_kv_args& a, hipStream_t st) {
  PagedParams P;
  for (int l = 0; l < kMaxLayers; ++l) {
    P.k[l] = l < a.num_layers ? a.k_cache[l] : nullptr;
    P.v[l] = l < a.num_layers ? a.v_cache[l] : nullptr;
  }
  P.bt = a.block_table;
  P.path = a.path_nodes;
  P.plen = a.path_len;
  P.committed = a.committed_len;
  P.free_list = a.free_list;
  P.free_count = a.free_count;
  P.flags = a.seq_flags;
  P.block_stride = a.block_stride;
  P.slot_stride = a.slot_stride;
  P.head_stride = a.head_stride;
  P.B = a.batch;
  P.NL = a.num_layers;
  P.H = a.num_kv_heads;
  P.chunks = a.head_dim / 8;
  P.bs = a.block_size;
  P.max_blocks = a.max_blocks;
  P.num_blocks = a.num_blocks;
  P.free_cap = a.free_capacity;
  P.lead = a.lead_slots;
  P.max_depth = a.max_depth;
  const int64_t total = (int64_t)a.batch * a.num_layers * 2 * a.num_kv_heads * P.chunks;
  if (total > 0) {
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(paged_copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, P,
                       total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(paged_release_kernel, dim3(1), dim3(kRelThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace specv
