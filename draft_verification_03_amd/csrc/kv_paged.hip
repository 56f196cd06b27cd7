// kv_paged.hip -- paged KV commit, pointer update and block release on gfx950 ("10.6 投机解码"
// §10.6.3: after a rejection the cache length is cut back and a paged cache releases the
// blocks it no longer needs; "KV Cache 优化（四）：Speculative Decoding 投机解码" §6: one
// committed-length pointer, the same boundary in every layer).
//
//  1. paged_copy_kernel    -- S 256-thread workgroups per sequence (workgroup b * S + s), each
//     over a share of the sequence's 16-byte chunks (8 elements of one head's K or V row in
//     one layer). A workgroup reads the sequence's length, path length and path once; thread
//     j-1 checks step j and translates its source and destination slots through the block
//     table into physical offsets in LDS, and the threads check the table entries the
//     release would free. For its chunk a thread then moves slot base +
//     path[j-1] to slot base + j for j = 1..D in increasing order -- in-order copying for
//     any path -- kGroup steps at a time: when no source of a group is the destination of an
//     earlier step of the group (always so for a tree path, path[j-1] >= j), the group's
//     loads, for kBatch chunks at once, are issued before its stores; otherwise one
//     load-store pair at a time.
//  2. paged_release_kernel -- one 1024-thread workgroup over tiles of whole table rows. Each
//     tile first issues all of its global reads together -- the rows' lengths, their path
//     rows and their table entries, kept in LDS -- and then decides from LDS alone: the
//     commit predicate (one thread per path step, one per table entry for the ids of the
//     blocks that would be freed), the new committed lengths, then the tile's entries taken
//     in row-major order (8 consecutive per thread, read and written back as two 16-byte
//     vectors where aligned) are flagged and scanned, and a released entry's place in the
//     free list is the number of released entries before it -- so the ids land in (sequence,
//     logical block) order whatever the launch timing; they are gathered in LDS and written
//     to the free list in one coalesced pass. An entry whose place falls at or past the free
//     list's capacity stays in its table (FREE_FULL). It runs after every copy has read the
//     tables.
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
constexpr int kRelThreads = 1024;
constexpr int kRelWaves = kRelThreads / kWave;
constexpr int kRun = 8;           // table entries per thread per chunk
constexpr int kRelEntries = kRelThreads * kRun;  // table entries per tile (whole rows)
constexpr int kRelRows = kRelThreads;            // rows per tile at most (one per thread)
constexpr int kRelPath = 4 * kRelThreads;        // path entries per tile at most

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
  int32_t split;  // copy workgroups per sequence
};

// The commit predicate, checked in both kernels: with L = committed_len, D = path_len and
// base = L + lead - 1, a sequence is committed when 0 <= D <= max_depth, base >= -1, the new
// length L + lead + D fits max_blocks blocks, every path node is >= 1, for every step
// j = 1..D that moves a slot (base + path[j-1] != base + j) both slots lie inside the table
// in blocks with valid ids (0 <= id < num_blocks), and no table entry at or past the first
// block beyond the new length (the blocks the release frees) is >= num_blocks. Otherwise it
// is flagged SLOT_OOB and left untouched.

__global__ __launch_bounds__(kThreads) void paged_copy_kernel(PagedParams P) {
  __shared__ int64_t s_so[kMaxDepth], s_do[kMaxDepth];  // physical element offsets per step
  __shared__ int32_t s_path[kMaxDepth];
  __shared__ uint8_t s_mv[kMaxDepth];
  __shared__ int s_bad;
  const int b = blockIdx.x / P.split, part = blockIdx.x % P.split, tid = threadIdx.x;
  const int nch = P.NL * 2 * P.H * P.chunks;
  const int c0 = part * kChunksPerWg + tid;
  // chunk addresses within a slot, computed before the barrier so that the layer pointers
  // load while the sequence is read: a slot past the sequence's chunks repeats chunk c0 and
  // stores nothing, and a thread past them all (c0 >= nch) never uses its addresses
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
    head[u] = cache + (int64_t)h * P.head_stride + ch * 8;
  }
  // the sequence's length, path length and path step tid + 1 load together (the step from
  // a clamped index, used only below D), before the barrier that clears s_bad
  const int L = P.committed[b], D = P.plen[b];
  const int node = P.path[(size_t)b * P.max_depth + min(tid, P.max_depth - 1)];
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // the commit predicate, step j by thread j - 1
  const int64_t base = (int64_t)L + P.lead - 1;
  const int64_t slots = (int64_t)P.max_blocks * P.bs;
  const bool head_ok = D >= 0 && D <= P.max_depth && base >= -1 &&
                       ((int64_t)L + P.lead + D + P.bs - 1) / P.bs <= P.max_blocks;
  if (head_ok && tid < D) {
    const int32_t* bt = P.bt + (size_t)b * P.max_blocks;
    const int64_t src = base + node, dst = base + tid + 1;
    bool ok = node >= 1;
    bool mv = false;
    if (ok && src != dst) {
      const int pbs = src < slots ? bt[src / P.bs] : -1;
      const int pbd = dst < slots ? bt[dst / P.bs] : -1;
      ok = pbs >= 0 && pbs < P.num_blocks && pbd >= 0 && pbd < P.num_blocks;
      mv = ok;
      s_so[tid] = (int64_t)pbs * P.block_stride + (src % P.bs) * P.slot_stride;
      s_do[tid] = (int64_t)pbd * P.block_stride + (dst % P.bs) * P.slot_stride;
    }
    s_path[tid] = node;
    s_mv[tid] = mv;
    if (!ok) atomicOr(&s_bad, 1);
  }
  if (head_ok) {  // the blocks the release would free must hold block ids
    const int need = (int)(((int64_t)L + P.lead + D + P.bs - 1) / P.bs);
    const int32_t* bt = P.bt + (size_t)b * P.max_blocks;
    for (int lb = need + tid; lb < P.max_blocks; lb += kThreads)
      if (bt[lb] >= P.num_blocks) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (!head_ok || s_bad || D == 0 || c0 >= nch) return;
  for (int j0 = 1; j0 <= D; j0 += kGroup) {
    const int n = min(kGroup, D - j0 + 1);
    int64_t so[kGroup], dof[kGroup];
    bool mv[kGroup];
    int first = -1;  // the group's first step that moves a slot
    bool together = true;  // no source of the group is an earlier step's destination
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      mv[g] = g < n && s_mv[j0 + g - 1];
      if (mv[g] && first < 0) first = g;
      so[g] = g < n ? s_so[j0 + g - 1] : 0;
      dof[g] = g < n ? s_do[j0 + g - 1] : 0;
#pragma unroll
      for (int e = 0; e < g; ++e) together &= g >= n || s_path[j0 + g - 1] != j0 + e;
    }
    if (first < 0) continue;  // nothing moves in this group
    if (together) {
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

// kRun consecutive table entries from entry g (entries at or past gend read as -1): two
// 16-byte loads when the run lies before gend and starts 16-byte aligned (then a wave's loads
// touch half the cache lines and issue a quarter of the instructions of 4-byte loads), else
// kRun 4-byte loads.
__device__ __forceinline__ void load_run(const int32_t* bt, int64_t g, int64_t gend,
                                         int v[kRun]) {
  static_assert(kRun == 8, "a run is two 16-byte vectors");
  if (g + kRun <= gend && (reinterpret_cast<uintptr_t>(bt + g) & 15) == 0) {
    const int4 a = *reinterpret_cast<const int4*>(bt + g);
    const int4 c = *reinterpret_cast<const int4*>(bt + g + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
    v[4] = c.x, v[5] = c.y, v[6] = c.z, v[7] = c.w;
  } else {
#pragma unroll
    for (int r = 0; r < kRun; ++r) v[r] = g + r < gend ? bt[g + r] : -1;
  }
}

// Writes back a run whose entries rel[r] were released (set to -1 in v): as two 16-byte
// stores when the run lies before gend and is 16-byte aligned (the other entries keep the
// values just read: nothing else writes the table during the release), else the released
// entries alone.
__device__ __forceinline__ void store_run(int32_t* bt, int64_t g, int64_t gend,
                                          const int v[kRun], const bool rel[kRun]) {
  if (g + kRun <= gend && (reinterpret_cast<uintptr_t>(bt + g) & 15) == 0) {
    *reinterpret_cast<int4*>(bt + g) = make_int4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<int4*>(bt + g + 4) = make_int4(v[4], v[5], v[6], v[7]);
  } else {
#pragma unroll
    for (int r = 0; r < kRun; ++r)
      if (rel[r]) bt[g + r] = -1;
  }
}

__global__ __launch_bounds__(kRelThreads) void paged_release_kernel(PagedParams P) {
  // the tile's table entries, row-major; in the release step, the chunk's released ids in
  // free-list order
  __shared__ __align__(16) int32_t s_bt[kRelEntries];
  __shared__ int32_t s_path[kRelPath];    // the tile's path rows
  __shared__ int s_need[kRelRows];        // first released logical block of a row (-1: invalid)
  __shared__ int s_L[kRelRows], s_D[kRelRows];
  __shared__ int s_wave[kRelWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int fc0 = min(max(*P.free_count, 0), P.free_cap);
  const int mb = P.max_blocks, md = P.max_depth;
  const bool in_lds = mb <= kRelEntries;  // a whole table row fits the tile's LDS
  const int rows = max(1, min(min(kRelRows, kRelEntries / mb), kRelPath / md));
  int carry = 0;  // blocks released before this tile (uniform)
  for (int b0 = 0; b0 < P.B; b0 += rows) {
    const int nr = min(rows, P.B - b0);
    const int64_t e0 = (int64_t)b0 * mb, ne = (int64_t)nr * mb;
    // 1. every global read of the tile at once -- lengths, path rows, table entries -- as
    //    unconditional loads from clamped indexes (a value past the tile is dropped), all
    //    issued before the first one is used, so that the phase costs one memory round trip;
    //    then the values go to LDS (and kRun consecutive entries per thread stay in registers
    //    for the scan)
    const int li = min(tid, nr - 1);
    const int L0 = P.committed[b0 + li], D0 = P.plen[b0 + li];
    int p_reg[kRelPath / kRelThreads];
#pragma unroll
    for (int k = 0; k < kRelPath / kRelThreads; ++k)
      p_reg[k] = P.path[(size_t)b0 * md + min(tid + k * kRelThreads, nr * md - 1)];
    int v_reg[kRun];  // the tile's first chunk, entries past the tile read as -1
    load_run(P.bt, e0 + (int64_t)tid * kRun, e0 + ne, v_reg);
    if (tid < nr) {
      s_L[tid] = L0;
      s_D[tid] = D0;
      const int64_t base = (int64_t)L0 + P.lead - 1;
      const int64_t need = ((int64_t)L0 + P.lead + D0 + P.bs - 1) / P.bs;
      const bool ok = D0 >= 0 && D0 <= md && base >= -1 && need <= mb;
      s_need[tid] = ok ? (int)need : -1;
    }
#pragma unroll
    for (int k = 0; k < kRelPath / kRelThreads; ++k)
      if (tid + k * kRelThreads < nr * md) s_path[tid + k * kRelThreads] = p_reg[k];
    if (in_lds) {
      const int64_t e = (int64_t)tid * kRun;
      if (e + kRun <= ne) {
        *reinterpret_cast<int4*>(&s_bt[e]) = make_int4(v_reg[0], v_reg[1], v_reg[2], v_reg[3]);
        *reinterpret_cast<int4*>(&s_bt[e + 4]) = make_int4(v_reg[4], v_reg[5], v_reg[6], v_reg[7]);
      } else {
#pragma unroll
        for (int r = 0; r < kRun; ++r)
          if (e + r < ne) s_bt[e + r] = v_reg[r];
      }
    }
    __syncthreads();
    // 2. the commit predicate from LDS: path steps (slots mapped to valid blocks), and the
    //    entries the release would free (valid ids)
    for (int q = tid; q < nr * md; q += kRelThreads) {
      const int i = q / md, j = q - i * md;
      const int D = s_D[i];
      if (s_need[i] < 0 || j >= D) continue;
      const int node = s_path[q];
      const int64_t base = (int64_t)s_L[i] + P.lead - 1;
      const int64_t src = base + node, dst = base + j + 1;
      const int64_t slots = (int64_t)mb * P.bs;
      bool ok = node >= 1;
      if (ok && src != dst) {
        const int64_t row = (int64_t)(b0 + i) * mb;
        // the LDS tile and the global table in branches of their own: one load that picked
        // either per thread would be a generic flat load
        int pbs = -1, pbd = -1;
        const bool sv = src >= 0 && src < slots, dv = dst >= 0 && dst < slots;
        if (in_lds) {
          if (sv) pbs = s_bt[i * mb + src / P.bs];
          if (dv) pbd = s_bt[i * mb + dst / P.bs];
        } else {
          if (sv) pbs = P.bt[row + src / P.bs];
          if (dv) pbd = P.bt[row + dst / P.bs];
        }
        ok = pbs >= 0 && pbs < P.num_blocks && pbd >= 0 && pbd < P.num_blocks;
      }
      if (!ok) atomicMin(&s_need[i], -1);
    }
    // (a tile holds at most max(kRelEntries, max_blocks) entries: indexes within it fit an
    // int; a thread's row and block follow its first entry's, one division per chunk)
    const int ne32 = (int)ne;
    for (int c0 = 0; c0 < ne32; c0 += kRelThreads * kRun) {
      const int ef = c0 + tid * kRun;
      int i = ef / mb, lb = ef - i * mb;
      int vr[kRun];
      if (c0 == 0) {
#pragma unroll
        for (int r = 0; r < kRun; ++r) vr[r] = v_reg[r];
      } else {
        load_run(P.bt, e0 + ef, e0 + ne, vr);
      }
#pragma unroll
      for (int r = 0; r < kRun; ++r) {
        const int e = ef + r;
        if (e < ne32) {
          const int need = s_need[i];
          if (need >= 0 && lb >= need && vr[r] >= P.num_blocks) atomicMin(&s_need[i], -1);
        }
        if (++lb == mb) {
          lb = 0;
          ++i;
        }
      }
    }
    __syncthreads();
    // 3. the tile's entries in row-major order, kRun consecutive per thread: a released
    //    entry's free-list position is the count of released entries before it; one that
    //    lands at or past the capacity stays in the table and flags its sequence FREE_FULL.
    //    The placed ids go to LDS at their positions, then to the free list in one coalesced
    //    pass; a thread writes its run back with the placed entries set to -1.
    for (int c0 = 0; c0 < ne32; c0 += kRelThreads * kRun) {
      const int ef = c0 + tid * kRun;
      const int i0 = ef / mb;
      int vr[kRun], pb[kRun], pi[kRun];
      if (c0 == 0) {
#pragma unroll
        for (int r = 0; r < kRun; ++r) vr[r] = v_reg[r];
      } else {
        load_run(P.bt, e0 + ef, e0 + ne, vr);
      }
      int cnt = 0;
      {
        int i = i0, lb = ef - i0 * mb;
#pragma unroll
        for (int r = 0; r < kRun; ++r) {
          const int e = ef + r;
          pb[r] = -1;
          pi[r] = i;
          if (e < ne32) {
            const int need = s_need[i];
            if (need >= 0 && lb >= need && vr[r] >= 0) pb[r] = vr[r];
          }
          cnt += pb[r] >= 0;
          if (++lb == mb) {
            lb = 0;
            ++i;
          }
        }
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
      const int room = max(P.free_cap - (fc0 + carry), 0);  // free-list entries left
      int k = before + incl - cnt;  // the chunk's count of released entries before this run
      bool rel[kRun], any = false;
#pragma unroll
      for (int r = 0; r < kRun; ++r) {
        rel[r] = false;
        if (pb[r] >= 0) {
          if (k < room) {
            s_bt[k] = pb[r];
            vr[r] = -1;
            rel[r] = any = true;
          } else if (P.flags) {
            atomicOr(&P.flags[b0 + pi[r]], SPEC_FLAG_FREE_FULL);
          }
          ++k;
        }
      }
      __syncthreads();  // the chunk's placed ids are in LDS
      // the global stores last: a register that a store reads is not reused before the
      // store completes, so stores issued early would hold up the work after them
      const int placed = min(total, room);
      for (int j = tid; j < placed; j += kRelThreads) P.free_list[fc0 + carry + j] = s_bt[j];
      if (any) store_run(P.bt, e0 + ef, e0 + ne, vr, rel);
      carry += total;
      if (c0 + kRelThreads * kRun < ne32)
        __syncthreads();  // s_wave and the ids are read before the next chunk writes them
    }
    // 4. the new lengths and SLOT_OOB flags
    for (int i = tid; i < nr; i += kRelThreads) {
      if (s_need[i] >= 0) {
        P.committed[b0 + i] = s_L[i] + P.lead + s_D[i];
      } else if (P.flags) {
        P.flags[b0 + i] |= SPEC_FLAG_SLOT_OOB;
      }
    }
    if (b0 + rows < P.B) __syncthreads();  // the tile's LDS is read before the next tile's
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
  if (a.batch > 0) {
    const int nch = a.num_layers * 2 * a.num_kv_heads * P.chunks;  // bounded by the host check
    P.split = (nch + kChunksPerWg - 1) / kChunksPerWg;
    hipLaunchKernelGGL(paged_copy_kernel, dim3((unsigned)((int64_t)a.batch * P.split)),
                       dim3(kThreads), 0, st, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(paged_release_kernel, dim3(1), dim3(kRelThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace specv
