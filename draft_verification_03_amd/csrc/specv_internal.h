// specv_internal.h -- host-side interface between the C ABI layer (spec_abi.cpp) and the
// kernel launchers (*.hip). Not installed; the public interface is include/spec_verify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace specv {

// Longest nucleus list a row statistic keeps for the resolve step; longer nuclei are re-read
// from the logits instead.
constexpr int kNucMax = 256;

// Statistics the row pass leaves for one logits row of a draft position: its target row
// (index 0) or its draft row (index 1). Weights are exp2((l - m) * log2(e) / T), so the
// row's largest logit weighs 1.
struct RowStat {
  float m;         // largest logit of the row (T > 0)
  float z;         // normaliser: summed weight of the kept set
  float t;         // nucleus threshold logit (-inf: every token kept)
  float wd;        // weight of the draft token if kept, else 0 (T = 0: [token == argmax])
  int32_t argmax;  // greedy rows: argmax, lowest id on ties
  int32_t nuc;     // entries in the row's nucleus list (-1: no list, re-read the row)
  int32_t flags;   // SPEC_FLAG_TOPP_SLOW
  int32_t valid;   // 1 once written
};
static_assert(sizeof(RowStat) == 32, "RowStat must stay 32 bytes");

struct NucEntry {
  int32_t idx;  // token id
  float w;      // exp((l - m)/T), unnormalised weight
};

size_t chain_workspace_bytes(int32_t batch, int32_t total_draft_rows, int32_t vocab);
// events: NULL, or two hipEvent_t recorded just before and just after the row-statistics
// kernel (spec_verify_chain_timed).
hipError_t launch_chain(const spec_chain_args& a, void* ws, hipStream_t s,
                        void* const* events = nullptr);

// spec_verify_chain_noalloc's scratch: the library's own device array of this many bytes per
// GPU (chain_noalloc.hip); chain_scratch() returns the current device's address of it.
constexpr size_t kChainScratchBytes = SPEC_CHAIN_SCRATCH_BYTES;
hipError_t chain_scratch(void** ptr);

size_t tree_workspace_bytes(int32_t batch, int32_t rows_per_seq);
hipError_t launch_tree(const spec_tree_args& a, void* ws, hipStream_t s);

hipError_t launch_kv(const spec_kv_args& a, hipStream_t s);
hipError_t launch_kv_paged(const spec_paged_kv_args& a, hipStream_t s);
hipError_t launch_ngram(const spec_ngram_args& a, hipStream_t s);

// Tree drafting: limits and the geometry of one step, derived on the host from the tree
// configuration (top_head, top_k_spec) and the step index.
constexpr int kTreeDraftMaxK = 64;       // children per expanded node
constexpr int kTreeDraftMaxHead = 64;    // expanded nodes per step
constexpr int kTreeDraftMaxNodes = 256;  // nodes per tree
constexpr int kTreeDraftMaxSplits = 16;  // workgroups per draft row

struct TreeDraftPlan {
  int32_t h;              // nodes expanded at this step (draft rows per sequence)
  int32_t kmax;           // largest child count of this step
  int32_t splits;         // workgroups per draft row
  int32_t par_lo, par_hi; // node range the expanded nodes must lie in (step 0: the root)
  int32_t first_new;      // index of the first node this step creates
  int32_t n_new;          // nodes this step creates
  int32_t h_next;         // nodes the next step expands (0 after the last step)
  int32_t row_base_next;  // target row of the next step's first expanded node
  int32_t kk[kTreeDraftMaxHead];    // children of the j-th expanded node
  int32_t koff[kTreeDraftMaxHead];  // its first child, relative to first_new
};

int tree_draft_splits(int32_t rows, int32_t vocab);
size_t tree_draft_record_bytes(int32_t kmax);
hipError_t launch_tree_draft(const spec_tree_draft_args& a, const TreeDraftPlan& p, void* ws,
                             hipStream_t s);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace specv
