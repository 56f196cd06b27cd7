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
hipError_t launch_chain(const spec_chain_args& a, void* ws, hipStream_t s);

size_t tree_workspace_bytes(int32_t batch, int32_t rows_per_seq);
hipError_t launch_tree(const spec_tree_args& a, void* ws, hipStream_t s);

hipError_t launch_kv(const spec_kv_args& a, hipStream_t s);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace specv
