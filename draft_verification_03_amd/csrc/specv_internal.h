// specv_internal.h -- host-side interface between the C ABI layer (spec_abi.cpp) and the
// kernel launchers (*.hip). Not installed; the public interface is include/spec_verify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace specv {

// Longest nucleus list a row record keeps for the resolve step; longer nuclei are re-read
// from the logits instead.
constexpr int kNucMax = 256;

// Per-(sequence, position) record the row pass leaves for the resolve step. Index 0 is the
// target row (p), index 1 the draft row (q).
struct RowRec {
  float m[2];      // largest logit of the row
  float z[2];      // normaliser of the kept set, in units of exp((m - m)/T) = 1
  float t[2];      // nucleus threshold logit (-inf: every token kept)
  float pd, qd;    // p_k(d_k), q_k(d_k)
  int32_t argmax;  // target-row argmax (greedy rows)
  int32_t accept;  // 1 accepted, 0 rejected
  int32_t flags;   // SPEC_FLAG_* seen by this item
  int32_t nuc[2];  // entries in the nucleus list (-1: list not kept, re-read the row)
  int32_t valid;   // 1 once the item ran
  int32_t pad[2];
};
static_assert(sizeof(RowRec) == 64, "RowRec must stay 64 bytes");

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
