// spec_abi.cpp -- the exported C entry points of libspecv: argument validation (host-visible
// fields only, before any HIP call), workspace sizing, error reporting, and the hand-off to
// the kernel launchers. The contract of every call is documented in include/spec_verify.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "spec_verify.h"
#include "specv_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int32_t kMaxVocab = 1 << 19;  // resolve-pass tile table bound (1024 tiles of 512)
constexpr int32_t kMaxGamma = 64;       // first-rejection scan is one wave64 ballot

int hip_fail(hipError_t e, const char* what) {
  return fail(SPEC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks a tree configuration (top_head, top_k_spec host arrays over `depth` steps). Returns
// SPEC_OK and the node count (root included) in *nodes, or fails with a message.
int check_tree_config(int32_t vocab, int32_t depth, const int32_t* top_head,
                      const int32_t* top_k_spec, int* nodes) {
  if (depth < 1 || depth > 64)
    return fail(SPEC_ERR_INVALID_ARG, "depth must be in [1, 64] (got %d)", depth);
  if (!top_head || !top_k_spec)
    return fail(SPEC_ERR_INVALID_ARG, "top_head and top_k_spec are required host arrays");
  if (top_head[0] != 1)
    return fail(SPEC_ERR_INVALID_ARG, "top_head[0] must be 1: step 0 expands the root");
  int n = 1, layer = 1, ko = 0;
  for (int s = 0; s < depth; ++s) {
    const int h = top_head[s];
    if (h < 1 || h > layer || h > specv::kTreeDraftMaxHead)
      return fail(SPEC_ERR_INVALID_ARG,
                  "top_head[%d] = %d must be in [1, min(%d, %d nodes made at the step before)]",
                  s, h, specv::kTreeDraftMaxHead, layer);
    layer = 0;
    for (int j = 0; j < h; ++j) {
      const int k = top_k_spec[ko + j];
      if (k < 1 || k > specv::kTreeDraftMaxK || k > vocab)
        return fail(SPEC_ERR_INVALID_ARG, "top_k_spec[%d][%d] = %d must be in [1, min(%d, vocab)]",
                    s, j, k, specv::kTreeDraftMaxK);
      layer += k;
    }
    ko += h;
    n += layer;
    if (n > specv::kTreeDraftMaxNodes)
      return fail(SPEC_ERR_INVALID_ARG, "the tree has more than %d nodes",
                  specv::kTreeDraftMaxNodes);
  }
  *nodes = n;
  return SPEC_OK;
}

// Geometry of one step of a checked configuration.
specv::TreeDraftPlan tree_draft_plan(int32_t batch, int32_t vocab, int32_t depth, int32_t step,
                                     const int32_t* top_head, const int32_t* top_k_spec) {
  specv::TreeDraftPlan p = {};
  int first = 1, prev_first = 0, ko = 0, rows = 0;
  for (int s = 0; s < step; ++s) {
    int made = 0;
    for (int j = 0; j < top_head[s]; ++j) made += top_k_spec[ko + j];
    ko += top_head[s];
    rows += top_head[s];
    prev_first = first;
    first += made;
  }
  p.h = top_head[step];
  p.par_lo = step == 0 ? 0 : prev_first;
  p.par_hi = step == 0 ? 1 : first;
  p.first_new = first;
  int off = 0;
  for (int j = 0; j < p.h; ++j) {
    p.kk[j] = top_k_spec[ko + j];
    p.koff[j] = off;
    off += p.kk[j];
    p.kmax = p.kk[j] > p.kmax ? p.kk[j] : p.kmax;
  }
  p.n_new = off;
  p.h_next = step + 1 < depth ? top_head[step + 1] : 0;
  p.row_base_next = rows + p.h;
  p.splits = specv::tree_draft_splits(batch * p.h, vocab);
  return p;
}

size_t tree_draft_bytes(int32_t batch, int32_t vocab, int32_t depth, const int32_t* top_head,
                        const int32_t* top_k_spec) {
  size_t need = 256;
  for (int s = 0; s < depth; ++s) {
    const specv::TreeDraftPlan p = tree_draft_plan(batch, vocab, depth, s, top_head, top_k_spec);
    const size_t b = (size_t)batch * p.h * p.splits * specv::tree_draft_record_bytes(p.kmax);
    need = b > need ? b : need;
  }
  return specv::align256(need);
}

}  // namespace

extern "C" {

int spec_abi_version(void) { return SPEC_ABI_VERSION; }

const char* spec_last_error(void) { return g_err; }

size_t spec_verify_chain_workspace_size(int32_t batch, int32_t total_draft_rows, int32_t vocab) {
  if (batch < 0 || total_draft_rows < 0 || vocab < 1 || vocab > kMaxVocab) return 0;
  return specv::chain_workspace_bytes(batch, total_draft_rows, vocab);
}

namespace {

// Host-visible checks of a chain call (who names the entry point). SPEC_OK with *empty set
// when the batch is empty and there is nothing to launch.
int check_chain(const spec_chain_args* a, const char* who, bool* empty) {
  *empty = false;
  if (!a) return fail(SPEC_ERR_INVALID_ARG, "%s: args is NULL", who);
  if (a->batch < 0) return fail(SPEC_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->vocab < 1 || a->vocab > kMaxVocab)
    return fail(SPEC_ERR_INVALID_ARG, "vocab must be in [1, %d] (got %d)", kMaxVocab, a->vocab);
  if (a->row_stride < a->vocab || a->row_stride % 8 != 0)
    return fail(SPEC_ERR_INVALID_ARG,
                "row_stride must be >= vocab and a multiple of 8 (got %d, vocab %d)",
                a->row_stride, a->vocab);
  if (a->max_gamma < 0 || a->max_gamma > kMaxGamma)
    return fail(SPEC_ERR_INVALID_ARG, "max_gamma must be in [0, %d] (got %d)", kMaxGamma,
                a->max_gamma);
  if (a->total_draft_rows < 0 ||
      (int64_t)a->total_draft_rows > (int64_t)a->batch * a->max_gamma)
    return fail(SPEC_ERR_INVALID_ARG, "total_draft_rows must be in [0, batch*max_gamma] (got %d)",
                a->total_draft_rows);
  if (a->lead_slots != 0 && a->lead_slots != 1)
    return fail(SPEC_ERR_INVALID_ARG, "lead_slots must be 0 or 1 (got %d)", a->lead_slots);
  if (a->batch == 0) {
    *empty = true;
    return SPEC_OK;
  }
  if (!a->target_logits || !a->cu_gamma || !a->temperature || !a->committed_len ||
      !a->out_tokens || !a->num_accepted)
    return fail(SPEC_ERR_INVALID_ARG,
                "target_logits, cu_gamma, temperature, committed_len, out_tokens and "
                "num_accepted are required");
  if (a->total_draft_rows > 0 && !a->draft_tokens)
    return fail(SPEC_ERR_INVALID_ARG, "draft_tokens is required when total_draft_rows > 0");
  if (!aligned16(a->target_logits) || (a->draft_logits && !aligned16(a->draft_logits)))
    return fail(SPEC_ERR_INVALID_ARG, "logits base pointers must be 16-byte aligned");
  if ((int64_t)a->batch * (2 * a->max_gamma + 1) > 0x7FFFFFFFLL)
    return fail(SPEC_ERR_INVALID_ARG, "batch * (2 * max_gamma + 1) exceeds the grid limit");
  return SPEC_OK;
}

}  // namespace

int spec_verify_chain(const spec_chain_args* a, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  g_err[0] = '\0';
  bool empty = false;
  const int rc = check_chain(a, "spec_verify_chain", &empty);
  if (rc != SPEC_OK || empty) return rc;
  const size_t need =
      specv::chain_workspace_bytes(a->batch, a->total_draft_rows, a->vocab);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned and >= %zu bytes", need);
  hipError_t e = specv::launch_chain(*a, workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "spec_verify_chain launch");
  return SPEC_OK;
}

int spec_verify_chain_timed(const spec_chain_args* a, void* workspace, size_t workspace_bytes,
                            void* hip_stream, void* const* events) {
  g_err[0] = '\0';
  if (!events) return fail(SPEC_ERR_INVALID_ARG, "spec_verify_chain_timed: events is NULL");
  bool empty = false;
  const int rc = check_chain(a, "spec_verify_chain_timed", &empty);
  if (rc != SPEC_OK || empty) return rc;
  const size_t need =
      specv::chain_workspace_bytes(a->batch, a->total_draft_rows, a->vocab);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned and >= %zu bytes", need);
  hipError_t e = specv::launch_chain(*a, workspace, (hipStream_t)hip_stream, events);
  if (e != hipSuccess) return hip_fail(e, "spec_verify_chain_timed launch");
  return SPEC_OK;
}

int spec_verify_chain_noalloc(const spec_chain_args* a, void* hip_stream) {
  g_err[0] = '\0';
  bool empty = false;
  const int rc = check_chain(a, "spec_verify_chain_noalloc", &empty);
  if (rc != SPEC_OK || empty) return rc;
  const size_t need =
      specv::chain_workspace_bytes(a->batch, a->total_draft_rows, a->vocab);
  if (need > specv::kChainScratchBytes)
    return fail(SPEC_ERR_WORKSPACE,
                "spec_verify_chain_noalloc: this call needs %zu bytes of scratch, more than the "
                "%zu the library holds per GPU; use spec_verify_chain with a workspace",
                need, specv::kChainScratchBytes);
  void* ws = nullptr;
  hipError_t e = specv::chain_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "spec_verify_chain_noalloc: scratch address");
  e = specv::launch_chain(*a, ws, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "spec_verify_chain_noalloc launch");
  return SPEC_OK;
}

size_t spec_verify_tree_workspace_size(int32_t batch, int32_t rows_per_seq) {
  if (batch < 0 || rows_per_seq < 1 || rows_per_seq > 256) return 0;
  return specv::tree_workspace_bytes(batch, rows_per_seq);
}

int spec_verify_tree(const spec_tree_args* a, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
  g_err[0] = '\0';
  if (!a) return fail(SPEC_ERR_INVALID_ARG, "spec_verify_tree: args is NULL");
  if (a->batch < 0) return fail(SPEC_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->vocab < 1 || a->vocab > kMaxVocab)
    return fail(SPEC_ERR_INVALID_ARG, "vocab must be in [1, %d] (got %d)", kMaxVocab, a->vocab);
  if (a->row_stride < a->vocab || a->row_stride % 8 != 0)
    return fail(SPEC_ERR_INVALID_ARG, "row_stride must be >= vocab and a multiple of 8");
  if (a->num_nodes < 1 || a->num_nodes > 256)
    return fail(SPEC_ERR_INVALID_ARG, "num_nodes must be in [1, 256] (got %d)", a->num_nodes);
  if (a->rows_per_seq < 1 || a->rows_per_seq > 256)
    return fail(SPEC_ERR_INVALID_ARG, "rows_per_seq must be in [1, 256] (got %d)",
                a->rows_per_seq);
  if (a->max_depth < 1 || a->max_depth > 64)
    return fail(SPEC_ERR_INVALID_ARG, "max_depth must be in [1, 64] (got %d)", a->max_depth);
  if (a->tree_stride != 0 && a->tree_stride < a->num_nodes)
    return fail(SPEC_ERR_INVALID_ARG, "tree_stride must be 0 or >= num_nodes");
  if (a->batch == 0) return SPEC_OK;
  if (!a->target_logits || !a->parent || !a->node_row || !a->node_token || !a->path_nodes ||
      !a->path_len || !a->out_tokens || !a->num_emitted)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(a->target_logits))
    return fail(SPEC_ERR_INVALID_ARG, "target_logits must be 16-byte aligned");
  if ((int64_t)a->batch * a->rows_per_seq > 0x7FFFFFFFLL)
    return fail(SPEC_ERR_INVALID_ARG, "batch * rows_per_seq exceeds the grid limit");
  const size_t need = specv::tree_workspace_bytes(a->batch, a->rows_per_seq);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned and >= %zu bytes", need);
  hipError_t e = specv::launch_tree(*a, workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "spec_verify_tree launch");
  return SPEC_OK;
}

int kv_commit_path(const spec_kv_args* a, void* hip_stream) {
  g_err[0] = '\0';
  if (!a) return fail(SPEC_ERR_INVALID_ARG, "kv_commit_path: args is NULL");
  if (a->batch < 0) return fail(SPEC_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->num_layers < 1 || a->num_layers > 128)
    return fail(SPEC_ERR_INVALID_ARG, "num_layers must be in [1, 128] (got %d)", a->num_layers);
  if (a->num_kv_heads < 1)
    return fail(SPEC_ERR_INVALID_ARG, "num_kv_heads must be >= 1 (got %d)", a->num_kv_heads);
  if (a->head_dim < 8 || a->head_dim % 8 != 0)
    return fail(SPEC_ERR_INVALID_ARG,
                "head_dim must be a positive multiple of 8 (16-byte rows; got %d)", a->head_dim);
  if (a->seq_stride < 0 || a->slot_stride < 0 || a->head_stride < 0 ||
      a->seq_stride % 8 || a->slot_stride % 8 || a->head_stride % 8)
    return fail(SPEC_ERR_INVALID_ARG, "strides must be non-negative multiples of 8 elements");
  if (a->slot_capacity < 1)
    return fail(SPEC_ERR_INVALID_ARG, "slot_capacity must be >= 1");
  if (a->lead_slots != 0 && a->lead_slots != 1)
    return fail(SPEC_ERR_INVALID_ARG, "lead_slots must be 0 or 1 (got %d)", a->lead_slots);
  if (a->max_depth < 1 || a->max_depth > 64)
    return fail(SPEC_ERR_INVALID_ARG, "max_depth must be in [1, 64] (got %d)", a->max_depth);
  {
    // 16-byte chunks of one slot over every layer, K and V, and head; the copy grid
    const int64_t chunks = (int64_t)a->num_layers * 2 * a->num_kv_heads * (a->head_dim / 8);
    if (chunks > (1 << 30) || (int64_t)a->batch * ((chunks + 1023) / 1024) > 0x7FFFFFFF)
      return fail(SPEC_ERR_INVALID_ARG,
                  "num_layers * 2 * num_kv_heads * head_dim / 8 (or that times batch / 1024) "
                  "exceeds the grid limit");
  }
  if (a->batch == 0) return SPEC_OK;
  if (!a->k_cache || !a->v_cache || !a->path_nodes || !a->path_len || !a->committed_len)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  for (int l = 0; l < a->num_layers; ++l) {
    if (!a->k_cache[l] || !a->v_cache[l])
      return fail(SPEC_ERR_INVALID_ARG, "k_cache[%d] / v_cache[%d] is NULL", l, l);
    if (!aligned16(a->k_cache[l]) || !aligned16(a->v_cache[l]))
      return fail(SPEC_ERR_INVALID_ARG, "cache pointers of layer %d must be 16-byte aligned", l);
  }
  hipError_t e = specv::launch_kv(*a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "kv_commit_path launch");
  return SPEC_OK;
}

size_t spec_tree_draft_workspace_size(int32_t batch, int32_t vocab, int32_t depth,
                                      const int32_t* top_head, const int32_t* top_k_spec) {
  if (batch < 0 || vocab < 1 || vocab > kMaxVocab) return 0;
  char saved[sizeof g_err];
  std::memcpy(saved, g_err, sizeof g_err);
  int nodes = 0;
  const int rc = check_tree_config(vocab, depth, top_head, top_k_spec, &nodes);
  std::memcpy(g_err, saved, sizeof g_err);  // a size query leaves the error string alone
  if (rc != SPEC_OK) return 0;
  return tree_draft_bytes(batch, vocab, depth, top_head, top_k_spec);
}

int spec_tree_draft_step(const spec_tree_draft_args* a, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
  g_err[0] = '\0';
  if (!a) return fail(SPEC_ERR_INVALID_ARG, "spec_tree_draft_step: args is NULL");
  if (a->batch < 0) return fail(SPEC_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->vocab < 1 || a->vocab > kMaxVocab)
    return fail(SPEC_ERR_INVALID_ARG, "vocab must be in [1, %d] (got %d)", kMaxVocab, a->vocab);
  if (a->row_stride < a->vocab || a->row_stride % 8 != 0)
    return fail(SPEC_ERR_INVALID_ARG, "row_stride must be >= vocab and a multiple of 8");
  int nodes = 0;
  const int rc = check_tree_config(a->vocab, a->depth, a->top_head, a->top_k_spec, &nodes);
  if (rc != SPEC_OK) return rc;
  if (a->step < 0 || a->step >= a->depth)
    return fail(SPEC_ERR_INVALID_ARG, "step must be in [0, depth) (got %d, depth %d)", a->step,
                a->depth);
  if (a->tree_stride < nodes || a->tree_stride > specv::kTreeDraftMaxNodes)
    return fail(SPEC_ERR_INVALID_ARG, "tree_stride must be in [%d, %d] (got %d)", nodes,
                specv::kTreeDraftMaxNodes, a->tree_stride);
  int hmax = 0;
  for (int s = 0; s < a->depth; ++s) hmax = a->top_head[s] > hmax ? a->top_head[s] : hmax;
  if (a->expand_stride < hmax)
    return fail(SPEC_ERR_INVALID_ARG, "expand_stride must be >= %d (got %d)", hmax,
                a->expand_stride);
  if (a->batch == 0) return SPEC_OK;
  if (!a->draft_logits || !a->parent || !a->node_token || !a->node_row || !a->node_logp ||
      !a->position_ids || !a->ancestor_mask || !a->expand_nodes ||
      (a->step == 0 && !a->root_token))
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(a->draft_logits))
    return fail(SPEC_ERR_INVALID_ARG, "draft_logits must be 16-byte aligned");
  const specv::TreeDraftPlan p =
      tree_draft_plan(a->batch, a->vocab, a->depth, a->step, a->top_head, a->top_k_spec);
  if ((int64_t)a->batch * p.h * p.splits > 0x7FFFFFFFLL)
    return fail(SPEC_ERR_INVALID_ARG, "batch * top_head[step] exceeds the grid limit");
  const size_t need = tree_draft_bytes(a->batch, a->vocab, a->depth, a->top_head, a->top_k_spec);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned and >= %zu bytes", need);
  hipError_t e = specv::launch_tree_draft(*a, p, workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "spec_tree_draft_step launch");
  return SPEC_OK;
}

int kv_commit_paged(const spec_paged_kv_args* a, void* hip_stream) {
  g_err[0] = '\0';
  if (!a) return fail(SPEC_ERR_INVALID_ARG, "kv_commit_paged: args is NULL");
  if (a->batch < 0) return fail(SPEC_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->num_layers < 1 || a->num_layers > 128)
    return fail(SPEC_ERR_INVALID_ARG, "num_layers must be in [1, 128] (got %d)", a->num_layers);
  if (a->num_kv_heads < 1)
    return fail(SPEC_ERR_INVALID_ARG, "num_kv_heads must be >= 1 (got %d)", a->num_kv_heads);
  if (a->head_dim < 8 || a->head_dim % 8 != 0)
    return fail(SPEC_ERR_INVALID_ARG,
                "head_dim must be a positive multiple of 8 (16-byte rows; got %d)", a->head_dim);
  if (a->block_size < 1 || a->max_blocks < 1 || a->num_blocks < 1)
    return fail(SPEC_ERR_INVALID_ARG, "block_size, max_blocks and num_blocks must be >= 1");
  if ((int64_t)a->max_blocks * a->block_size > 0x7FFFFFFFLL)
    return fail(SPEC_ERR_INVALID_ARG, "max_blocks * block_size exceeds the slot index range");
  if (a->max_blocks > (1 << 24))
    return fail(SPEC_ERR_INVALID_ARG, "max_blocks must be <= 2^24 (got %d)", a->max_blocks);
  if (a->free_capacity < a->num_blocks)
    return fail(SPEC_ERR_INVALID_ARG, "free_capacity must be >= num_blocks (got %d < %d)",
                a->free_capacity, a->num_blocks);
  if (a->block_stride < 0 || a->slot_stride < 0 || a->head_stride < 0 ||
      a->block_stride % 8 || a->slot_stride % 8 || a->head_stride % 8)
    return fail(SPEC_ERR_INVALID_ARG, "strides must be non-negative multiples of 8 elements");
  if (a->lead_slots != 0 && a->lead_slots != 1)
    return fail(SPEC_ERR_INVALID_ARG, "lead_slots must be 0 or 1 (got %d)", a->lead_slots);
  if (a->max_depth < 1 || a->max_depth > 64)
    return fail(SPEC_ERR_INVALID_ARG, "max_depth must be in [1, 64] (got %d)", a->max_depth);
  {
    // 16-byte chunks of one slot over every layer, K and V, and head; the copy grid
    const int64_t chunks = (int64_t)a->num_layers * 2 * a->num_kv_heads * (a->head_dim / 8);
    if (chunks > (1 << 30) || (int64_t)a->batch * ((chunks + 1023) / 1024) > 0x7FFFFFFF)
      return fail(SPEC_ERR_INVALID_ARG,
                  "num_layers * 2 * num_kv_heads * head_dim / 8 (or that times batch / 1024) "
                  "exceeds the grid limit");
  }
  if (a->batch == 0) return SPEC_OK;
  if (!a->k_cache || !a->v_cache || !a->block_table || !a->path_nodes || !a->path_len ||
      !a->committed_len || !a->free_list || !a->free_count)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  for (int l = 0; l < a->num_layers; ++l) {
    if (!a->k_cache[l] || !a->v_cache[l])
      return fail(SPEC_ERR_INVALID_ARG, "k_cache[%d] / v_cache[%d] is NULL", l, l);
    if (!aligned16(a->k_cache[l]) || !aligned16(a->v_cache[l]))
      return fail(SPEC_ERR_INVALID_ARG, "cache pointers of layer %d must be 16-byte aligned", l);
  }
  hipError_t e = specv::launch_kv_paged(*a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "kv_commit_paged launch");
  return SPEC_OK;
}

int spec_ngram_draft(const spec_ngram_args* a, void* hip_stream) {
  g_err[0] = '\0';
  if (!a) return fail(SPEC_ERR_INVALID_ARG, "spec_ngram_draft: args is NULL");
  if (a->batch < 0) return fail(SPEC_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->hist_stride < 4 || a->hist_stride % 4 != 0)
    return fail(SPEC_ERR_INVALID_ARG, "hist_stride must be a positive multiple of 4 (got %d)",
                a->hist_stride);
  if (a->ngram_min < 1 || a->ngram_max < a->ngram_min || a->ngram_max > 64)
    return fail(SPEC_ERR_INVALID_ARG, "need 1 <= ngram_min <= ngram_max <= 64 (got %d, %d)",
                a->ngram_min, a->ngram_max);
  if (a->num_draft < 1 || a->num_draft > 64)
    return fail(SPEC_ERR_INVALID_ARG, "num_draft must be in [1, 64] (got %d)", a->num_draft);
  if (a->draft_stride < a->num_draft)
    return fail(SPEC_ERR_INVALID_ARG, "draft_stride must be >= num_draft");
  if (a->batch == 0) return SPEC_OK;
  if (!a->tokens || !a->hist_len || !a->draft_tokens || !a->num_drafts)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(a->tokens))
    return fail(SPEC_ERR_INVALID_ARG, "tokens must be 16-byte aligned");
  hipError_t e = specv::launch_ngram(*a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "spec_ngram_draft launch");
  return SPEC_OK;
}

}  // extern "C"
