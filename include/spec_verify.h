/*
 * spec_verify.h -- C ABI of the MI355X speculative-sampling verification library
 * (libspecv.so, gfx950).
 *
 * One round of speculative sampling: a drafter proposes d_1..d_gamma with laws q_1..q_gamma;
 * the target scores [x, d_1..d_gamma] in one causal forward and yields p_1..p_{gamma+1};
 * the verifier tests the drafts left to right, keeps the accepted prefix, and adds one
 * token -- a residual draw at the first rejection or a bonus draw after a full accept; the
 * KV cache keeps the accepted prefix and drops the rest. Sources (page title, section):
 *   "10.6 投机解码：为什么'先猜后验'能加速" (llm_internals) §10.6.1 (the round in five
 *     steps; greedy special case), §10.6.3 (the verify step's logits[B, gamma+1, n_vocab],
 *     per-request start points, cache truncation after a rejection, tree drafts);
 *   "KV Cache 优化（四）：Speculative Decoding 投机解码" §4 (eq. a(x) and eq. p'(x); the law
 *     after temperature and top-k/top-p is the one to test), §5 (bonus token), §6 (reserved
 *     slots and one committed-length pointer, the same in every layer);
 *   "投机解码" (LLM glossary), exact acceptance section (q = 0 and zero-residual cases);
 *   "投机推理：小模型搭树，大模型一次验证", validation and path-walk sections (tree), tree
 *     configuration and draft-step sections (tree drafting).
 *
 * Conventions for every call
 *  - Logits are bf16, passed as raw uint16 bit patterns, row-major with row_stride elements
 *    per row (row_stride >= vocab, a multiple of 8; base pointers 16-byte aligned). A row
 *    must hold at least one finite logit; NaN and +inf logits are not supported.
 *  - All array arguments are DEVICE pointers owned by the caller, except where a field says
 *    "host". The library allocates nothing, keeps no pointer after returning, and holds no
 *    global state except a thread-local error string and the scratch array of
 *    spec_verify_chain_noalloc (below). Calls are thread-safe, except that calls of
 *    spec_verify_chain_noalloc that overlap on one GPU race on that GPU's array.
 *  - Work is enqueued on hip_stream (a hipStream_t; NULL = the default stream). Outputs are
 *    valid after the stream is synchronised; inputs must stay alive until then.
 *  - Host validation reads only host-visible fields and makes no HIP call before it passes.
 *    On SPEC_ERR_INVALID_ARG / SPEC_ERR_UNSUPPORTED / SPEC_ERR_WORKSPACE nothing is enqueued
 *    and no output is touched. spec_last_error() then describes the failure.
 *  - Data errors only visible on the device set bits in seq_flags[b]; see SPEC_FLAG_*.
 *  - Results are a pure function of the inputs and the seed: independent of batch
 *    composition (uniforms are keyed by seq_id) and of launch geometry; repeated calls give
 *    identical bits.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 8

/* ---- status codes ---------------------------------------------------------------------- */
#define SPEC_OK 0
#define SPEC_ERR_INVALID_ARG (-1)  /* a host-visible argument is out of range            */
#define SPEC_ERR_UNSUPPORTED (-2)  /* a reserved feature was requested                   */
#define SPEC_ERR_HIP (-3)          /* a HIP launch or event call failed                   */
#define SPEC_ERR_WORKSPACE (-4)    /* workspace NULL, misaligned or smaller than required */

/* ---- seq_flags bits -------------------------------------------------------------------- */
#define SPEC_FLAG_BAD_TOKEN 1       /* a draft token is outside [0, vocab): no progress      */
#define SPEC_FLAG_Q_ZERO 2          /* q_k(d_k) = 0 at a tested position (a = [p_k(d_k)>0]) */
#define SPEC_FLAG_RESID_FALLBACK 4  /* residual mass was 0: the draw used p_k itself        */
#define SPEC_FLAG_NO_ROW 8          /* tree walk stopped at a node without a target row     */
#define SPEC_FLAG_SLOT_OOB 16       /* KV slot outside [0, slot_capacity): no progress      */
#define SPEC_FLAG_BAD_TREE 32       /* parent/node_row malformed: no progress               */
#define SPEC_FLAG_TOPP_SLOW 64      /* a top-k/top-p threshold needed another read of a row
                                       (a second capture, or the exact multi-pass search)   */
#define SPEC_FLAG_BAD_PARAM 128     /* T neither 0 nor in [2^-126, 2^126] (negative, NaN,
                                       inf, subnormal, huge), top_p outside (0,1], gamma_b
                                       out of range, or a history length outside its row:
                                       no progress                                          */
#define SPEC_FLAG_FREE_FULL 1024    /* paged release: the free list was full; the blocks
                                       that did not fit stay in the block table            */
#define SPEC_FLAG_EOS 256           /* the round's last emitted token is the EOS id         */
#define SPEC_FLAG_LEN_CAP 512       /* the emission cap cut the round short                 */

/* ---- uniform purposes (third word of the Philox counter) ------------------------------- */
#define SPEC_PURPOSE_ACCEPT 0
#define SPEC_PURPOSE_RESIDUAL 1
#define SPEC_PURPOSE_BONUS 2

/*
 * Chain verification of a ragged batch ("10.6 投机解码" §10.6.1 steps 1-5; §10.6.3).
 *
 * Sequence b has gamma_b = cu_gamma[b+1] - cu_gamma[b] drafts (0 <= gamma_b <= max_gamma).
 * Target row of (b, k), k = 1..gamma_b+1, is cu_gamma[b] + b + k - 1 (p_k predicts the k-th
 * new token); draft row of (b, k), k = 1..gamma_b, is cu_gamma[b] + k - 1.
 *
 * Per sequence, with L = committed_len[b] on entry, T = temperature[b], P = top_p[b],
 * K = top_k[b]:
 *  - laws: p_k = top-p_P(top-k_K(softmax(target row / T))), q_k likewise from the draft row
 *    (the same T, K and P; "KV Cache 优化（四）" §4 names top-k/top-p). Top-k keeps every token
 *    whose logit is >= the K-th largest logit (repeats counted, so ties at the boundary are
 *    kept); K <= 0 or K >= V keeps all. Top-p then keeps every token whose logit is >= t*,
 *    t* the largest logit value at which the mass of all kept tokens at or above it reaches
 *    P of the top-k set's mass. T = 0 is greedy: p_k is one-hot at the target argmax (lowest
 *    id on ties) and q is not read. With draft_logits NULL and T > 0, q_k is the point mass
 *    at d_k -- a drafter without a law, such as spec_ngram_draft, proposes d_k with
 *    certainty -- so a_k = p_k(d_k) and the residual is p_k without d_k.
 *  - test: a_k = min(1, p_k(d_k)/q_k(d_k)) (eq. a(x)); where q_k(d_k) = 0, a_k = [p_k(d_k) > 0]
 *    and SPEC_FLAG_Q_ZERO is set; accept iff u_acc < a_k, u_acc = U(L+k, ACCEPT). Greedy:
 *    accept iff d_k equals the target argmax.
 *  - first rejection at k: the emitted token is the inverse-CDF draw (ascending token id)
 *    from max(0, p_k - q_k) with u = U(L+k, RESIDUAL) (eq. p'(x)); if that mass is 0, from p_k
 *    (SPEC_FLAG_RESID_FALLBACK). Greedy: the target argmax.
 *  - all accepted: a bonus draw from p_{gamma_b+1} with u = U(L+gamma_b+1, BONUS) ("KV Cache
 *    优化（四）" §5). Greedy: the argmax. gamma_b = 0 is allowed: the round is one draw from
 *    p_1 -- which is also how a drafter can draw its own tokens through this call.
 *  - early stop ("KV Cache 优化（四）" §5: EOS and the length cap end a round early): the
 *    round emits the accepted drafts in order, then y; emission stops after the first
 *    emitted token equal to eos_token[b] (SPEC_FLAG_EOS) and after max_emit[b] tokens
 *    (SPEC_FLAG_LEN_CAP when that cuts the round short). A stop inside the accepted drafts
 *    ends the round there: no later position is tested and no y is drawn.
 *  - outputs: out_tokens[target row (b, 1..m)] = the m emitted tokens (d_1..d_n, then y if
 *    drawn); num_accepted[b] = n (accepted drafts emitted); num_emitted[b] = m (n or n+1);
 *    committed_len[b] = L + lead_slots + n (pointer-only rollback, "KV Cache 优化（四）" §6:
 *    no KV byte moves; the rejected drafts' slots are simply past the pointer).
 *  U(pos, purpose) = Philox4x32-10 with key (seed low 32 bits, seed high 32 bits), counter
 *  (seq_id[b], pos, purpose, 0); u = (first output word >> 8) * 2^-24.
 */
typedef struct spec_chain_args {
  int32_t batch;            /* B >= 0 (0: nothing to do)                                    */
  int32_t vocab;            /* V >= 1                                                        */
  int32_t row_stride;       /* elements between rows; >= vocab, multiple of 8               */
  int32_t max_gamma;        /* 0..64: bound on every gamma_b                                 */
  int32_t total_draft_rows; /* = cu_gamma[B] (sum of gamma_b); >= 0                          */
  int32_t lead_slots;       /* 0 or 1 (1: the round also wrote x's slot at L)                */
  uint64_t seed;            /* Philox key                                                    */
  const uint16_t* target_logits; /* [total_draft_rows + B][row_stride] bf16                 */
  const uint16_t* draft_logits;  /* [total_draft_rows][row_stride] bf16, or NULL: point-mass
                                    draft laws (no draft row is read)                      */
  const int32_t* cu_gamma;       /* [B+1], cu_gamma[0] = 0, non-decreasing                    */
  const int32_t* draft_tokens;   /* [total_draft_rows]; may be NULL if total_draft_rows = 0  */
  const float* temperature;      /* [B], 0 (greedy) or in [2^-126, 2^126] (else BAD_PARAM)   */
  const float* top_p;            /* [B] in (0, 1], or NULL = no top-p                        */
  const int32_t* top_k;          /* [B] or NULL = no top-k; K <= 0 or K >= vocab: off        */
  const uint32_t* seq_id;        /* [B] Philox stream ids, or NULL = b                       */
  int32_t* committed_len;        /* [B] in/out: L on entry, L + lead_slots + n on exit       */
  int32_t* out_tokens;           /* [total_draft_rows + B]; entries past the m emitted tokens
                                    of a sequence are untouched                              */
  int32_t* num_accepted;         /* [B]                                                      */
  int32_t* seq_flags;            /* [B] or NULL                                              */
  float* probe_rows;             /* [total_draft_rows][3] or NULL: {p_k(d_k), q_k(d_k), a_k}
                                    for tested positions (greedy: {[d=argmax], NaN, accept}) */
  float* probe_seq;              /* [B][2] or NULL: {residual mass R (NaN if no rejection),
                                    probability of the emitted last token under its law}    */
  const float* uniform_override; /* [total_draft_rows + B][2] or NULL (test hook): row (b,k)
                                    supplies {u_acc for k, u for the residual/bonus draw at k}
                                    in place of the Philox uniforms                          */
  const int32_t* eos_token;      /* [B] or NULL: a sequence's EOS id (< 0: none)              */
  const int32_t* max_emit;       /* [B] or NULL: most tokens the round may emit (<= 0: no cap) */
  int32_t* num_emitted;          /* [B] or NULL: tokens emitted this round                   */
} spec_chain_args;

/*
 * Greedy tree verification ("投机推理：小模型搭树，大模型一次验证", validation and path walk;
 * "10.6 投机解码" §10.6.3 tree drafts).
 *
 * Node 0 is the root (the last committed token; never verified). Node i >= 1 has parent
 * parent[i] < i and token node_token[b][i]. node_row[i] is the target row holding the
 * target's next-token logits after node i, or -1. The walk starts at v = 0: if v has no row
 * it stops (SPEC_FLAG_NO_ROW, no extra token); else t = argmax of v's row (lowest id on
 * ties); the lowest-index child c of v with node_token[c] = t is appended to the path and
 * the walk continues from c; if no child matches (or the path already holds max_depth
 * nodes) t is emitted as the extra token and the walk ends. Matches on other branches are
 * never counted.
 *
 * Outputs: path_nodes[b][0..D) (rest set to -1), path_len[b] = D,
 * out_tokens[b][0..D) = tokens of the path, out_tokens[b][D] = the extra token if any,
 * num_emitted[b] = D or D+1. A malformed tree (parent[0] != -1, parent[i] outside [0, i),
 * node_row outside [-1, rows_per_seq)) sets SPEC_FLAG_BAD_TREE and emits nothing.
 */
typedef struct spec_tree_args {
  int32_t batch;          /* B >= 0                                                        */
  int32_t vocab;          /* V >= 1                                                        */
  int32_t row_stride;     /* elements; >= vocab, multiple of 8                             */
  int32_t num_nodes;      /* N+1 including the root; 1..256                                */
  int32_t rows_per_seq;   /* target rows per sequence; 1..256                              */
  int32_t max_depth;      /* path capacity; 1..64                                          */
  int32_t tree_stride;    /* elements between sequences in parent/node_row; 0 = one
                             topology for the whole batch, else >= num_nodes              */
  const uint16_t* target_logits; /* [B][rows_per_seq][row_stride] bf16                    */
  const int32_t* parent;         /* [B or 1][tree_stride or num_nodes]                    */
  const int32_t* node_row;       /* same layout as parent                                 */
  const int32_t* node_token;     /* [B][num_nodes]                                        */
  int32_t* path_nodes;           /* [B][max_depth]                                        */
  int32_t* path_len;             /* [B]                                                   */
  int32_t* out_tokens;           /* [B][max_depth + 1]                                    */
  int32_t* num_emitted;          /* [B]                                                   */
  int32_t* seq_flags;            /* [B] or NULL                                           */
} spec_tree_args;

/*
 * KV commit of an accepted path ("KV Cache 优化（四）" §6; "10.6 投机解码" §10.6.3).
 *
 * The verify forward wrote node i's K/V (i >= 1, tree node index or chain draft index) at
 * slot base + i, base = L + lead_slots - 1, L = committed_len[b]. For j = 1..D (D =
 * path_len[b], in increasing j) every layer's K and V rows of every KV head are copied from
 * slot base + path_nodes[b][j-1] to slot base + j (skipped when equal), then committed_len[b]
 * becomes L + lead_slots + D. Slots outside [0, slot_capacity) set SPEC_FLAG_SLOT_OOB
 * (OR-ed into seq_flags) and leave that sequence untouched. A chain round's path is the
 * identity (path[j-1] = j), which moves no byte: the commit is then a pointer update, which
 * is also how a draft model's cache is rolled back.
 *
 * Element (b, slot, head, e) of layer l's K cache is k_cache[l][b*seq_stride +
 * slot*slot_stride + head*head_stride + e], e < head_dim, bf16 (copied bit for bit).
 * num_layers * 2 * num_kv_heads * head_dim / 8 must not exceed 2^30, nor that count / 1024
 * times batch 2^31 - 1 (SPEC_ERR_INVALID_ARG).
 */
typedef struct spec_kv_args {
  int32_t batch;          /* B >= 0                                                       */
  int32_t num_layers;     /* 1..128                                                       */
  int32_t num_kv_heads;   /* >= 1                                                         */
  int32_t head_dim;       /* elements; head_dim * 2 bytes a multiple of 16                */
  int64_t seq_stride;     /* elements; multiples of 8                                     */
  int64_t slot_stride;
  int64_t head_stride;
  int32_t slot_capacity;  /* slots per sequence                                           */
  int32_t lead_slots;     /* 0 or 1                                                       */
  int32_t max_depth;      /* row length of path_nodes; 1..64                              */
  uint16_t* const* k_cache; /* HOST array [num_layers] of device pointers (16-B aligned)   */
  uint16_t* const* v_cache; /* HOST array [num_layers] of device pointers (16-B aligned)   */
  const int32_t* path_nodes; /* [B][max_depth], node indices >= 1 in depth order           */
  const int32_t* path_len;   /* [B], 0..max_depth                                          */
  int32_t* committed_len;    /* [B] in/out                                                 */
  int32_t* seq_flags;        /* [B] or NULL (bits OR-ed in)                                */
} spec_kv_args;

/*
 * One drafting step of a token tree ("投机推理：小模型搭树，大模型一次验证", sections on the
 * tree configuration -- gamma, topKSpec, topHead -- and on the three draft steps of the dump
 * example; "10.6 投机解码" §10.6.3, tree drafts, Table 10-17 and the depth positions).
 *
 * A tree is grown by `depth` calls, step = 0, 1, ..., depth-1, with the draft model's forward
 * between them. Step s reads one draft logits row per node expanded at this step: row j of
 * sequence b follows expand_nodes[b][j], j < top_head[s] (step 0 expands the root alone). The
 * j-th expanded node gets as children the top_k_spec[s][j] tokens of largest draft logit,
 * larger first, ties to the lower token id. A node's path log-probability (node_logp) is its
 * parent's plus the natural log of its token's draft softmax probability (temperature 1, no
 * filter); the root's is 0. Unless s is the last step, the top_head[s+1] nodes of the new
 * layer with the largest path log-probability (compared as float; ties to the lower node
 * index) then become expand_nodes[b][0..top_head[s+1]), most probable first, and receive
 * the target rows sum(top_head[0..s]) + j in that order (node_row).
 *
 * Node numbering: root 0, then layer by layer; inside a layer by the rank of the parent and
 * then of the child. Target rows belong to the expanded nodes in expansion order (the root
 * has row 0): the layout spec_verify_tree reads with rows_per_seq = sum(top_head). With
 * tree_stride = 1 + sum(top_k_spec) the arrays pass to spec_verify_tree as they are
 * (num_nodes = tree_stride, max_depth = depth).
 *
 * Step 0 writes every entry of each sequence's arrays: node 0 gets token root_token[b],
 * parent -1, row 0, log-probability 0, position pos_base[b] (0 if pos_base is NULL) and
 * mask bit 0; every other entry parent -1, token -1, row -1, log-probability -inf, position
 * -1 and no mask bits, until a later step creates the node. A created node's mask row holds
 * its own bit and its ancestors' (node i sees node j iff bit j%32 of word j/32 is set), and
 * its position is its parent's plus one.
 *
 * Data errors: at step s >= 1, an expand_nodes[b][j] outside the previous step's layer sets
 * SPEC_FLAG_BAD_TREE in seq_flags[b] (when given) and that sequence's step writes nothing.
 */
typedef struct spec_tree_draft_args {
  int32_t batch;          /* B >= 0                                                        */
  int32_t vocab;          /* V >= 1                                                        */
  int32_t row_stride;     /* elements; >= vocab, multiple of 8                             */
  int32_t depth;          /* steps per tree (gamma); 1..64                                 */
  int32_t step;           /* this step; 0..depth-1                                         */
  int32_t tree_stride;    /* node entries per sequence; 1 + sum(top_k_spec) .. 256         */
  int32_t expand_stride;  /* entries per sequence of expand_nodes; >= every top_head[s]    */
  const int32_t* top_head;    /* HOST [depth]: top_head[0] = 1, and for s >= 1
                                 1 <= top_head[s] <= the number of nodes made at step s-1 */
  const int32_t* top_k_spec;  /* HOST: top_k_spec[s][0..top_head[s]) for s = 0..depth-1,
                                 concatenated; each in 1..min(64, vocab)                   */
  const uint16_t* draft_logits; /* [B][top_head[step]][row_stride] bf16                     */
  const int32_t* root_token;    /* [B]; read at step 0                                      */
  const int32_t* pos_base;      /* [B] or NULL; the root's position, read at step 0         */
  int32_t* parent;              /* [B][tree_stride] in/out                                  */
  int32_t* node_token;          /* [B][tree_stride] in/out                                  */
  int32_t* node_row;            /* [B][tree_stride] in/out                                  */
  float* node_logp;             /* [B][tree_stride] in/out                                  */
  int32_t* position_ids;        /* [B][tree_stride] in/out                                  */
  uint32_t* ancestor_mask;      /* [B][tree_stride][(tree_stride + 31) / 32] in/out         */
  int32_t* expand_nodes;        /* [B][expand_stride] in/out                                */
  int32_t* seq_flags;           /* [B] or NULL (bits OR-ed in)                              */
} spec_tree_draft_args;

/*
 * Paged KV commit and release ("10.6 投机解码" §10.6.3: after a rejection the cache length is
 * cut back, and a paged cache releases the blocks it no longer needs; "KV Cache 优化（四）"
 * §6: one committed-length pointer, the same in every layer).
 *
 * Sequence b's logical slot s lives in physical block block_table[b][s / block_size] at
 * offset s % block_size; element (block p, offset o, head h, e) of layer l's K cache is
 * k_cache[l][p*block_stride + o*slot_stride + h*head_stride + e], e < head_dim (bf16,
 * copied bit for bit). With L = committed_len[b], D = path_len[b] and base = L + lead_slots
 * - 1, for j = 1..D (in increasing j) every layer's K and V rows of every KV head move from
 * logical slot base + path_nodes[b][j-1] to logical slot base + j (skipped when equal), as
 * kv_commit_path does in a contiguous cache. Then committed_len[b] becomes L' = L +
 * lead_slots + D, and every mapped logical block at or past ceil(L' / block_size) is
 * released: its id is appended to free_list after the free_count[0] ids already there --
 * sequences in order, each sequence's blocks in logical order -- and its table entry becomes
 * -1. A chain round's identity path (path_nodes[b][j-1] = j) moves no byte: the call is then
 * the rollback itself, length cut back and surplus blocks released; a draft model's cache is
 * rolled back the same way.
 *
 * A sequence with a copied slot outside its table or in an unmapped block (or a block id
 * outside [0, num_blocks)), a path node < 1, or an L' needing more than max_blocks blocks
 * gets SPEC_FLAG_SLOT_OOB and is left untouched. Table entries are -1 or block ids; each
 * block id appears at most once in the tables and the free list together (no shared
 * blocks). A table entry among the blocks the release would free that is >= num_blocks
 * (not a block id) also gives SLOT_OOB, sequence untouched; negative entries are unmapped.
 * free_list has free_capacity entries (>= num_blocks); a released block that finds it full
 * stays in its table entry and the sequence gets SPEC_FLAG_FREE_FULL (copy and length done;
 * only a pool that breaks the rule above gets there).
 * num_layers * 2 * num_kv_heads * head_dim / 8 must not exceed 2^30, nor that count / 1024
 * times batch 2^31 - 1 (SPEC_ERR_INVALID_ARG).
 */
typedef struct spec_paged_kv_args {
  int32_t batch;          /* B >= 0                                                        */
  int32_t num_layers;     /* 1..128                                                        */
  int32_t num_kv_heads;   /* >= 1                                                          */
  int32_t head_dim;       /* elements; a positive multiple of 8 (16-byte rows)             */
  int32_t block_size;     /* slots per block; >= 1                                         */
  int32_t max_blocks;     /* entries per sequence in block_table; 1..2^24                  */
  int32_t num_blocks;     /* physical blocks of every layer's pool; >= 1                   */
  int32_t free_capacity;  /* entries of free_list; >= num_blocks                           */
  int32_t lead_slots;     /* 0 or 1                                                        */
  int32_t max_depth;      /* row length of path_nodes; 1..64                               */
  int64_t block_stride;   /* elements between blocks; multiples of 8                       */
  int64_t slot_stride;    /* elements between a block's slots                              */
  int64_t head_stride;    /* elements between a slot's heads                               */
  uint16_t* const* k_cache; /* HOST array [num_layers] of device pointers (16-B aligned)    */
  uint16_t* const* v_cache; /* HOST array [num_layers] of device pointers (16-B aligned)    */
  int32_t* block_table;      /* [B][max_blocks] in/out                                      */
  const int32_t* path_nodes; /* [B][max_depth], node indices >= 1 in depth order            */
  const int32_t* path_len;   /* [B], 0..max_depth                                           */
  int32_t* committed_len;    /* [B] in/out                                                  */
  int32_t* free_list;        /* [free_capacity] in/out                                      */
  int32_t* free_count;       /* [1] in/out; taken within [0, free_capacity]                */
  int32_t* seq_flags;        /* [B] or NULL (bits OR-ed in)                                 */
} spec_paged_kv_args;

/*
 * n-gram prompt lookup, a drafter without weights ("KV Cache 优化（四）", variants section on
 * n-gram / prefix matching; "10.6 投机解码" §10.6.3: model-free drafts look for the history's
 * trailing n-gram earlier in the prompt or the generated text and propose what followed it;
 * the ngram method's prompt_lookup_min / prompt_lookup_max bound the match window).
 *
 * For sequence b with history h = tokens[b][0..len), len = hist_len[b]: the trailing n-gram
 * h[len-n..len) is looked up among the earlier occurrences h[i..i+n), i < len - n. The longest
 * n in [ngram_min, ngram_max] with an occurrence wins, and for that n the latest occurrence
 * (largest i). The drafts are h[i+n .. min(i+n+num_draft, len)): draft_tokens[b][0..nd) with
 * nd = num_drafts[b], then -1 up to draft_stride; no occurrence gives nd = 0. match_len[b] = n
 * (0 if none) and match_pos[b] = i (-1 if none), when given. A history length outside
 * [0, hist_stride] sets SPEC_FLAG_BAD_PARAM and gives no draft. The drafts of a batch feed
 * spec_verify_chain with gamma_b = num_drafts[b] (cu_gamma its exclusive prefix sum).
 */
typedef struct spec_ngram_args {
  int32_t batch;         /* B >= 0                                                         */
  int32_t hist_stride;   /* elements per history row; a positive multiple of 4             */
  int32_t ngram_min;     /* prompt_lookup_min; 1..ngram_max                                */
  int32_t ngram_max;     /* prompt_lookup_max; ngram_min..64                               */
  int32_t num_draft;     /* drafts per sequence at most (gamma); 1..64                     */
  int32_t draft_stride;  /* elements per row of draft_tokens; >= num_draft                 */
  const int32_t* tokens;   /* [B][hist_stride] token ids (16-byte aligned)                  */
  const int32_t* hist_len; /* [B]                                                          */
  int32_t* draft_tokens;   /* [B][draft_stride]                                            */
  int32_t* num_drafts;     /* [B]                                                          */
  int32_t* match_len;      /* [B] or NULL                                                  */
  int32_t* match_pos;      /* [B] or NULL                                                  */
  int32_t* seq_flags;      /* [B] or NULL (bits OR-ed in)                                  */
} spec_ngram_args;

/* ABI revision of this header (SPEC_ABI_VERSION). */
int spec_abi_version(void);

/* Last error message of the calling thread ("" if none). Valid until the thread's next call. */
const char* spec_last_error(void);

/* Workspace bytes spec_verify_chain needs for this batch shape (device memory, 256-byte
 * aligned, caller-owned, contents need not be initialised). Returns 0 for invalid sizes. */
size_t spec_verify_chain_workspace_size(int32_t batch, int32_t total_draft_rows, int32_t vocab);

/* Enqueue chain verification. Returns SPEC_OK or a negative status. */
int spec_verify_chain(const spec_chain_args* args, void* workspace, size_t workspace_bytes,
                      void* hip_stream);

/*
 * spec_verify_chain without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, checks, kernels and results as spec_verify_chain; the
 * workspace is the library's own scratch array of SPEC_CHAIN_SCRATCH_BYTES per GPU, held by
 * every GPU the library runs on until the process ends. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine). A call whose workspace would exceed
 * the array (spec_verify_chain_workspace_size > SPEC_CHAIN_SCRATCH_BYTES) fails with
 * SPEC_ERR_WORKSPACE before any HIP call; use spec_verify_chain for it. Every call on one
 * GPU uses that GPU's array: calls that may overlap on one GPU (other streams, other host
 * threads) race on it and must be serialized by the caller. Nothing in the array needs to
 * hold anything between calls.
 */
#define SPEC_CHAIN_SCRATCH_BYTES ((size_t)80 << 20)
int spec_verify_chain_noalloc(const spec_chain_args* args, void* hip_stream);

/*
 * Measurement variant of spec_verify_chain: the same call, with two caller-created
 * hipEvent_t (events[0], events[1], a host array) recorded on hip_stream just before and just
 * after the row-statistics kernel, so that a benchmark can time that kernel on the stream it
 * runs on. events must not be NULL; otherwise as spec_verify_chain.
 */
int spec_verify_chain_timed(const spec_chain_args* args, void* workspace, size_t workspace_bytes,
                            void* hip_stream, void* const* events);

/* Workspace bytes spec_verify_tree needs (device memory, 256-byte aligned). */
size_t spec_verify_tree_workspace_size(int32_t batch, int32_t rows_per_seq);

/* Enqueue greedy tree verification. Returns SPEC_OK or a negative status. */
int spec_verify_tree(const spec_tree_args* args, void* workspace, size_t workspace_bytes,
                     void* hip_stream);

/* Enqueue the KV path commit and pointer update. Returns SPEC_OK or a negative status. */
int kv_commit_path(const spec_kv_args* args, void* hip_stream);

/* Workspace bytes every step of spec_tree_draft_step needs for this tree configuration
 * (top_head and top_k_spec are HOST arrays as in spec_tree_draft_args; device memory,
 * 256-byte aligned, contents need not be initialised). Returns 0 for an invalid
 * configuration. */
size_t spec_tree_draft_workspace_size(int32_t batch, int32_t vocab, int32_t depth,
                                      const int32_t* top_head, const int32_t* top_k_spec);

/* Enqueue one tree-drafting step. Returns SPEC_OK or a negative status. */
int spec_tree_draft_step(const spec_tree_draft_args* args, void* workspace,
                         size_t workspace_bytes, void* hip_stream);

/* Enqueue the paged KV commit, pointer update and block release (no workspace). Returns
 * SPEC_OK or a negative status. */
int kv_commit_paged(const spec_paged_kv_args* args, void* hip_stream);

/* Enqueue the n-gram prompt lookup (no workspace). Returns SPEC_OK or a negative status. */
int spec_ngram_draft(const spec_ngram_args* args, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
