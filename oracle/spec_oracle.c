/*
 * spec_oracle.c -- plain fp64 CPU oracle of the speculative-sampling verification step.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark may load or call this library. The GPU library never links,
 * includes or calls it, and it shares no header, helper, table or constant generator with
 * the GPU library: everything below is written out here, once, from the pages.
 *
 * Sources (page title, then section):
 *   [KV]   "KV Cache 优化（四）：Speculative Decoding 投机解码"
 *          §4 acceptance and rejection (eq. a(x), eq. p'(x), the A/B table),
 *          §5 complete example, §6 KV cache commit and rollback.
 *   [LI]   "10.6 投机解码：为什么'先猜后验'能加速" (llm_internals)
 *          §10.6.1 the round in five steps, the losslessness argument, the greedy special case;
 *          §10.6.2 expected tokens per round; §10.6.3 verify-step shape and cache truncation,
 *          tree drafts and Table 10-17.
 *   [GL]   "投机解码" (LLM glossary), section on exact acceptance and the correction
 *          distribution, incl. its edge cases q=0 and a vanishing residual mass.
 *   [TR]   "投机推理：小模型搭树，大模型一次验证", sections on the validation pass and on
 *          walking the accepted path.
 *
 * Readings where the pages leave a step open (each is a plain reading, stated once here):
 *   R1  temperature is applied as softmax(l/T); T = 0 means greedy (one-hot argmax). Other
 *       than 0, T must lie in [2^-126, 2^126], where 1/T is a normal binary32; a negative,
 *       NaN, infinite, subnormal or larger T is invalid (flag BAD_PARAM).
 *   R2  temperature first, then top-p on the tempered law; the same T and top-p for p and q.
 *   R3  top-p is a value threshold over the logits: t* is the largest logit value whose
 *       cumulative mass (all tokens with logit >= t*) reaches P; every token with logit
 *       >= t* is kept (ties included). P = 1 switches the filter off.
 *   R4  acceptance is the strict test u < a.
 *   R5  q(d) = 0: a = 1 if p(d) > 0 else 0 (flag Q_ZERO).
 *   R6  residual mass R <= 0: sample from p itself (flag RESID_FALLBACK).
 *   R7  sampling is the inverse CDF in ascending token id: the smallest v whose running sum
 *       exceeds u*W; if rounding leaves none, the largest v with positive weight.
 *   R8  uniforms: Philox4x32-10, key = (seed low 32, seed high 32), counter = (id, pos,
 *       purpose, 0), u = (word0 >> 8) * 2^-24. pos is the absolute slot of the token being
 *       decided: L+k for the test and residual at draft k, L+gamma+1 for the bonus.
 *   R9  argmax ties go to the lowest token id.
 *   R10 committed length after a chain round is L + lead_slots + n_acc.
 *   R11 tree walk: greedy, lowest node index among matching siblings; the extra token is
 *       the argmax at the stopping node and is emitted only if that node has a row.
 *   R12 tree KV commit copies, in depth order, slot base+path[j] to slot base+j,
 *       base = L + lead_slots - 1, for every layer, K and V, and head.
 *   R18 top-k is a value threshold too: t_k is the K-th largest logit counting repeats, and
 *       every token with logit >= t_k is kept (ties at the boundary included, so the kept
 *       set can exceed K). K <= 0 or K >= V switches it off. Top-k comes first and top-p
 *       then applies to the top-k law (mass measured within the top-k set), in the order
 *       the pages name them ([KV] §4, "top-k/top-p"); both apply to p and q alike.
 *   R19 early stop ([KV] §5: EOS and the length cap end a round early): the round's
 *       emitted tokens are the accepted drafts in order, then the correction or bonus token.
 *       Emission stops after the first emitted token equal to the sequence's EOS id
 *       (flag EOS), and after max_emit tokens (flag LEN_CAP when that cuts the round short).
 *       A stop inside the accepted drafts ends the round there: later positions are not
 *       tested and no correction or bonus token is drawn; n_acc counts the emitted drafts
 *       and the committed length follows R10 with that n_acc. eos < 0 and max_emit <= 0
 *       switch the respective stop off.
 *   R20 tree drafting ([TR] tree configuration and draft steps): an expanded node's children
 *       are the K tokens of largest draft logit, ties to the lower token id (a rank cut:
 *       exactly K children, as the page's node counts 6 + 4 + 2 require). A node's path
 *       probability is the product of the draft softmax probabilities (temperature 1, no
 *       filter) of the tokens on its path below the root. The nodes expanded at the next
 *       step are the top_head[s+1] nodes of the newest layer with the largest path
 *       probability, ties to the lower node index, in descending order; the j-th of them
 *       gets top_k_spec[s+1][j] children. Nodes are numbered root 0, then layer by layer,
 *       within a layer by the rank of the parent and then of the child. Target rows belong
 *       to the expanded nodes in expansion order (root row 0). The ancestor mask lets node
 *       i see node j iff j is i or an ancestor of i, and a node's position is the root's
 *       plus its depth ([LI] §10.6.3, Table 10-17). The selection compares the fp64 path
 *       log-probabilities themselves; equal values go to the lower node index.
 *   R22 paged KV commit ([LI] §10.6.3: after a rejection the cache length is cut back, and a
 *       paged cache releases the blocks it no longer needs): logical slot s of sequence b
 *       lives in physical block block_table[b][s / block_size] at offset s % block_size.
 *       The path copy of R12 runs through that mapping; then the committed length becomes
 *       L' = L + lead_slots + D, and every mapped logical block at or past ceil(L' /
 *       block_size) is released: its id is appended to the free list, sequences in order and
 *       each sequence's blocks in logical order, and its table entry becomes -1. A sequence
 *       with a copied slot outside the table or in an unmapped block, or whose L' needs more
 *       blocks than the table has, or whose table holds a block id >= num_blocks among the
 *       blocks the release would free, is flagged SLOT_OOB and left untouched. A released
 *       block that finds the free list full (free_capacity ids) stays in the table and the
 *       sequence is flagged FREE_FULL (a pool that keeps every id once never gets there).
 *   R23 n-gram prompt lookup ([KV] variants, n-gram and prefix matching; [LI] §10.6.3,
 *       model-free drafts and the ngram method's prompt_lookup_min / prompt_lookup_max):
 *       the suffix of length n of the history h[0..len) is looked up among the earlier
 *       occurrences h[i..i+n), i < len - n; the longest n in [min, max] with an occurrence
 *       wins, and for it the latest occurrence (largest i). The drafts are the tokens that
 *       follow it, h[i+n .. min(i+n+gamma, len)); no occurrence for any n gives no draft.
 *   R24 a drafter without a law (the n-gram lookup above) proposes each draft with certainty:
 *       with no draft rows and T > 0 the draft law q_k is the point mass at d_k, so
 *       a = min(1, p_k(d_k)) and the residual max(0, p_k - q_k) is p_k with d_k removed
 *       ([KV] §4 eq. a(x) and eq. p'(x) with that q). Filters leave a point mass as it is.
 */
#include <math.h>
#include <stdint.h>
#include <float.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Sequence flag bits reported by the oracle (same meaning as the library's, defined here
 * independently). */
#define OF_BAD_TOKEN 1
#define OF_Q_ZERO 2
#define OF_RESID_FALLBACK 4
#define OF_NO_ROW 8
#define OF_SLOT_OOB 16
#define OF_BAD_TREE 32
#define OF_BAD_PARAM 128
#define OF_EOS 256
#define OF_LEN_CAP 512
#define OF_FREE_FULL 1024

#define PURPOSE_ACCEPT 0u
#define PURPOSE_RESIDUAL 1u
#define PURPOSE_BONUS 2u

/* ------------------------------------------------------------------------------------ */
/* Philox4x32-10: J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random numbers: as easy */
/* as 1, 2, 3", SC'11. Ten rounds of the 4x32 Philox S-box with the Weyl key schedule.      */
/* ------------------------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u; /* round multipliers */
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u; /* key increments    */
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t prod0 = (uint64_t)M0 * (uint64_t)c0;
    uint64_t prod1 = (uint64_t)M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += W0;
    k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Reading R8. */
double oracle_uniform(uint64_t seed, uint32_t id, uint32_t pos, uint32_t purpose) {
  uint32_t ctr[4] = {id, pos, purpose, 0u};
  uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

/* bf16 bit pattern -> double, exactly (bf16 is the top half of an IEEE binary32). */
double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------------------ */
/* The per-row law: temperature softmax and top-p ([KV] §4: the law actually sampled,      */
/* after temperature and top-k/top-p, is the one the acceptance rule must use; [LI] §10.6.1 */
/* greedy special case). Readings R1-R3, R9.                                               */
/* ------------------------------------------------------------------------------------ */
typedef struct {
  int argmax;          /* lowest token id holding the maximum logit            */
  int nucleus;         /* |S|                                                  */
  double m;            /* maximum logit                                        */
  double tk;           /* top-k threshold logit; -inf when top-k is off        */
  double tstar;        /* kept-set threshold logit; -inf when no filter is on  */
  double z;            /* sum over all tokens of exp((l-m)/T)                  */
  double zs;           /* the same sum over S                                  */
  double topp_margin;  /* min(|mass(S)-P|, |mass(S minus lowest group)-P|),
                          masses relative to the top-k set                     */
} orow_t;

static int cmp_desc(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x < y) - (x > y);
}

/* Fills pi[0..V) with the filtered, normalised law of one bf16 logits row (top-k K, then
 * top-p P on the top-k law; readings R1-R3, R18). scratch must hold V doubles. Returns 0,
 * or -1 if the row has no finite maximum. */
int oracle_dist(const uint16_t* row, int V, double T, double P, int K, double* pi,
                double* scratch, orow_t* info) {
  double m = -INFINITY;
  int am = 0;
  for (int v = 0; v < V; ++v) {
    double l = oracle_bf16_to_double(row[v]);
    if (l > m) { m = l; am = v; }
  }
  info->argmax = am;
  info->m = m;
  info->tk = -INFINITY;
  info->tstar = -INFINITY;
  info->topp_margin = INFINITY;
  if (!(m > -INFINITY) || isinf(m) || isnan(m)) return -1;
  if (T == 0.0) { /* greedy: the target law is one-hot at the argmax */
    for (int v = 0; v < V; ++v) pi[v] = 0.0;
    pi[am] = 1.0;
    info->nucleus = 1;
    info->z = info->zs = 1.0;
    return 0;
  }
  double z = 0.0;
  for (int v = 0; v < V; ++v) {
    pi[v] = exp((oracle_bf16_to_double(row[v]) - m) / T);
    z += pi[v];
  }
  info->z = z;
  const int use_k = K >= 1 && K < V, use_p = P < 1.0;
  double tstar = -INFINITY;
  if (use_k || use_p) {
    for (int v = 0; v < V; ++v) scratch[v] = oracle_bf16_to_double(row[v]);
    qsort(scratch, (size_t)V, sizeof(double), cmp_desc);
    /* Top-k: the K-th largest value, repeats counted; the top-k set is every token at or
     * above it, and its mass zk is the reference mass for top-p. */
    double tk = -INFINITY, zk = z;
    if (use_k) {
      tk = scratch[K - 1];
      zk = 0.0;
      for (int v = 0; v < V; ++v)
        if (oracle_bf16_to_double(row[v]) >= tk) zk += pi[v];
    }
    info->tk = tk;
    tstar = tk;
    if (use_p) {
      /* Walk the distinct logit values of the top-k set from the largest down; the first
       * value at which the mass of all tokens at or above it reaches P * zk is the
       * threshold. */
      double cum = 0.0, above = 0.0;
      int found = 0;
      for (int i = 0; i < V && scratch[i] >= tk; ++i) {
        cum += exp((scratch[i] - m) / T);
        int group_end = (i + 1 == V) || (scratch[i + 1] != scratch[i]);
        if (!group_end) continue;
        if (cum / zk >= P) {
          tstar = scratch[i];
          double d1 = fabs(cum / zk - P), d2 = fabs(above / zk - P);
          info->topp_margin = d1 < d2 ? d1 : d2;
          found = 1;
          break;
        }
        above = cum;
      }
      if (!found) { /* rounding kept the total just below P: keep the whole top-k set */
        tstar = use_k ? tk : scratch[V - 1];
        info->topp_margin = 0.0;
      }
    }
  }
  info->tstar = tstar;
  double zs = 0.0;
  int count = 0;
  for (int v = 0; v < V; ++v) {
    if (oracle_bf16_to_double(row[v]) >= tstar) { zs += pi[v]; ++count; }
    else pi[v] = 0.0;
  }
  info->zs = zs;
  info->nucleus = count;
  for (int v = 0; v < V; ++v) pi[v] /= zs;
  return 0;
}

/* Inverse-CDF draw from non-negative weights (reading R7). *margin receives the distance of
 * the uniform u from the nearer of the two decision boundaries that bracket the chosen
 * token, in u's own units: min(u - C_{y-1}/W, C_y/W - u). */
int oracle_sample(const double* w, int V, double u, double* margin) {
  double W = 0.0;
  for (int v = 0; v < V; ++v) W += w[v];
  double x = u * W, c = 0.0;
  for (int v = 0; v < V; ++v) {
    double prev = c;
    c += w[v];
    if (c > x) {
      double a = x - prev, b = c - x;
      if (margin) *margin = (a < b ? a : b) / W;
      return v;
    }
  }
  if (margin) *margin = 0.0;
  for (int v = V - 1; v >= 0; --v)
    if (w[v] > 0.0) return v;
  return 0;
}

/* One verified position on probability vectors ([KV] §4 eq. a(x) and eq. p'(x); [LI]
 * §10.6.1 steps 3-4; [GL] exact acceptance and its q=0 / vanishing-residual cases).
 * Returns 1 if the draft token d is accepted, else 0 with *token set to the residual draw.
 * info[0] = a, info[1] = R (NaN when accepted), info[2] = the drawn token's probability
 * under the residual law (NaN when accepted), info[3] = smallest decision margin: the
 * distance of a uniform from its decision boundary (|u - a|, and the draw's margin), 0 when
 * R < 1e-5. */
int oracle_position_step(const double* p, const double* q, int V, int d, double u_acc,
                         double u_res, int* token, int* flags, double* r_scratch,
                         double info[4]) {
  double pd = p[d], qd = q[d], a;
  if (qd > 0.0) a = fmin(1.0, pd / qd);
  else { a = pd > 0.0 ? 1.0 : 0.0; *flags |= OF_Q_ZERO; }
  info[0] = a;
  info[3] = fabs(u_acc - a);
  if (u_acc < a) { info[1] = NAN; info[2] = NAN; return 1; }
  double R = 0.0;
  for (int v = 0; v < V; ++v) {
    double r = p[v] - q[v];
    r_scratch[v] = r > 0.0 ? r : 0.0;
    R += r_scratch[v];
  }
  double sm;
  int y;
  if (R > 0.0) {
    y = oracle_sample(r_scratch, V, u_res, &sm);
    info[2] = r_scratch[y] / R;
  } else {
    *flags |= OF_RESID_FALLBACK;
    y = oracle_sample(p, V, u_res, &sm);
    info[2] = p[y];
  }
  info[1] = R;
  if (sm < info[3]) info[3] = sm;
  if (R < 1e-5) info[3] = 0.0; /* a vanishing residual is itself a boundary case */
  *token = y;
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Chain verification over a ragged batch ([LI] §10.6.1 steps 1-5; [KV] §5 and §6;        */
/* [LI] §10.6.3 verify shape logits[B, gamma+1, n_vocab] and per-request start points).    */
/* Row layout: target row of (b,k), k=1..gamma_b+1, is cu_gamma[b]+b+k-1; draft row of     */
/* (b,k), k=1..gamma_b, is cu_gamma[b]+k-1.                                                */
/* ------------------------------------------------------------------------------------ */
int oracle_verify_chain(int B, int V, int row_stride, const uint16_t* target,
                        const uint16_t* draft, const int32_t* cu_gamma,
                        const int32_t* draft_tokens, const float* temperature,
                        const float* top_p, const int32_t* top_k, const int32_t* eos_token,
                        const int32_t* max_emit, const uint32_t* seq_id,
                        const int32_t* committed_len_in, int lead_slots, uint64_t seed,
                        const float* uniform_override, int32_t* out_tokens,
                        int32_t* num_accepted, int32_t* num_emitted, int32_t* committed_len_out,
                        int32_t* seq_flags, double* probe_rows, double* probe_seq,
                        double* margin_out, double* row_margin, double* draw_margin,
                        int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int failed = 0;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    double* scratch = (double*)malloc(sizeof(double) * (size_t)V);
    if (!p || !q || !r || !scratch) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
      if (failed) continue;
      const int g = cu_gamma[b + 1] - cu_gamma[b];
      const int trow0 = cu_gamma[b] + b, drow0 = cu_gamma[b];
      const int L = committed_len_in[b];
      const uint32_t id = seq_id ? seq_id[b] : (uint32_t)b;
      const double T = (double)temperature[b];
      const double P = top_p ? (double)top_p[b] : 1.0;
      const int K = top_k ? top_k[b] : 0;
      const int eos = eos_token ? eos_token[b] : -1;
      const int cap = max_emit ? max_emit[b] : 0;
      int flags = 0, n_acc = 0, y = -1;
      /* margin: smallest distance to a decision boundary among the acceptance tests and the
       * top-p cuts of the rows they use; dmargin: the same for the final draw. */
      double margin = INFINITY, dmargin = INFINITY, R_out = NAN, py_out = NAN;
      for (int k = 0; k < g; ++k) {
        double* pr = probe_rows ? probe_rows + 3 * (size_t)(drow0 + k) : NULL;
        if (pr) pr[0] = pr[1] = pr[2] = NAN;
        if (row_margin) row_margin[2 * (size_t)(drow0 + k)] = row_margin[2 * (size_t)(drow0 + k) + 1] = INFINITY;
      }
      if (draw_margin) draw_margin[2 * b] = draw_margin[2 * b + 1] = INFINITY;
      int bad = 0;
      for (int k = 0; k < g; ++k) {
        int d = draft_tokens[drow0 + k];
        if (d < 0 || d >= V) bad = 1;
      }
      if (bad) flags |= OF_BAD_TOKEN;
      /* T: 0 (greedy) or 2^-126 <= T <= 2^126, where 1/T is a normal binary32 */
      if (!(T == 0.0 || (T >= (double)FLT_MIN && T <= ldexp(1.0, 126))) ||
          !(P > 0.0 && P <= 1.0)) {
        flags |= OF_BAD_PARAM;
        bad = 1;
      }
      if (bad) {
        num_accepted[b] = 0;
        if (num_emitted) num_emitted[b] = 0;
        committed_len_out[b] = L;
        if (seq_flags) seq_flags[b] = flags;
        if (probe_seq) { probe_seq[2 * b] = NAN; probe_seq[2 * b + 1] = NAN; }
        if (margin_out) margin_out[2 * b] = margin_out[2 * b + 1] = INFINITY;
        continue;
      }
      orow_t ip, iq;
      int stopped = 0, drawn = 1; /* drawn: the round ends with a correction/bonus token */
      for (int k = 1; k <= g && !stopped; ++k) {
        const uint16_t* trow = target + (size_t)(trow0 + k - 1) * row_stride;
        const int d = draft_tokens[drow0 + k - 1];
        double* pr = probe_rows ? probe_rows + 3 * (size_t)(drow0 + k - 1) : NULL;
        const size_t ovr = (size_t)(trow0 + k - 1) * 2;
        if (T == 0.0) {
          /* Greedy: accept iff the draft token is the target argmax; at the first mismatch
           * the target's argmax is emitted ([LI] §10.6.1 greedy special case; [KV] §4). */
          oracle_dist(trow, V, 0.0, 1.0, 0, p, scratch, &ip);
          int acc = (d == ip.argmax);
          if (pr) { pr[0] = acc ? 1.0 : 0.0; pr[1] = NAN; pr[2] = acc ? 1.0 : 0.0; }
          if (acc) {
            n_acc = k;
            /* reading R19: an emitted EOS, or the emission cap, ends the round here */
            if (d == eos) { flags |= OF_EOS; stopped = 1; drawn = 0; break; }
            if (cap > 0 && k >= cap) { flags |= OF_LEN_CAP; stopped = 1; drawn = 0; break; }
            continue;
          }
          y = ip.argmax;
          py_out = 1.0;
          stopped = 1;
          break;
        }
        oracle_dist(trow, V, T, P, K, p, scratch, &ip);
        if (ip.topp_margin < margin) margin = ip.topp_margin;
        double cut_margin = ip.topp_margin; /* the top-p cuts of this position's rows */
        if (draft) {
          const uint16_t* drow = draft + (size_t)(drow0 + k - 1) * row_stride;
          oracle_dist(drow, V, T, P, K, q, scratch, &iq);
          if (iq.topp_margin < margin) margin = iq.topp_margin;
          if (iq.topp_margin < cut_margin) cut_margin = iq.topp_margin;
        } else { /* reading R24: the point mass at the draft token */
          for (int v = 0; v < V; ++v) q[v] = 0.0;
          q[d] = 1.0;
        }
        double u_acc = uniform_override ? (double)uniform_override[ovr]
                                        : oracle_uniform(seed, id, (uint32_t)(L + k), PURPOSE_ACCEPT);
        double u_res = uniform_override ? (double)uniform_override[ovr + 1]
                                        : oracle_uniform(seed, id, (uint32_t)(L + k), PURPOSE_RESIDUAL);
        double info[4];
        int tok = -1;
        int acc = oracle_position_step(p, q, V, d, u_acc, u_res, &tok, &flags, r, info);
        if (pr) { pr[0] = p[d]; pr[1] = q[d]; pr[2] = info[0]; }
        double am = fabs(u_acc - info[0]);
        if (am < margin) margin = am;
        if (row_margin) {
          row_margin[2 * (size_t)(drow0 + k - 1)] = am;
          row_margin[2 * (size_t)(drow0 + k - 1) + 1] = cut_margin;
        }
        if (acc) {
          n_acc = k;
          if (d == eos) { flags |= OF_EOS; stopped = 1; drawn = 0; break; }
          if (cap > 0 && k >= cap) { flags |= OF_LEN_CAP; stopped = 1; drawn = 0; break; }
          continue;
        }
        dmargin = info[3];
        if (draw_margin) draw_margin[2 * b + 1] = info[3];
        y = tok;
        R_out = info[1];
        py_out = info[2];
        stopped = 1;
      }
      if (!stopped) {
        /* Every draft accepted: one more token from p_{gamma+1} ([LI] §10.6.1 step 5;
         * [KV] §5 bonus token). */
        const uint16_t* trow = target + (size_t)(trow0 + g) * row_stride;
        const size_t ovr = (size_t)(trow0 + g) * 2;
        if (T == 0.0) {
          oracle_dist(trow, V, 0.0, 1.0, 0, p, scratch, &ip);
          y = ip.argmax;
          py_out = 1.0;
        } else {
          oracle_dist(trow, V, T, P, K, p, scratch, &ip);
          if (ip.topp_margin < dmargin) dmargin = ip.topp_margin;
          double u = uniform_override ? (double)uniform_override[ovr + 1]
                                      : oracle_uniform(seed, id, (uint32_t)(L + g + 1), PURPOSE_BONUS);
          double sm;
          y = oracle_sample(p, V, u, &sm);
          if (sm < dmargin) dmargin = sm;
          if (draw_margin) {
            draw_margin[2 * b] = ip.topp_margin;
            draw_margin[2 * b + 1] = sm;
          }
          py_out = p[y];
        }
        n_acc = g;
      }
      for (int k = 0; k < n_acc; ++k) out_tokens[trow0 + k] = draft_tokens[drow0 + k];
      if (drawn) {
        out_tokens[trow0 + n_acc] = y;
        if (y == eos) flags |= OF_EOS;
      }
      num_accepted[b] = n_acc;
      if (num_emitted) num_emitted[b] = n_acc + drawn;
      committed_len_out[b] = L + lead_slots + n_acc; /* reading R10 ([KV] §6 pointer) */
      if (seq_flags) seq_flags[b] = flags;
      if (probe_seq) { probe_seq[2 * b] = R_out; probe_seq[2 * b + 1] = py_out; }
      if (margin_out) {
        margin_out[2 * b] = margin;
        margin_out[2 * b + 1] = dmargin < margin ? dmargin : margin;
      }
    }
    free(p); free(q); free(r); free(scratch);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------------------ */
/* Greedy tree verification ([TR] validation and path walk; [LI] §10.6.3 tree drafts).     */
/* Reading R11. parent/node_row are [num_nodes] per sequence (tree_stride elements apart,  */
/* 0 = one topology for the batch); node_token is [B][num_nodes]; rows are                  */
/* [B][rows_per_seq][row_stride].                                                          */
/* ------------------------------------------------------------------------------------ */
int oracle_verify_tree(int B, int V, int row_stride, int rows_per_seq, int num_nodes,
                       int max_depth, int tree_stride, const uint16_t* logits,
                       const int32_t* parent, const int32_t* node_row,
                       const int32_t* node_token, int32_t* path_nodes, int32_t* path_len,
                       int32_t* out_tokens, int32_t* num_emitted, int32_t* seq_flags,
                       int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    const int32_t* par = parent + (size_t)b * tree_stride;
    const int32_t* nrow = node_row + (size_t)b * tree_stride;
    const int32_t* tok = node_token + (size_t)b * num_nodes;
    int flags = 0, ok = (par[0] == -1);
    for (int i = 1; i < num_nodes; ++i)
      if (par[i] < 0 || par[i] >= i) ok = 0;
    for (int i = 0; i < num_nodes; ++i)
      if (nrow[i] < -1 || nrow[i] >= rows_per_seq) ok = 0;
    for (int j = 0; j < max_depth; ++j) path_nodes[(size_t)b * max_depth + j] = -1;
    if (!ok) {
      path_len[b] = 0;
      num_emitted[b] = 0;
      if (seq_flags) seq_flags[b] = OF_BAD_TREE;
      continue;
    }
    int v = 0, D = 0, extra = -1;
    for (;;) {
      if (nrow[v] < 0) { flags |= OF_NO_ROW; break; }
      const uint16_t* row = logits + ((size_t)b * rows_per_seq + nrow[v]) * row_stride;
      int am = 0;
      double best = -INFINITY;
      for (int t = 0; t < V; ++t) {
        double l = oracle_bf16_to_double(row[t]);
        if (l > best) { best = l; am = t; }
      }
      int child = -1;
      if (D < max_depth)
        for (int i = v + 1; i < num_nodes; ++i)
          if (par[i] == v && tok[i] == am) { child = i; break; }
      if (child < 0) { extra = am; break; }
      path_nodes[(size_t)b * max_depth + D] = child;
      out_tokens[(size_t)b * (max_depth + 1) + D] = tok[child];
      ++D;
      v = child;
    }
    path_len[b] = D;
    if (extra >= 0) out_tokens[(size_t)b * (max_depth + 1) + D] = extra;
    num_emitted[b] = D + (extra >= 0 ? 1 : 0);
    if (seq_flags) seq_flags[b] = flags;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* KV commit of an accepted path ([KV] §6: reserved slots and one committed-length pointer, */
/* the same boundary in every layer; [LI] §10.6.3 cache truncation after a rejection).     */
/* Reading R12. Caches are host arrays of uint16 (bf16 bits); layer l's K cache starts at  */
/* k_cache[l]. Element (b, slot, head, e) sits at b*seq_stride + slot*slot_stride +        */
/* head*head_stride + e.                                                                   */
/* ------------------------------------------------------------------------------------ */
int oracle_kv_commit(int B, int num_layers, int num_kv_heads, int head_dim,
                     uint16_t* const* k_cache, uint16_t* const* v_cache, int64_t seq_stride,
                     int64_t slot_stride, int64_t head_stride, int slot_capacity,
                     int lead_slots, int max_depth, const int32_t* path_nodes,
                     const int32_t* path_len, int32_t* committed_len, int32_t* seq_flags) {
  for (int b = 0; b < B; ++b) {
    const int L = committed_len[b], D = path_len[b];
    const int base = L + lead_slots - 1;
    int ok = (D >= 0 && D <= max_depth);
    for (int j = 0; ok && j < D; ++j) {
      int node = path_nodes[(size_t)b * max_depth + j];
      if (node < 1 || base + node >= slot_capacity || base + j + 1 >= slot_capacity) ok = 0;
    }
    if (!ok || base + D + 1 > slot_capacity || base < -1) {
      if (seq_flags) seq_flags[b] |= OF_SLOT_OOB;
      continue;
    }
    for (int j = 1; j <= D; ++j) {
      const int src = base + path_nodes[(size_t)b * max_depth + j - 1], dst = base + j;
      if (src == dst) continue;
      for (int l = 0; l < num_layers; ++l)
        for (int kv = 0; kv < 2; ++kv) {
          uint16_t* c = kv ? v_cache[l] : k_cache[l];
          for (int h = 0; h < num_kv_heads; ++h)
            memmove(c + b * seq_stride + (int64_t)dst * slot_stride + h * head_stride,
                    c + b * seq_stride + (int64_t)src * slot_stride + h * head_stride,
                    sizeof(uint16_t) * (size_t)head_dim);
        }
    }
    committed_len[b] = L + lead_slots + D;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Tree drafting ([TR] sections on the tree configuration and on the three draft steps;   */
/* [LI] §10.6.3 tree drafts and Table 10-17). Reading R20.                                 */
/* rows holds the draft rows of steps 0..depth-1 in order; step s contributes B*top_head[s] */
/* rows, row (b, j) being the draft model's logits after the j-th node expanded at step s.  */
/* top_k_spec concatenates top_k_spec[s][0..top_head[s]) over s. Per sequence (tree_stride  */
/* entries apart): parent, node_token, node_row, node_logp (natural log of the path        */
/* probability), position_ids, and ancestor[i*tree_stride + j] = 1 iff node i sees node j. */
/* expand[(s*B + b)*expand_stride + j] = the j-th node expanded at step s; select_margin   */
/* [s*B + b] = the smallest nonzero gap between neighbouring path log-probabilities among  */
/* the first top_head[s]+1 of the ranked layer (+inf for step 0: the root is fixed).       */
/* Returns 0, or -1 for an invalid configuration.                                          */
/* ------------------------------------------------------------------------------------ */
typedef struct {
  double l;
  int id;
} otok_t;

static int cmp_tok(const void* a, const void* b) {
  const otok_t* x = (const otok_t*)a;
  const otok_t* y = (const otok_t*)b;
  if (x->l != y->l) return x->l > y->l ? -1 : 1;
  return (x->id > y->id) - (x->id < y->id);
}

typedef struct {
  double lp;
  int node;
} onode_t;

static int cmp_node(const void* a, const void* b) {
  const onode_t* x = (const onode_t*)a;
  const onode_t* y = (const onode_t*)b;
  if (x->lp != y->lp) return x->lp > y->lp ? -1 : 1;
  return (x->node > y->node) - (x->node < y->node);
}

int oracle_tree_draft(int B, int V, int row_stride, int depth, const int32_t* top_head,
                      const int32_t* top_k_spec, const uint16_t* rows,
                      const int32_t* root_token, const int32_t* pos_base, int tree_stride,
                      int32_t* parent, int32_t* node_token, int32_t* node_row,
                      double* node_logp, int32_t* position_ids, uint8_t* ancestor,
                      int32_t* expand, int expand_stride, double* select_margin,
                      int nthreads) {
  /* configuration: the root alone at step 0, every expansion within its layer */
  if (depth < 1 || top_head[0] != 1) return -1;
  int nodes = 1, kofs = 0, layer = 1;
  for (int s = 0; s < depth; ++s) {
    if (top_head[s] < 1 || top_head[s] > layer || top_head[s] > expand_stride) return -1;
    layer = 0;
    for (int j = 0; j < top_head[s]; ++j) {
      const int k = top_k_spec[kofs + j];
      if (k < 1 || k > V) return -1;
      layer += k;
    }
    kofs += top_head[s];
    nodes += layer;
  }
  if (nodes > tree_stride) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    otok_t* tok = (otok_t*)malloc(sizeof(otok_t) * (size_t)V);
    onode_t* lay = (onode_t*)malloc(sizeof(onode_t) * (size_t)tree_stride);
#pragma omp for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
      int32_t* par = parent + (size_t)b * tree_stride;
      int32_t* ntok = node_token + (size_t)b * tree_stride;
      int32_t* nrow = node_row + (size_t)b * tree_stride;
      double* lp = node_logp + (size_t)b * tree_stride;
      int32_t* pos = position_ids + (size_t)b * tree_stride;
      uint8_t* anc = ancestor + (size_t)b * tree_stride * tree_stride;
      for (int i = 0; i < tree_stride; ++i) {
        par[i] = -1;
        ntok[i] = -1;
        nrow[i] = -1;
        lp[i] = -INFINITY;
        pos[i] = -1;
      }
      memset(anc, 0, (size_t)tree_stride * tree_stride);
      /* the root: the round's last confirmed token */
      ntok[0] = root_token[b];
      lp[0] = 0.0;
      pos[0] = pos_base ? pos_base[b] : 0;
      nrow[0] = 0;
      int32_t exp_now[256];
      exp_now[0] = 0;
      int n = 1;          /* nodes so far            */
      int rows_done = 0;  /* rows before this step's */
      size_t row_base = 0;
      int ko = 0;
      for (int s = 0; s < depth; ++s) {
        const int h = top_head[s];
        for (int j = 0; j < h; ++j) expand[((size_t)s * B + b) * expand_stride + j] = exp_now[j];
        if (s == 0) select_margin[b] = INFINITY;
        const int first = n; /* first node of the new layer */
        for (int j = 0; j < h; ++j) {
          const int pnode = exp_now[j];
          const uint16_t* row = rows + (row_base + (size_t)b * h + j) * row_stride;
          /* log of the draft softmax: log pi(v) = l_v - m - log(sum_u exp(l_u - m)) */
          double m = -INFINITY;
          for (int v = 0; v < V; ++v) {
            const double l = oracle_bf16_to_double(row[v]);
            if (l > m) m = l;
          }
          double z = 0.0;
          for (int v = 0; v < V; ++v) z += exp(oracle_bf16_to_double(row[v]) - m);
          const double logz = m + log(z);
          /* the K largest logits, ties to the lower id: sort all tokens */
          for (int v = 0; v < V; ++v) {
            tok[v].l = oracle_bf16_to_double(row[v]);
            tok[v].id = v;
          }
          qsort(tok, (size_t)V, sizeof(otok_t), cmp_tok);
          const int K = top_k_spec[ko + j];
          for (int r = 0; r < K; ++r) {
            const int c = n++;
            par[c] = pnode;
            ntok[c] = tok[r].id;
            lp[c] = lp[pnode] + (tok[r].l - logz);
            pos[c] = pos[pnode] + 1;
          }
        }
        ko += h;
        row_base += (size_t)B * h;
        rows_done += h;
        if (s + 1 < depth) {
          /* the next step expands the newest layer's most probable nodes */
          const int cnt = n - first, hn = top_head[s + 1];
          for (int i = 0; i < cnt; ++i) {
            lay[i].lp = lp[first + i];
            lay[i].node = first + i;
          }
          qsort(lay, (size_t)cnt, sizeof(onode_t), cmp_node);
          double mg = INFINITY;
          for (int i = 0; i < hn && i + 1 < cnt; ++i) {
            const double d = fabs(lay[i].lp - lay[i + 1].lp);
            if (d > 0.0 && d < mg) mg = d;
          }
          select_margin[(size_t)(s + 1) * B + b] = mg;
          for (int j = 0; j < hn; ++j) {
            exp_now[j] = lay[j].node;
            nrow[lay[j].node] = rows_done + j;
          }
        }
      }
      /* ancestor mask: each node sees itself and every node on its path to the root */
      for (int i = 0; i < n; ++i)
        for (int a = i; a >= 0; a = par[a]) anc[(size_t)i * tree_stride + a] = 1;
    }
    free(tok);
    free(lay);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Paged KV commit and release ([LI] §10.6.3 cache truncation and block release; [KV] §6   */
/* committed-length pointer). Reading R22. Layer l's K cache starts at k_cache[l]; element */
/* (physical block p, offset o, head h, e) sits at p*block_stride + o*slot_stride +        */
/* h*head_stride + e. block_table is [B][max_blocks] (-1 = unmapped); free_list holds      */
/* free_count[0] ids and receives the released ones after them.                            */
/* ------------------------------------------------------------------------------------ */
static int64_t paged_off(const int32_t* bt, int block_size, int slot, int64_t block_stride,
                         int64_t slot_stride) {
  return (int64_t)bt[slot / block_size] * block_stride + (int64_t)(slot % block_size) * slot_stride;
}

int oracle_kv_commit_paged(int B, int num_layers, int num_kv_heads, int head_dim,
                           uint16_t* const* k_cache, uint16_t* const* v_cache, int block_size,
                           int max_blocks, int num_blocks, int64_t block_stride,
                           int64_t slot_stride, int64_t head_stride, int lead_slots,
                           int max_depth, int32_t* block_table, const int32_t* path_nodes,
                           const int32_t* path_len, int32_t* committed_len, int32_t* free_list,
                           int free_capacity, int32_t* free_count, int32_t* seq_flags) {
  /* the count of ids already listed, taken within [0, free_capacity] */
  if (free_count[0] < 0) free_count[0] = 0;
  if (free_count[0] > free_capacity) free_count[0] = free_capacity;
  for (int b = 0; b < B; ++b) {
    int32_t* bt = block_table + (size_t)b * max_blocks;
    const int L = committed_len[b], D = path_len[b];
    const int base = L + lead_slots - 1;
    const int64_t new_len = (int64_t)L + lead_slots + D;
    int ok = D >= 0 && D <= max_depth && base >= -1 &&
             (new_len + block_size - 1) / block_size <= max_blocks;
    /* every slot a copy touches must be mapped */
    for (int j = 1; ok && j <= D; ++j) {
      const int node = path_nodes[(size_t)b * max_depth + j - 1];
      if (node < 1) { ok = 0; break; }
      const int src = base + node, dst = base + j;
      if (src == dst) continue;
      const int slots[2] = {src, dst};
      for (int q = 0; q < 2; ++q) {
        const int sl = slots[q];
        if (sl < 0 || sl >= max_blocks * block_size) { ok = 0; break; }
        const int pb = bt[sl / block_size];
        if (pb < 0 || pb >= num_blocks) { ok = 0; break; }
      }
    }
    /* every block the release would free must be a valid id */
    const int need = ok ? (int)((new_len + block_size - 1) / block_size) : max_blocks;
    for (int lb = need; ok && lb < max_blocks; ++lb)
      if (bt[lb] >= num_blocks) ok = 0;
    if (!ok) {
      if (seq_flags) seq_flags[b] |= OF_SLOT_OOB;
      continue;
    }
    for (int j = 1; j <= D; ++j) {
      const int src = base + path_nodes[(size_t)b * max_depth + j - 1], dst = base + j;
      if (src == dst) continue;
      const int64_t so = paged_off(bt, block_size, src, block_stride, slot_stride);
      const int64_t d_o = paged_off(bt, block_size, dst, block_stride, slot_stride);
      for (int l = 0; l < num_layers; ++l)
        for (int kv = 0; kv < 2; ++kv) {
          uint16_t* c = kv ? v_cache[l] : k_cache[l];
          for (int h = 0; h < num_kv_heads; ++h)
            memmove(c + d_o + h * head_stride, c + so + h * head_stride,
                    sizeof(uint16_t) * (size_t)head_dim);
        }
    }
    committed_len[b] = (int32_t)new_len;
    for (int lb = need; lb < max_blocks; ++lb) {
      if (bt[lb] < 0) continue;
      if (free_count[0] >= free_capacity) { /* no room: the block stays in the table */
        if (seq_flags) seq_flags[b] |= OF_FREE_FULL;
        continue;
      }
      free_list[free_count[0]++] = bt[lb];
      bt[lb] = -1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* n-gram prompt lookup ([KV] variants section on n-gram / prefix matching; [LI] §10.6.3   */
/* model-free drafts, prompt_lookup_min / prompt_lookup_max). Reading R23. tokens is       */
/* [B][stride]; drafts is [B][draft_stride] (tokens, then -1); num_drafts, match_len and    */
/* match_pos are [B]. A history length outside [0, stride] is flagged BAD_PARAM (no draft). */
/* ------------------------------------------------------------------------------------ */
int oracle_ngram_draft(int B, int stride, const int32_t* tokens, const int32_t* hist_len,
                       int nmin, int nmax, int gamma, int draft_stride, int32_t* drafts,
                       int32_t* num_drafts, int32_t* match_len, int32_t* match_pos,
                       int32_t* seq_flags) {
  for (int b = 0; b < B; ++b) {
    const int32_t* h = tokens + (size_t)b * stride;
    int len = hist_len[b];
    if (len < 0 || len > stride) {
      if (seq_flags) seq_flags[b] |= OF_BAD_PARAM;
      len = 0;
    }
    int best_n = 0, best_i = -1;
    for (int n = nmax; n >= nmin && best_i < 0; --n) {
      if (n > len - 1) continue; /* an earlier occurrence needs i >= 0 and i < len - n */
      for (int i = len - n - 1; i >= 0; --i) {
        int same = 1;
        for (int k = 0; k < n; ++k)
          if (h[i + k] != h[len - n + k]) { same = 0; break; }
        if (same) { best_n = n; best_i = i; break; }
      }
    }
    int32_t* d = drafts + (size_t)b * draft_stride;
    for (int j = 0; j < draft_stride; ++j) d[j] = -1;
    int nd = 0;
    if (best_i >= 0)
      for (int j = 0; j < gamma && best_i + best_n + j < len; ++j) d[nd++] = h[best_i + best_n + j];
    num_drafts[b] = nd;
    match_len[b] = best_n;
    match_pos[b] = best_i;
  }
  return 0;
}
