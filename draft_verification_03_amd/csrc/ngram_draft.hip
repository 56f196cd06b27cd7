// ngram_draft.hip -- n-gram prompt lookup on gfx950 ("KV Cache 优化（四）", variants section on
// n-gram / prefix matching; "10.6 投机解码" §10.6.3, model-free drafts and the ngram method's
// prompt_lookup_min / prompt_lookup_max).
//
// ngram_draft_kernel -- one 1024-thread workgroup per sequence. For every position p of the
// history below len - 1 (the last token of a possible earlier occurrence, which ends at
// e = p + 1 <= len - 1), m(p) = how many tokens match backwards from p against the history's
// end (h[p-k] == h[len-1-k], k = 0, 1, ..., at most ngram_max). Threads take four positions
// per 16-byte load and compare them with the last token first, so the walk backwards only
// starts on a hit. The best key (min(m, ngram_max), e), among m >= ngram_min, is the longest
// n-gram with an occurrence and, for it, the latest occurrence; the drafts are the tokens from
// e on, at most num_draft of them and none past the history.
#include "spec_device.h"
#include "specv_internal.h"

namespace specv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxN = 64;

struct NgramParams {
  const int32_t* tokens;
  const int32_t* hist_len;
  int32_t* drafts;
  int32_t* num_drafts;
  int32_t* match_len;
  int32_t* match_pos;
  int32_t* flags;
  int32_t stride, nmin, nmax, gamma, draft_stride;
};

__device__ __forceinline__ uint64_t wave_max_u64_shfl(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void ngram_draft_kernel(NgramParams P) {
  __shared__ int32_t s_suf[kMaxN];  // s_suf[k] = h[len - 1 - k]
  __shared__ uint64_t s_best[kWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int32_t* h = P.tokens + (size_t)b * P.stride;
  int len = P.hist_len[b];
  const bool bad = len < 0 || len > P.stride;
  if (bad) len = 0;
  if (tid < P.nmax) s_suf[tid] = tid < len ? h[len - 1 - tid] : -1;
  __syncthreads();
  uint64_t best = 0;
  const int32_t last = len > 0 ? s_suf[0] : 0;
  // positions p = 4q .. 4q + 3 with p <= len - 2
  for (int q = tid; 4 * q <= len - 2; q += kThreads) {
    const int4 v = *reinterpret_cast<const int4*>(h + 4 * q);
    const int32_t t[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 4 * q + r;
      if (p > len - 2 || t[r] != last) continue;
      int m = 1;
      while (m < P.nmax && p - m >= 0 && h[p - m] == s_suf[m]) ++m;
      if (m >= P.nmin) {
        const uint64_t key = ((uint64_t)m << 32) | (uint32_t)(p + 1);
        best = key > best ? key : best;
      }
    }
  }
  best = wave_max_u64_shfl(best);
  if (lane == 0) s_best[wave] = best;
  __syncthreads();
  if (wave != 0) return;
  best = lane < kWaves ? s_best[lane] : 0;
  best = wave_max_u64_shfl(best);
  const int n = (int)(best >> 32);
  const int e = (int)(uint32_t)best;  // the drafts start here
  const int nd = n > 0 ? min(P.gamma, len - e) : 0;
  int32_t* d = P.drafts + (size_t)b * P.draft_stride;
  for (int j = lane; j < P.draft_stride; j += kWave) d[j] = j < nd ? h[e + j] : -1;
  if (lane == 0) {
    P.num_drafts[b] = nd;
    if (P.match_len) P.match_len[b] = n;
    if (P.match_pos) P.match_pos[b] = n > 0 ? e - n : -1;
    if (bad && P.flags) P.flags[b] |= SPEC_FLAG_BAD_PARAM;
  }
}

}  // namespace

hipError_t launch_ngram(const spec_ngram_args& a, hipStream_t st) {
  NgramParams P;
  P.tokens = a.tokens;
  P.hist_len = a.hist_len;
  P.drafts = a.draft_tokens;
  P.num_drafts = a.num_drafts;
  P.match_len = a.match_len;
  P.match_pos = a.match_pos;
  P.flags = a.seq_flags;
  P.stride = a.hist_stride;
  P.nmin = a.ngram_min;
  P.nmax = a.ngram_max;
  P.gamma = a.num_draft;
  P.draft_stride = a.draft_stride;
  hipLaunchKernelGGL(ngram_draft_kernel, dim3((unsigned)a.batch), dim3(kThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace specv
