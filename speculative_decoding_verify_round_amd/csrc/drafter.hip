// Copy-from-the-conversation drafter (n-gram prompt lookup), the history update of a
// multi-round loop, and the token counts the per-row penalties use (gfx950).
//
// "Speculative decoding" (mashbox docs, "Where it runs", --speculation ngram): the
// drafter looks up the last few tokens earlier in the request and proposes the tokens
// that followed them there; it needs no model ("Draft heads and speculative decoding, in
// plain words", drafter table, row "No model at all").  Here: the history's suffix of
// length n, n from n_max down to n_min; the most recent earlier occurrence (largest p
// with p + n < len); the drafts copy what followed it, and a copy that reaches the end
// of the history goes on over the tokens it has just proposed (overlapping copy).  A
// lane without a match gets its anchor as filler guesses, so every round keeps k + 1
// columns and the loop needs no host round trip; the model checks every guess.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

constexpr int kDraftThreads = 256;

// One workgroup per lane.  tokens[l][0] = the anchor (the history's last token),
// tokens[l][1 .. k] = the drafts; n_match[l] = the length of the suffix that matched (0:
// none).  The scan for each n is split over the threads by position; the most recent
// match is a max-reduction, independent of the order in which threads find matches.
__global__ __launch_bounds__(kDraftThreads) void k_ngram_draft(const int32_t* __restrict__ hist,
                                                              const int32_t* __restrict__ hist_len, int max_len, int k,
                                                              int n_max, int n_min, int32_t* __restrict__ tokens,
                                                              int32_t* __restrict__ n_match) {
  __shared__ int best;
  const int l = blockIdx.x, tid = threadIdx.x;
  const int32_t* h = hist + (size_t)l * max_len;
  const int len = min(hist_len[l], max_len);
  int32_t* out = tokens + (size_t)l * (k + 1);
  if (len < 1) {   // no anchor: nothing to check, token 0 columns
    for (int i = tid; i <= k; i += blockDim.x) out[i] = 0;
    if (tid == 0) n_match[l] = 0;
    return;
  }
  const int32_t anchor = h[len - 1];
  int p_found = -1, n_found = 0;
  for (int n = min(n_max, len - 1); n >= n_min; --n) {
    int32_t suf[kMaxNgram];
#pragma unroll
    for (int i = 0; i < kMaxNgram; ++i) suf[i] = i < n ? h[len - n + i] : 0;
    if (tid == 0) best = -1;
    __syncthreads();
    int mine = -1;
    for (int p = tid; p + n < len; p += blockDim.x) {
      bool m = true;
#pragma unroll
      for (int i = 0; i < kMaxNgram; ++i)
        if (i < n) m = m && h[p + i] == suf[i];
      if (m) mine = p;   // p grows along the thread's positions: the last match is its largest
    }
    if (mine >= 0) atomicMax(&best, mine);
    __syncthreads();
    const int b = best;
    __syncthreads();   // every thread has read best before the next n resets it
    if (b >= 0) {
      p_found = b;
      n_found = n;
      break;
    }
  }
  if (tid == 0) {
    out[0] = anchor;
    n_match[l] = n_found;
  }
  // draft i = the token at p + n + i of the history extended by the drafts themselves:
  // with a copy distance q = len - (p + n), that is h[p + n + i mod q]
  const int start = p_found + n_found, q = len - start;
  for (int i = tid; i < k; i += blockDim.x) out[1 + i] = p_found >= 0 ? h[start + i % q] : anchor;
}

// After a round's commit: the lane's committed tokens (out_tokens[l][0 .. c)) are appended
// to its history; the history stops growing at max_len.
__global__ void k_history_append(int32_t* __restrict__ hist, int32_t* __restrict__ hist_len, int max_len,
                                 const int32_t* __restrict__ committed, const int32_t* __restrict__ out_tokens,
                                 int out_stride) {
  const int l = blockIdx.x;
  const int len = min(max(hist_len[l], 0), max_len);
  const int c = min(max(committed[l], 0), out_stride);
  for (int i = threadIdx.x; i < c; i += blockDim.x)
    if (len + i < max_len) hist[(size_t)l * max_len + len + i] = out_tokens[(size_t)l * out_stride + i];
  __syncthreads();
  if (threadIdx.x == 0) hist_len[l] = min(len + c, max_len);
}

// counts[l][t] += 1 for each token of lane l's committed run: one thread per lane, so a
// token that occurs twice in a run is counted twice without atomics.
__global__ void k_counts_add(int32_t* __restrict__ counts, int vocab, int lanes, const int32_t* __restrict__ committed,
                             const int32_t* __restrict__ out_tokens, int out_stride) {
  const int l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= lanes) return;
  const int c = min(max(committed[l], 0), out_stride);
  for (int i = 0; i < c; ++i) {
    const int t = out_tokens[(size_t)l * out_stride + i];
    if (t >= 0 && t < vocab) counts[(size_t)l * vocab + t] += 1;
  }
}

int launch_counts_add(int32_t* counts, int vocab, int lanes, const int32_t* committed, const int32_t* out_tokens,
                      int out_stride, hipStream_t st) {
  hipLaunchKernelGGL(k_counts_add, dim3((lanes + 63) / 64), dim3(64), 0, st, counts, vocab, lanes, committed,
                     out_tokens, out_stride);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_ngram_draft(const int32_t* hist, const int32_t* hist_len, int lanes, int max_len, int k, int n_max,
                       int n_min, int32_t* tokens, int32_t* n_match, hipStream_t st) {
  hipLaunchKernelGGL(k_ngram_draft, dim3(lanes), dim3(kDraftThreads), 0, st, hist, hist_len, max_len, k, n_max, n_min,
                     tokens, n_match);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_history_append(int32_t* hist, int32_t* hist_len, int lanes, int max_len, const int32_t* committed,
                          const int32_t* out_tokens, int out_stride, hipStream_t st) {
  hipLaunchKernelGGL(k_history_append, dim3(lanes), dim3(64), 0, st, hist, hist_len, max_len, committed, out_tokens,
                     out_stride);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
