// Exact top-k selection over keys held by one wave (persistent-mode routing and the
// persistent-memory update).
#pragma once
#include "common.h"

namespace pbsa {

// Exact top-k of the 64*E keys held by one wave (key 0 = no candidate; needs
// 1 <= k <= number of candidates, all candidate keys distinct and nonzero): on[e] is set
// for the k largest.  The k-th largest high word is found bit by bit (is there a value with
// this prefix that leaves >= k keys at or above it?), stopping as soon as a prefix leaves
// exactly k; then, if the keys tied on it are more than needed, the same search runs over
// their low words.
template <int E>
__device__ __forceinline__ void wave_topk(const uint64_t (&key)[E], int k, bool (&on)[E]) {
  uint32_t hi[E], lo[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    hi[e] = static_cast<uint32_t>(key[e] >> 32);
    lo[e] = static_cast<uint32_t>(key[e]);
  }
  uint32_t p = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = p | (1u << b);
    int n = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) n += __popcll(__ballot(hi[e] >= c));
    if (n == k) {
      // exactly k keys have a high word >= c: they are the top k (n is the same in every
      // lane, so the whole wave leaves here)
#pragma unroll
      for (int e = 0; e < E; ++e) on[e] = hi[e] >= c;
      return;
    }
    if (n > k) p = c;
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gt += __popcll(__ballot(hi[e] > p));
    eq += __popcll(__ballot(hi[e] == p));
  }
  const int need = k - gt;  // in [1, eq]
  uint32_t q = 0;
  if (need < eq) {
    for (int b = 31; b >= 0; --b) {
      const uint32_t c = q | (1u << b);
      int n = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) n += __popcll(__ballot(hi[e] == p && lo[e] >= c));
      if (n >= need) q = c;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) on[e] = hi[e] > p || (hi[e] == p && lo[e] >= q);
}

}  // namespace pbsa
