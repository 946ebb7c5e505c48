// Device side of the hash step: sequence lookup, token compression and the
// per-bucket multiply-XOR hash. Shared by hash_kernel and the fused
// small-batch hash + gather kernel, so both compute the same index.
//
// [zLLM] 第一步: token id -> compressed id -> current token and the three most
// recent positions -> 24 hashes over 2/3/4-grams -> 24 row numbers, with
// per-layer multipliers, prime buckets and offsets as static tables.
// [vLLM] How it works (multi-head hashing): each (order, head) pair applies a
// multiply-XOR hash to the compressed suffix n-gram and indexes its own
// prime-sized bucket range.
#pragma once

#include "engram_internal.h"

namespace engram {

// Sequence owning global token position t: the s with cu[s] <= t < cu[s+1].
// cu values are clamped to [0, T] so a malformed list cannot send a read out
// of bounds; inconsistencies are flagged. cu may point to global memory or to
// an LDS copy.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int32_t S, int64_t T,
                                        int64_t t, uint32_t* err) {
  int lo = 0, hi = S;  // invariant: answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    int64_t c = cu[mid];
    c = c < 0 ? 0 : (c > T ? T : c);
    if (c <= t) lo = mid; else hi = mid;
  }
  if (cu[0] != 0 || cu[S] != T) set_err(err, ENGRAM_ERR_SEQLENS);
  return lo;
}

__device__ __forceinline__ uint32_t compress(const uint32_t* __restrict__ map, uint32_t map_len,
                                             uint32_t vocab_c, uint32_t pad_cid, uint32_t tok,
                                             uint32_t* err) {
  if (tok >= map_len) {
    set_err(err, ENGRAM_ERR_TOKEN_RANGE);
    return pad_cid;
  }
  const uint32_t c = map[tok];
  if (c >= vocab_c) set_err(err, ENGRAM_ERR_MAP_RANGE);
  return c;
}

// Row index of bucket j (n = 2 + j / 8) for the non-DEAD token t whose raw id
// is tk. Window slots w_0..w_{n-1} walk back from t: inside the segment a
// DEAD ends the walk (everything behind it is PAD); before the segment the
// history supplies the slots (it already holds PAD where a DEAD was).
__device__ __forceinline__ uint32_t bucket_row(const uint32_t* __restrict__ tok,
                                               const int32_t* __restrict__ cu, int32_t S, int64_t T,
                                               const uint32_t* __restrict__ hist,
                                               const uint32_t* __restrict__ map, uint32_t map_len,
                                               const engram_hash_params& p, int64_t t, int j,
                                               uint32_t tk, uint32_t* err) {
  const int n = 2 + j / ENGRAM_HEADS_PER_ORDER;
  const int s = find_seq(cu, S, T, t, err);
  int64_t start = cu[s];
  start = start < 0 ? 0 : (start > t ? t : start);

  uint64_t w[4];
  w[0] = compress(map, map_len, p.vocab_c, p.pad_cid, tk, err);
  bool behind_dead = false;
  for (int k = 1; k < n; ++k) {
    const int64_t pos = t - k;
    uint32_t c;
    if (behind_dead) {
      c = p.pad_cid;
    } else if (pos >= start) {
      const uint32_t tp = tok[pos];
      if (tp == ENGRAM_DEAD_TOKEN) {
        behind_dead = true;
        c = p.pad_cid;
      } else {
        c = compress(map, map_len, p.vocab_c, p.pad_cid, tp, err);
      }
    } else {
      c = hist[(int64_t)s * ENGRAM_HIST + (k - 1 - (t - start))];
    }
    w[k] = c;
  }
  uint64_t x = 0;
  for (int k = 0; k < n; ++k) x ^= w[k] * p.mult[j][k];   // products wrap mod 2^64
  return (uint32_t)(p.offset[j] + x % (uint64_t)p.prime[j]);
}

}  // namespace engram
