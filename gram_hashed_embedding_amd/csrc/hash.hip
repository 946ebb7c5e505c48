// Hashing and per-sequence history for the Engram retrieval step.
//
// [zLLM] 第一步: token id -> compressed id -> current token and the three most
// recent positions -> 24 hashes over 2/3/4-grams -> 24 row numbers, with
// per-layer multipliers, prime buckets and offsets as static tables.
// [vLLM] How it works (multi-head hashing): each (order, head) pair applies a
// multiply-XOR hash to the compressed suffix n-gram and indexes its own
// prime-sized bucket range.
// [zLLM] 第四步: each token enters the history once; DEAD image spans break
// text n-grams; fork copies a session's history, reset clears it.
//
// Integer work only. One lane per (token, bucket): the 24 lanes of a token
// write its 96-byte index row contiguously.

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kBlock = 256;

// Sequence owning global token position t: the s with cu[s] <= t < cu[s+1].
// cu values are clamped to [0, T] so a malformed list cannot send a read out
// of bounds; inconsistencies are flagged.
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

__global__ __launch_bounds__(kBlock) void hash_kernel(
    const uint32_t* __restrict__ tok, const int32_t* __restrict__ cu, int32_t S, int64_t T,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ map, uint32_t map_len,
    const engram_hash_params p, uint32_t* __restrict__ idx, uint32_t* err) {
  const int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (g >= T * ENGRAM_BUCKETS) return;
  const int64_t t = g / ENGRAM_BUCKETS;
  const int j = (int)(g - t * ENGRAM_BUCKETS);
  const int n = 2 + j / ENGRAM_HEADS_PER_ORDER;

  const uint32_t tk = tok[t];
  if (tk == ENGRAM_DEAD_TOKEN) {
    idx[g] = ENGRAM_DEAD_IDX;
    return;
  }
  const int s = find_seq(cu, S, T, t, err);
  int64_t start = cu[s];
  start = start < 0 ? 0 : (start > t ? t : start);

  // Window slots w_0..w_{n-1}: walk back from t. Inside the segment a DEAD
  // ends the walk (everything behind it is PAD); before the segment the
  // history supplies slots (it already holds PAD where a DEAD was).
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
  idx[g] = (uint32_t)(p.offset[j] + x % (uint64_t)p.prime[j]);
}

// One lane per sequence: the new history is the last three compressed ids of
// the segment, stopping at a DEAD (PAD behind it) or continuing into the old
// history when the segment is shorter than three.
__global__ __launch_bounds__(kBlock) void history_append_kernel(
    uint32_t* __restrict__ hist, const uint32_t* __restrict__ tok, const int32_t* __restrict__ cu,
    int32_t S, int64_t T, const uint32_t* __restrict__ map, uint32_t map_len, uint32_t pad_cid,
    uint32_t* err) {
  const int s = blockIdx.x * kBlock + threadIdx.x;
  if (s >= S) return;
  int64_t a = cu[s], b = cu[s + 1];
  if (s == 0 && a != 0) set_err(err, ENGRAM_ERR_SEQLENS);
  if (s == S - 1 && b != T) set_err(err, ENGRAM_ERR_SEQLENS);
  a = a < 0 ? 0 : (a > T ? T : a);
  b = b < a ? a : (b > T ? T : b);
  uint32_t* h = hist + (int64_t)s * ENGRAM_HIST;
  const uint32_t old[3] = {h[0], h[1], h[2]};
  uint32_t nh[3];
  int filled = 0;
  bool dead = false;
  for (int64_t pos = b - 1; pos >= a && filled < 3; --pos) {
    const uint32_t tp = tok[pos];
    if (tp == ENGRAM_DEAD_TOKEN) { dead = true; break; }
    nh[filled++] = compress(map, map_len, 0xFFFFFFFFu, pad_cid, tp, err);
  }
  for (int i = filled; i < 3; ++i) nh[i] = dead ? pad_cid : old[i - filled];
  h[0] = nh[0];
  h[1] = nh[1];
  h[2] = nh[2];
}

__global__ __launch_bounds__(kBlock) void history_fill_kernel(uint32_t* __restrict__ dst,
                                                             const uint32_t* __restrict__ src,
                                                             int64_t n, uint32_t value) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : value;
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kBlock - 1) / kBlock); }

}  // namespace

hipError_t launch_history_reset(uint32_t* hist, int32_t S, uint32_t pad_cid, hipStream_t st) {
  const int64_t n = (int64_t)S * ENGRAM_HIST;
  if (n == 0) return hipSuccess;
  history_fill_kernel<<<blocks_for(n), kBlock, 0, st>>>(hist, nullptr, n, pad_cid);
  return hipGetLastError();
}

hipError_t launch_history_copy(uint32_t* dst, const uint32_t* src, int32_t S, hipStream_t st) {
  const int64_t n = (int64_t)S * ENGRAM_HIST;
  if (n == 0) return hipSuccess;
  history_fill_kernel<<<blocks_for(n), kBlock, 0, st>>>(dst, src, n, 0);
  return hipGetLastError();
}

hipError_t launch_history_append(uint32_t* hist, const uint32_t* tok, const int32_t* cu,
                                 int32_t S, int64_t T, const uint32_t* map, uint32_t map_len,
                                 uint32_t pad_cid, uint32_t* err, hipStream_t st) {
  if (S == 0) return hipSuccess;
  history_append_kernel<<<blocks_for(S), kBlock, 0, st>>>(hist, tok, cu, S, T, map, map_len,
                                                          pad_cid, err);
  return hipGetLastError();
}

hipError_t launch_hash(const uint32_t* tok, const int32_t* cu, int32_t S, int64_t T,
                       const uint32_t* hist, const uint32_t* map, uint32_t map_len,
                       const engram_hash_params& p, uint32_t* idx, uint32_t* err,
                       hipStream_t st) {
  const int64_t n = T * ENGRAM_BUCKETS;
  if (n == 0) return hipSuccess;
  hash_kernel<<<blocks_for(n), kBlock, 0, st>>>(tok, cu, S, T, hist, map, map_len, p, idx, err);
  return hipGetLastError();
}

}  // namespace engram
