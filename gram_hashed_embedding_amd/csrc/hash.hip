// Hashing and per-sequence history for the Engram retrieval step.
//
// [zLLM] 第一步: each token's 24 row numbers come from its compressed
// suffix n-grams (the hash itself is in hash_device.h).
// [zLLM] 第四步: each token enters the history once; DEAD image spans break
// text n-grams; fork copies a session's history, reset clears it.
//
// Integer work only. One lane per (token, bucket): the 24 lanes of a token
// write its 96-byte index row contiguously.

#include "hash_device.h"

namespace engram {
namespace {

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void hash_kernel(
    const uint32_t* __restrict__ tok, const int32_t* __restrict__ cu, int32_t S, int64_t T,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ map, uint32_t map_len,
    const engram_hash_params p, uint32_t* __restrict__ idx, uint32_t* err) {
  const int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (g >= T * ENGRAM_BUCKETS) return;
  const int64_t t = g / ENGRAM_BUCKETS;
  const int j = (int)(g - t * ENGRAM_BUCKETS);
  const uint32_t tk = tok[t];
  idx[g] = tk == ENGRAM_DEAD_TOKEN ? ENGRAM_DEAD_IDX
                                   : bucket_row(tok, cu, S, T, hist, map, map_len, p, t, j, tk, err);
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

// Rows of the live (non-DEAD) positions: slot[t] = number of live positions
// before t, or ENGRAM_DEAD_IDX for a DEAD one, and *count = number of live
// positions. Two passes over chunks of kLiveChunk positions (kLivePer
// consecutive ones per thread): live_count_kernel counts each chunk's live
// positions, then live_slots_kernel adds up the counts of the chunks before
// its own (at most a few hundred) and scans its chunk (wave shuffles, then
// the wave totals). Both passes spread over the whole GPU.
constexpr int kLiveThreads = 256, kLivePer = 16, kLiveChunk = kLiveThreads * kLivePer;
static_assert(kLiveChunk == kLiveChunkPositions, "chunk size");

__device__ __forceinline__ uint32_t live_bits(const uint32_t* __restrict__ tok, int64_t T, int64_t t0) {
  uint32_t live = 0;    // bit i: position t0 + i is live
#pragma unroll
  for (int i = 0; i < kLivePer; ++i)
    if (t0 + i < T && tok[t0 + i] != ENGRAM_DEAD_TOKEN) live |= 1u << i;
  return live;
}

template <int WAVES>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t total = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) total += sh[w];
  return total;
}

__global__ __launch_bounds__(kLiveThreads) void live_count_kernel(const uint32_t* __restrict__ tok,
                                                                  int64_t T, uint32_t* __restrict__ chunk_count) {
  __shared__ uint32_t sh[kLiveThreads / 64];
  const int64_t t0 = (int64_t)blockIdx.x * kLiveChunk + (int64_t)threadIdx.x * kLivePer;
  const uint32_t total = block_sum<kLiveThreads / 64>((uint32_t)__builtin_popcount(live_bits(tok, T, t0)), sh);
  if (threadIdx.x == 0) chunk_count[blockIdx.x] = total;
}

__global__ __launch_bounds__(kLiveThreads) void live_slots_kernel(const uint32_t* __restrict__ tok,
                                                                  int64_t T,
                                                                  const uint32_t* __restrict__ chunk_count,
                                                                  uint32_t* __restrict__ slot,
                                                                  uint32_t* __restrict__ count,
                                                                  uint32_t* __restrict__ live_pos) {
  constexpr int WAVES = kLiveThreads / 64;
  __shared__ uint32_t sh[WAVES], wave_tot[WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // live positions in the chunks before this one
  uint32_t before = 0;
  for (int c = tid; c < (int)blockIdx.x; c += kLiveThreads) before += chunk_count[c];
  before = block_sum<WAVES>(before, sh);
  const int64_t t0 = (int64_t)blockIdx.x * kLiveChunk + (int64_t)tid * kLivePer;
  const uint32_t live = live_bits(tok, T, t0);
  const uint32_t c = (uint32_t)__builtin_popcount(live);
  uint32_t incl = c;   // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t chunk_total = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    if (w < wave) before += wave_tot[w];
    chunk_total += wave_tot[w];
  }
  uint32_t r = before + incl - c;
#pragma unroll
  for (int i = 0; i < kLivePer; ++i) {
    if (t0 + i >= T) continue;
    if ((live >> i) & 1u) {
      if (live_pos != nullptr) live_pos[r] = (uint32_t)(t0 + i);   // the inverse map
      slot[t0 + i] = r++;
    } else {
      slot[t0 + i] = ENGRAM_DEAD_IDX;
    }
  }
  if (blockIdx.x == gridDim.x - 1 && tid == WAVES * 64 - 1) *count = r;   // the last live row + 1
  (void)chunk_total;
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

hipError_t launch_live_slots(const uint32_t* tok, int64_t T, uint32_t* slot, uint32_t* count,
                             uint32_t* chunk_count, uint32_t* live_pos, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const unsigned chunks = (unsigned)((T + kLiveChunk - 1) / kLiveChunk);
  live_count_kernel<<<chunks, kLiveThreads, 0, st>>>(tok, T, chunk_count);
  live_slots_kernel<<<chunks, kLiveThreads, 0, st>>>(tok, T, chunk_count, slot, count, live_pos);
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
