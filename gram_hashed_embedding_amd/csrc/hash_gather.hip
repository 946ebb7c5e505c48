// Hash, gather and decode in one kernel, for small batches (decode steps).
//
// [zLLM] 第一步 and 第二步: a token's 24 row numbers come from its hashed
// n-grams, and only those rows and their scales are read and decoded. For a
// few hundred tokens neither step moves enough data to be bound by
// bandwidth: each is a chain of dependent loads (sequence search, token,
// map, history, then the row), and running them as two kernels adds a
// second launch and a round trip of the indices through memory. Here a
// 16-lane group takes one (token, bucket): all 16 lanes compute its row
// number (the same value; the loads they share coalesce), lane 0 stores it,
// and the group loads and decodes the row with the lane layout of
// gather_decode_kernel. cu_seqlens is copied into LDS first, so the
// per-lane sequence search reads LDS.
//
// The index and the decoded row are bit-identical to engram_hash followed by
// engram_gather_decode, and the error flags are the same bits.

#include "decode_device.h"
#include "hash_device.h"

namespace engram {
namespace {

constexpr int kBlock = 256;
constexpr int kGroups = kBlock / 16;   // rows per pass of one workgroup

template <int RIF, bool BK>
__global__ __launch_bounds__(kBlock) void hash_gather_kernel(
    const uint32_t* __restrict__ tok, const int32_t* __restrict__ cu, int32_t S, int64_t T,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ map, uint32_t map_len,
    const engram_hash_params p, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, uint32_t* __restrict__ idx, uint16_t* __restrict__ mem,
    uint32_t* err, const TableBuckets tb) {
  __shared__ int32_t cu_s[kHashGatherMaxSeqs + 1];
  __shared__ BucketLds bl;
  for (int i = threadIdx.x; i <= S; i += kBlock) cu_s[i] = cu[i];
  if constexpr (BK) load_buckets(tb, bl);   // (its barrier also publishes cu_s)
  __syncthreads();

  const int l = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int64_t total_rows = T * ENGRAM_BUCKETS;
  const int64_t base = (int64_t)blockIdx.x * (kGroups * RIF);
  const int sh = 8 * (l >> 2);
  uint2 ca[RIF], cb[RIF];
  uint32_t sa[RIF], sb[RIF];
  bool live[RIF];
#pragma unroll
  for (int u = 0; u < RIF; ++u) {
    const int64_t r = base + u * kGroups + grp;
    live[u] = false;
    ca[u] = cb[u] = make_uint2(0, 0);
    sa[u] = sb[u] = 127;
    if (r < total_rows) {
      const int64_t t = r / ENGRAM_BUCKETS;
      const int j = (int)(r - t * ENGRAM_BUCKETS);
      const uint32_t tk = tok[t];
      const uint32_t row = tk == ENGRAM_DEAD_TOKEN
                               ? ENGRAM_DEAD_IDX
                               : bucket_row(tok, cu_s, S, T, hist, map, map_len, p, t, j, tk, err);
      if (l == 0) idx[r] = row;
      if (row != ENGRAM_DEAD_IDX) {
        const uint8_t *cr = nullptr, *sr = nullptr;
        if (row_address<BK>(codes, scales, p.n_rows, &bl, j, row, cr, sr)) {
          live[u] = true;
          ca[u] = *reinterpret_cast<const uint2*>(cr + l * 8);
          cb[u] = *reinterpret_cast<const uint2*>(cr + 128 + l * 8);
          const uint2 s2 = *reinterpret_cast<const uint2*>(sr);
          sa[u] = (s2.x >> sh) & 0xFFu;
          sb[u] = (s2.y >> sh) & 0xFFu;
        } else {
          set_err(err, ENGRAM_ERR_ROW_RANGE);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < RIF; ++u) {
    const int64_t r = base + u * kGroups + grp;
    if (r >= total_rows) continue;
    decode_store_row(mem + r * ENGRAM_ROW, l, live[u], ca[u], cb[u], sa[u], sb[u]);
  }
}

}  // namespace

hipError_t launch_hash_gather(const uint32_t* tok, const int32_t* cu, int32_t S, int64_t T,
                              const uint32_t* hist, const uint32_t* map, uint32_t map_len,
                              const engram_hash_params& p, const uint8_t* codes,
                              const uint8_t* scales, uint32_t* idx, uint16_t* mem, uint32_t* err,
                              hipStream_t st, const TableBuckets* tb) {
  if (T == 0) return hipSuccess;
  if (T > kHashGatherMaxTokens || S < 1 || S > kHashGatherMaxSeqs) return hipErrorInvalidValue;
  constexpr int kRif = 1;
  const int64_t rows = T * ENGRAM_BUCKETS;
  const unsigned blocks = (unsigned)((rows + kGroups * kRif - 1) / (kGroups * kRif));
  if (tb != nullptr)
    hash_gather_kernel<kRif, true><<<blocks, kBlock, 0, st>>>(tok, cu, S, T, hist, map, map_len, p,
                                                              codes, scales, idx, mem, err, *tb);
  else
    hash_gather_kernel<kRif, false><<<blocks, kBlock, 0, st>>>(tok, cu, S, T, hist, map, map_len, p,
                                                               codes, scales, idx, mem, err,
                                                               TableBuckets{});
  return hipGetLastError();
}

}  // namespace engram
