// Sparse gather of the 24 selected MXFP8 rows per token and exact decode to a
// 6,144-wide BF16 memory vector.
//
// [zLLM] 第二步: read only the selected rows and the matching scales; the
// table is MXFP8 (E4M3 data plus one E8M0 scale per 32 values).
// [Storage]: FP8 E4M3 with UE8M0 group-32 scales, decoded straight to BF16.
// [vLLM] How it works: the fetched rows are concatenated into one memory
// vector per position (bucket j fills values j*256 .. j*256+255).
//
// HBM-bound. A 16-lane group owns one 256-byte row: each lane loads 16
// codes with one 16-byte load plus the byte of the scale its codes share
// (lanes 2q and 2q+1 share scale q), decodes, and writes 32 bytes. Each lane
// keeps kRowsInFlight rows' loads outstanding before decoding to cover the
// latency of random HBM reads.

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kBlock = 256;
constexpr int kGroups = kBlock / 16;     // rows per pass of one workgroup
constexpr int kRowsInFlight = 4;         // passes per workgroup (rows per lane)

// Exact E4M3 x 2^(s-127) -> BF16 bits, rounded to nearest even where the
// result falls below BF16's normal range. E4M3 is the OCP "FN" encoding
// (bias 7, exponent 0 subnormal, S.1111.111 NaN, no infinity); E8M0 s = 255
// is NaN. A NaN keeps the code's sign.
__device__ __forceinline__ uint32_t mxfp8_to_bf16(uint32_t b, uint32_t s) {
  const uint32_t sign = (b & 0x80u) << 8;
  const uint32_t mag = b & 0x7Fu;
  if (mag == 0x7Fu || s == 255u) return sign | 0x7FC0u;
  if (mag == 0u) return sign;
  const uint32_t e = mag >> 3, m = mag & 7u;
  // value = M * 2^X, M = 1.mmm as an integer (normal) or 0.mmm (subnormal)
  const int32_t M = e ? (int32_t)(8u | m) : (int32_t)m;
  const int32_t X = (e ? (int32_t)e - 10 : -9) + (int32_t)s - 127;
  const int32_t p = 31 - __builtin_clz((uint32_t)M);   // leading bit of M, 0..3
  const int32_t E = X + p;                             // value in [2^E, 2^(E+1))
  if (E > 127) return sign | 0x7F80u;                  // beyond BF16 range
  if (E >= -126)
    return sign | ((uint32_t)(E + 127) << 7) | (((uint32_t)M << (7 - p)) & 0x7Fu);
  // BF16 subnormal: count quanta of 2^-133, ties to even.
  const int32_t sh = X + 133;
  if (sh >= 0) return sign | ((uint32_t)M << sh);
  const int32_t r = -sh;
  if (r > 4) return sign;                              // M < 16: below half a quantum
  const uint32_t q = (uint32_t)M >> r;
  const uint32_t rem = (uint32_t)M & ((1u << r) - 1u);
  const uint32_t half = 1u << (r - 1);
  return sign | (q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u));
}

__device__ __forceinline__ uint32_t pack2(uint32_t w, int byte0, uint32_t s) {
  return mxfp8_to_bf16((w >> (8 * byte0)) & 0xFFu, s) |
         (mxfp8_to_bf16((w >> (8 * byte0 + 8)) & 0xFFu, s) << 16);
}

__global__ __launch_bounds__(kBlock) void gather_decode_kernel(
    const uint32_t* __restrict__ idx, int64_t total_rows, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, uint64_t n_rows, uint16_t* __restrict__ mem,
    uint32_t* err) {
  const int lane16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int64_t base = (int64_t)blockIdx.x * (kGroups * kRowsInFlight);

  uint4 c[kRowsInFlight];
  uint32_t sc[kRowsInFlight];
  bool live[kRowsInFlight];
#pragma unroll
  for (int u = 0; u < kRowsInFlight; ++u) {
    const int64_t r = base + u * kGroups + grp;
    live[u] = false;
    c[u] = make_uint4(0, 0, 0, 0);
    sc[u] = 127;
    if (r < total_rows) {
      const uint32_t row = idx[r];
      if (row != ENGRAM_DEAD_IDX) {
        if ((uint64_t)row < n_rows) {
          live[u] = true;
          c[u] = *reinterpret_cast<const uint4*>(codes + (uint64_t)row * ENGRAM_ROW + lane16 * 16);
          sc[u] = scales[(uint64_t)row * ENGRAM_SCALES_PER_ROW + (lane16 >> 1)];
        } else {
          set_err(err, ENGRAM_ERR_ROW_RANGE);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsInFlight; ++u) {
    const int64_t r = base + u * kGroups + grp;
    if (r >= total_rows) continue;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (live[u]) {
      const uint32_t s = sc[u];
      lo = make_uint4(pack2(c[u].x, 0, s), pack2(c[u].x, 2, s), pack2(c[u].y, 0, s), pack2(c[u].y, 2, s));
      hi = make_uint4(pack2(c[u].z, 0, s), pack2(c[u].z, 2, s), pack2(c[u].w, 0, s), pack2(c[u].w, 2, s));
    }
    uint4* out = reinterpret_cast<uint4*>(mem + r * ENGRAM_ROW + lane16 * 16);
    out[0] = lo;
    out[1] = hi;
  }
}

}  // namespace

hipError_t launch_gather_decode(const uint32_t* idx, int64_t T, const uint8_t* codes,
                                const uint8_t* scales, uint64_t n_rows, uint16_t* mem,
                                uint32_t* err, hipStream_t st) {
  const int64_t rows = T * ENGRAM_BUCKETS;
  if (rows == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kGroups * kRowsInFlight;
  const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
  gather_decode_kernel<<<blocks, kBlock, 0, st>>>(idx, rows, codes, scales, n_rows, mem, err);
  return hipGetLastError();
}

}  // namespace engram
