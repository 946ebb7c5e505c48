// Closed-form synthetic MXFP8 table, written on the device (benchmark and
// test data only; not part of the Engram method). A full-size layer table is
// about 101 GB (384M rows x (256 code + 8 scale) bytes), too large to build on
// the host, so it is generated where it lives.
//
//   codes[r][c]  = F[hi32(splitmix64(key_data + r*256 + c)) mod 254]
//   scales[r][q] = 119 + hi32(splitmix64(key_scale + r*8 + q)) mod 9
//
// F is the ascending list of the 254 E4M3 codes that are not NaN (every code
// except 0x7F and 0xFF): F[i] = i for i < 127, i + 1 otherwise. splitmix64(x)
// is the first output of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014)
// whose state is x.

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kMaxBlocks = 65536;

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t finite_code(uint64_t z) {
  const uint32_t i = (uint32_t)(z >> 32) % 254u;
  return i < 127u ? i : i + 1u;
}

// One 16-byte store per item: 16 consecutive codes of one row.
__global__ __launch_bounds__(kThreads) void gen_codes_kernel(uint8_t* __restrict__ codes,
                                                             uint64_t row_begin, uint64_t items,
                                                             uint64_t key) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < items; i += stride) {
    const uint64_t r = row_begin + (i >> 4);
    const uint64_t c0 = (i & 15u) * 16u;
    const uint64_t base = key + r * ENGRAM_ROW + c0;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) v |= finite_code(splitmix64(base + 4 * q + b)) << (8 * b);
      w[q] = v;
    }
    *reinterpret_cast<uint4*>(codes + i * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One 8-byte store per row.
__global__ __launch_bounds__(kThreads) void gen_scales_kernel(uint8_t* __restrict__ scales,
                                                              uint64_t row_begin, uint64_t rows,
                                                              uint64_t key) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < rows; i += stride) {
    const uint64_t base = key + (row_begin + i) * ENGRAM_SCALES_PER_ROW;
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        v |= (119u + (uint32_t)(splitmix64(base + 4 * h + b) >> 32) % 9u) << (8 * b);
      w[h] = v;
    }
    *reinterpret_cast<uint2*>(scales + i * ENGRAM_SCALES_PER_ROW) = make_uint2(w[0], w[1]);
  }
}

inline unsigned grid_for(uint64_t items) {
  const uint64_t b = (items + kThreads - 1) / kThreads;
  return (unsigned)(b < kMaxBlocks ? b : kMaxBlocks);
}

}  // namespace

hipError_t launch_gen_table(uint8_t* codes, uint8_t* scales, uint64_t row_begin,
                            uint64_t n_rows, uint64_t key_data, uint64_t key_scale,
                            hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const uint64_t items = n_rows * 16u;
  gen_codes_kernel<<<grid_for(items), kThreads, 0, st>>>(codes, row_begin, items, key_data);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gen_scales_kernel<<<grid_for(n_rows), kThreads, 0, st>>>(scales, row_begin, n_rows, key_scale);
  return hipGetLastError();
}

}  // namespace engram
