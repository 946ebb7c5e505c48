// Device side of the MXFP8 row decode, shared by gather_decode_kernel and the
// fused small-batch hash + gather kernel.
//
// [Storage]: FP8 E4M3 with UE8M0 group-32 scales, decoded straight to BF16.
#pragma once

#include "engram_internal.h"

namespace engram {

// Exact E4M3 x 2^(s-127) -> BF16, two codes at a time, on the gfx950
// scaled-convert unit: v_cvt_scalef32_pk_bf16_fp8 multiplies each OCP E4M3
// code by the power of two held in the exponent field of its float scale
// operand (for a scale byte s that is the float with bits s << 23, so s = 0
// and s = 255 need no special case) and rounds to BF16. Its results are exact
// for every finite code and scale, BF16 subnormals included; every NaN it
// produces is 0xFFC0. The method keeps each value's sign from its code, so
// the sign bits are re-applied from the codes: a no-op for all non-NaN
// results, and it turns NaNs into sign(code)|0x7FC0.
template <bool HI>
__device__ __forceinline__ uint32_t decode2(uint32_t w, float scale) {
  const auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
  const uint32_t bits = __builtin_bit_cast(uint32_t, r);
  const uint32_t b = HI ? (w >> 16) : w;                      // the two codes in bytes 0, 1
  const uint32_t signs = ((b << 8) & 0x8000u) | ((b << 16) & 0x80000000u);
  return (bits & 0x7FFF7FFFu) | signs;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void nt_store16(uint16_t* p, uint32_t a, uint32_t b, uint32_t c,
                                           uint32_t d) {
  const u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// One 16-lane group's share of a 256-byte row: lane l holds codes [8l, 8l+8)
// (ca) and [128+8l, 128+8l+8) (cb); their scales are byte l/4 of the row's
// first and second scale words. Writes the 16 decoded BF16 values of each
// half to out + 8l and out + 128 + 8l, or zeros for a row that is not live.
__device__ __forceinline__ void decode_store_row(uint16_t* out, int l, bool live, uint2 ca, uint2 cb,
                                                 uint32_t sa, uint32_t sb) {
  uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
  if (live) {
    const float s0 = __uint_as_float(sa << 23), s1 = __uint_as_float(sb << 23);
    a = make_uint4(decode2<false>(ca.x, s0), decode2<true>(ca.x, s0),
                   decode2<false>(ca.y, s0), decode2<true>(ca.y, s0));
    b = make_uint4(decode2<false>(cb.x, s1), decode2<true>(cb.x, s1),
                   decode2<false>(cb.y, s1), decode2<true>(cb.y, s1));
  }
  nt_store16(out + l * 8, a.x, a.y, a.z, a.w);
  nt_store16(out + 128 + l * 8, b.x, b.y, b.z, b.w);
}

// Rows of a table kept as one allocation per bucket (TableBuckets): a
// workgroup copies the 24 bases and row ranges into LDS once; a lane group
// then finds row `row` of bucket j at codes[j] + (row - first[j]) * 256.
struct BucketLds {
  uint64_t codes[ENGRAM_BUCKETS];
  uint64_t scales[ENGRAM_BUCKETS];
  uint32_t first[ENGRAM_BUCKETS];
  uint32_t count[ENGRAM_BUCKETS];
};

__device__ __forceinline__ void load_buckets(const TableBuckets& tb, BucketLds& b) {
  const int i = threadIdx.x;
  if (i < ENGRAM_BUCKETS) {
    b.codes[i] = tb.codes[i];
    b.scales[i] = tb.scales[i];
    b.first[i] = tb.first[i];
    b.count[i] = tb.count[i];
  }
  __syncthreads();
}

// Code and scale addresses of table row `row` for bucket j, and whether the
// row is in the table (for a bucketed table: in bucket j's range).
template <bool BK>
__device__ __forceinline__ bool row_address(const uint8_t* codes, const uint8_t* scales,
                                            uint64_t n_rows, const BucketLds* b, int j,
                                            uint32_t row, const uint8_t*& cr, const uint8_t*& sr) {
  if constexpr (BK) {
    const uint32_t k = row - b->first[j];
    if (k >= b->count[j]) return false;
    cr = reinterpret_cast<const uint8_t*>(b->codes[j]) + (uint64_t)k * ENGRAM_ROW;
    sr = reinterpret_cast<const uint8_t*>(b->scales[j]) + (uint64_t)k * ENGRAM_SCALES_PER_ROW;
    return true;
  } else {
    if ((uint64_t)row >= n_rows) return false;
    cr = codes + (uint64_t)row * ENGRAM_ROW;
    sr = scales + (uint64_t)row * ENGRAM_SCALES_PER_ROW;
    return true;
  }
}

}  // namespace engram
