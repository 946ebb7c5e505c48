// Sparse gather of the 24 selected MXFP8 rows per token and exact decode to a
// 6,144-wide BF16 memory vector.
//
// [zLLM] 第二步: read only the selected rows and the matching scales; the
// table is MXFP8 (E4M3 data plus one E8M0 scale per 32 values).
// [Storage]: FP8 E4M3 with UE8M0 group-32 scales, decoded straight to BF16.
// [vLLM] How it works: the fetched rows are concatenated into one memory
// vector per position (bucket j fills values j*256 .. j*256+255).
//
// HBM-bound. A 16-lane group owns one 256-byte row: lane l loads the 8 codes
// at l*8 and the 8 at 128 + l*8 (two 8-byte loads) plus the row's 8 scale
// bytes, decodes, and writes 16 bytes to each half of the 512-byte BF16 row,
// so every store instruction covers whole contiguous lines (stores of
// 16 bytes at a 32-byte stride left partial lines and cost 16% more time).
// Each lane keeps kRowsInFlight rows' loads outstanding before decoding to
// cover the latency of random HBM reads.

#include "decode_device.h"

namespace engram {
namespace {

constexpr int kBlock = 256;
constexpr int kGroups = kBlock / 16;     // rows per pass of one workgroup
constexpr int kRowsInFlight = 4;         // passes per workgroup (rows per lane)

// With `slot` (from live_slots_kernel), position t's rows go to row slot[t]
// of mem and a DEAD position writes nothing; without it, to row t. BK: the
// table is one allocation per bucket (tb), not codes/scales.
template <bool BK>
__global__ __launch_bounds__(kBlock) void gather_decode_kernel(
    const uint32_t* __restrict__ idx, int64_t total_rows, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, uint64_t n_rows, uint16_t* __restrict__ mem,
    const uint32_t* __restrict__ slot, bool staged, uint32_t* err, const TableBuckets tb) {
  __shared__ BucketLds bl;
  if constexpr (BK) load_buckets(tb, bl);
  const int l = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int64_t base = (int64_t)blockIdx.x * (kGroups * kRowsInFlight);

  // Codes [8l, 8l+8) use scale l/4 (byte l/4 of the first scale word) and
  // codes [128+8l, 128+8l+8) use scale 4 + l/4 (same byte of the second).
  const int sh = 8 * (l >> 2);
  uint2 ca[kRowsInFlight], cb[kRowsInFlight];
  uint32_t sa[kRowsInFlight], sb[kRowsInFlight];
  int64_t out_row[kRowsInFlight];   // destination row of mem, or -1 for none
  bool live[kRowsInFlight];
#pragma unroll
  for (int u = 0; u < kRowsInFlight; ++u) {
    const int64_t r = base + u * kGroups + grp;
    live[u] = false;
    ca[u] = cb[u] = make_uint2(0, 0);
    sa[u] = sb[u] = 127;
    out_row[u] = -1;
    if (r < total_rows) {
      if (slot == nullptr) {
        out_row[u] = r;
      } else {
        const int64_t t = r / ENGRAM_BUCKETS;
        const uint32_t st = slot[t];
        if (st != ENGRAM_DEAD_IDX) out_row[u] = (int64_t)st * ENGRAM_BUCKETS + (r - t * ENGRAM_BUCKETS);
      }
      const uint32_t row = idx[r];
      if (row != ENGRAM_DEAD_IDX) {
        const uint8_t *cr = nullptr, *sr = nullptr;
        const bool in_table = row_address<BK>(codes, scales, n_rows, &bl,
                                                       (int)(r % ENGRAM_BUCKETS), row, cr, sr);
        if (in_table) {
          live[u] = true;
          if (staged) {   // the row was copied to staging row r
            cr = codes + (uint64_t)r * ENGRAM_ROW;
            sr = scales + (uint64_t)r * ENGRAM_SCALES_PER_ROW;
          }
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
  for (int u = 0; u < kRowsInFlight; ++u) {
    if (out_row[u] < 0) continue;
    decode_store_row(mem + out_row[u] * ENGRAM_ROW, l, live[u], ca[u], cb[u], sa[u], sb[u]);
  }
}

// Staging copy for tables in pinned host memory: a 16-lane group moves one
// 256-byte row with one 16-byte load per lane (lane 0 also moves the row's
// 8 scale bytes), kStageRowsInFlight rows per lane outstanding, since every
// read crosses the host link and waits on its latency.
constexpr int kStageRowsInFlight = 8;

template <bool BK>
__global__ __launch_bounds__(kBlock) void stage_rows_kernel(
    const uint32_t* __restrict__ idx, int64_t total_rows, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, uint64_t n_rows, uint8_t* __restrict__ stage_codes,
    uint8_t* __restrict__ stage_scales, uint32_t* err, const TableBuckets tb) {
  __shared__ BucketLds bl;
  if constexpr (BK) load_buckets(tb, bl);
  const int l = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int64_t base = (int64_t)blockIdx.x * (kGroups * kStageRowsInFlight);
  uint4 c[kStageRowsInFlight];
  uint2 sc[kStageRowsInFlight];
  bool go[kStageRowsInFlight];
#pragma unroll
  for (int u = 0; u < kStageRowsInFlight; ++u) {
    const int64_t r = base + u * kGroups + grp;
    go[u] = false;
    c[u] = make_uint4(0, 0, 0, 0);
    sc[u] = make_uint2(0, 0);
    if (r < total_rows) {
      const uint32_t row = idx[r];
      if (row != ENGRAM_DEAD_IDX) {
        const uint8_t *cr = nullptr, *sr = nullptr;
        if (row_address<BK>(codes, scales, n_rows, &bl, (int)(r % ENGRAM_BUCKETS), row, cr, sr)) {
          go[u] = true;
          c[u] = *reinterpret_cast<const uint4*>(cr + l * 16);
          if (l == 0) sc[u] = *reinterpret_cast<const uint2*>(sr);
        } else {
          set_err(err, ENGRAM_ERR_ROW_RANGE);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kStageRowsInFlight; ++u) {
    if (!go[u]) continue;
    const int64_t r = base + u * kGroups + grp;
    *reinterpret_cast<uint4*>(stage_codes + r * ENGRAM_ROW + l * 16) = c[u];
    if (l == 0) *reinterpret_cast<uint2*>(stage_scales + r * ENGRAM_SCALES_PER_ROW) = sc[u];
  }
}

}  // namespace

hipError_t launch_stage_rows(const uint32_t* idx, int64_t T, const uint8_t* codes,
                             const uint8_t* scales, uint64_t n_rows, uint8_t* stage_codes,
                             uint8_t* stage_scales, uint32_t* err, hipStream_t st,
                             const TableBuckets* tb) {
  const int64_t rows = T * ENGRAM_BUCKETS;
  if (rows == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kGroups * kStageRowsInFlight;
  const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
  if (tb != nullptr)
    stage_rows_kernel<true><<<blocks, kBlock, 0, st>>>(idx, rows, codes, scales, n_rows, stage_codes,
                                                       stage_scales, err, *tb);
  else
    stage_rows_kernel<false><<<blocks, kBlock, 0, st>>>(idx, rows, codes, scales, n_rows,
                                                        stage_codes, stage_scales, err, TableBuckets{});
  return hipGetLastError();
}

hipError_t launch_gather_decode(const uint32_t* idx, int64_t T, const uint8_t* codes,
                                const uint8_t* scales, uint64_t n_rows, uint16_t* mem,
                                const uint32_t* slot, bool staged, uint32_t* err, hipStream_t st,
                                const TableBuckets* tb) {
  const int64_t rows = T * ENGRAM_BUCKETS;
  if (rows == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kGroups * kRowsInFlight;
  const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
  if (tb != nullptr && !staged)
    gather_decode_kernel<true><<<blocks, kBlock, 0, st>>>(idx, rows, codes, scales, n_rows, mem, slot,
                                                          false, err, *tb);
  else
    gather_decode_kernel<false><<<blocks, kBlock, 0, st>>>(idx, rows, codes, scales, n_rows, mem, slot,
                                                           staged, err, TableBuckets{});
  return hipGetLastError();
}

}  // namespace engram
