// Internal declarations shared by the libengram sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/engram.h"

namespace engram {

// ---------------------------------------------------------------- launchers
// Each launcher assumes the host-side checks in engram_api.cpp have passed
// and returns the hipError_t of its launch.
hipError_t launch_history_reset(uint32_t* hist, int32_t S, uint32_t pad_cid, hipStream_t st);
hipError_t launch_history_copy(uint32_t* dst, const uint32_t* src, int32_t S, hipStream_t st);
hipError_t launch_history_append(uint32_t* hist, const uint32_t* tok, const int32_t* cu,
                                 int32_t S, int64_t T, const uint32_t* map, uint32_t map_len,
                                 uint32_t pad_cid, uint32_t* err, hipStream_t st);
hipError_t launch_hash(const uint32_t* tok, const int32_t* cu, int32_t S, int64_t T,
                       const uint32_t* hist, const uint32_t* map, uint32_t map_len,
                       const engram_hash_params& p, uint32_t* idx, uint32_t* err,
                       hipStream_t st);
// Rows of the live (non-DEAD) positions of tok[T]: slot[t] = live positions
// before t (ENGRAM_DEAD_IDX for a DEAD one), *count = live positions, and,
// when live_pos is given, live_pos[slot[t]] = t (the live positions in
// order). chunk_count: scratch of live_chunks(T) words.
constexpr int64_t kLiveChunkPositions = 4096;
inline int64_t live_chunks(int64_t T) { return (T + kLiveChunkPositions - 1) / kLiveChunkPositions; }
hipError_t launch_live_slots(const uint32_t* tok, int64_t T, uint32_t* slot, uint32_t* count,
                             uint32_t* chunk_count, uint32_t* live_pos, hipStream_t st);
// A table kept as one allocation per bucket: bucket j's rows first[j] ..
// first[j] + count[j] - 1 start at codes[j] / scales[j] (device addresses).
struct TableBuckets {
  uint64_t codes[ENGRAM_BUCKETS];
  uint64_t scales[ENGRAM_BUCKETS];
  uint32_t first[ENGRAM_BUCKETS];
  uint32_t count[ENGRAM_BUCKETS];
};

// slot: NULL (position t's rows go to mem row t), or the live_slots map
// (they go to row slot[t]; DEAD positions write nothing).
// staged: codes/scales are launch_stage_rows' staging area, where row
// t*24 + j holds table row idx[t][j] (idx still marks DEAD and out-of-range
// rows); otherwise they are the table and row idx[t][j] is read.
// tb: NULL (codes/scales hold the table), or the table's buckets (codes and
// scales then only matter with `staged`).
hipError_t launch_gather_decode(const uint32_t* idx, int64_t T, const uint8_t* codes,
                                const uint8_t* scales, uint64_t n_rows, uint16_t* mem,
                                const uint32_t* slot, bool staged, uint32_t* err, hipStream_t st,
                                const TableBuckets* tb = nullptr);
// Copies table row idx[t][j] (256 code bytes, 8 scale bytes) to row t*24 + j
// of a staging area in device memory, for tables in pinned host memory:
// every row crosses the host link once, in 16-byte loads with many rows in
// flight. DEAD and out-of-range rows are skipped (the latter flagged).
hipError_t launch_stage_rows(const uint32_t* idx, int64_t T, const uint8_t* codes,
                             const uint8_t* scales, uint64_t n_rows, uint8_t* stage_codes,
                             uint8_t* stage_scales, uint32_t* err, hipStream_t st,
                             const TableBuckets* tb = nullptr);
// Hash, gather and decode as one kernel (hash_gather.hip): for batches of at
// most kHashGatherMaxTokens tokens in at most kHashGatherMaxSeqs sequences,
// where both steps are latency-bound chains of loads. Writes the same idx and
// mem as launch_hash followed by launch_gather_decode.
constexpr int64_t kHashGatherMaxTokens = 1024;
constexpr int32_t kHashGatherMaxSeqs = 1024;
hipError_t launch_hash_gather(const uint32_t* tok, const int32_t* cu, int32_t S, int64_t T,
                              const uint32_t* hist, const uint32_t* map, uint32_t map_len,
                              const engram_hash_params& p, const uint8_t* codes,
                              const uint8_t* scales, uint32_t* idx, uint16_t* mem, uint32_t* err,
                              hipStream_t st, const TableBuckets* tb = nullptr);
// live_rows: NULL, or a device word holding how many of the T rows of mem
// count (T > 256 only; rows past it are neither computed in full nor stored).
// wkv_packed: NULL, or wkv in the packed decode layout (launch_pack_wkv),
// which batches of at most kSkinnyMaxTokens tokens then read instead of wkv.
constexpr int64_t kSkinnyMaxTokens = 256;
hipError_t launch_project(const uint16_t* mem, int64_t T, const uint32_t* live_rows,
                          const uint16_t* wkv, const uint16_t* wkv_packed, int32_t N, uint16_t* kv,
                          hipStream_t st);
// Packed decode layout of wkv[N][6144]: groups of pack_group_rows(N) rows
// (ceil(N / 256) kept within 16..kPackMaxGroupRows, so 256 groups unless the
// clamp applies; the last group may be shorter), cut in 16-row tiles whose
// values are ordered [super-step of kPackSK][k-step][lane group][row][8].
constexpr int kPackSK = 64;
constexpr int kPackMaxGroupRows = 112;
inline int pack_group_rows(int32_t N) {
  const int g = (N + 255) / 256;
  return g < 16 ? 16 : (g > kPackMaxGroupRows ? kPackMaxGroupRows : g);
}
hipError_t launch_pack_wkv(const uint16_t* wkv, int32_t N, uint16_t* out, hipStream_t st);
// kv_row: NULL (position t reads kv row t), or the live_slots map. live_pos,
// live_count: NULL, or launch_live_slots' live_pos and count for the same
// tokens (kv_row given too): the kernels that walk tokens then walk the live
// rows only.
hipError_t launch_gate(uint16_t* hidden, const uint16_t* kv, const float* wqk,
                       const uint32_t* tok, const uint32_t* kv_row, const uint32_t* live_pos,
                       const uint32_t* live_count, int64_t T, int32_t H, int32_t hc, float eps,
                       float dot_scale, float* gate_out, hipStream_t st);
hipError_t launch_gen_table(uint8_t* codes, uint8_t* scales, uint64_t row_begin,
                            uint64_t n_rows, uint64_t key_data, uint64_t key_scale,
                            hipStream_t st);

// Compute units of the current device, looked up once per device (kernels
// that keep one workgroup per CU size their grids with it).
inline hipError_t cu_count(int* n) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *n = c;
      return hipSuccess;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (c < 1) c = 1;
  if (cached) cache[dev].store(c, std::memory_order_relaxed);
  *n = c;
  return hipSuccess;
}

// Batches above these limits pack the live positions' rows (see launch_live_slots).
inline bool packs_rows(int64_t T, int32_t S) {
  return T > kHashGatherMaxTokens || S > kHashGatherMaxSeqs;
}

// Sections of the per-layer workspace, each 256-byte aligned:
//   idx uint32[T][24] | slot uint32[T] | live count + per-chunk counts |
//   mem bf16[T][6144] | kv bf16[T][(hc+1)H] | live positions uint32[T].
// The kv section is at least T*24*264 bytes: rows staged from a host table
// (codes [T*24][256], then scales [T*24][8]) sit there until the decode has
// read them, before the projection writes kv.
struct WorkspaceLayout {
  size_t bytes;
  uint32_t* idx;
  uint32_t* slot;
  uint32_t* live;
  uint16_t* mem;
  uint16_t* kv;
  uint32_t* live_pos;
  uint8_t* stage_codes;
  uint8_t* stage_scales;
};

inline size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(void* ws, int64_t T, int32_t H, int32_t hc) {
  const size_t t = T > 0 ? (size_t)T : 0;
  const size_t kv_bytes = t * (size_t)(hc + 1) * (size_t)H * 2;
  const size_t stage_bytes = t * ENGRAM_BUCKETS * (ENGRAM_ROW + ENGRAM_SCALES_PER_ROW);
  const size_t o_slot = round256(t * ENGRAM_BUCKETS * 4);
  const size_t o_count = o_slot + round256(t * 4);
  const size_t o_mem = o_count + round256(4 * (1 + (size_t)live_chunks((int64_t)t)));
  const size_t o_kv = o_mem + round256(t * ENGRAM_MEM * 2);
  const size_t o_pos = o_kv + round256(kv_bytes > stage_bytes ? kv_bytes : stage_bytes);
  uint8_t* w = static_cast<uint8_t*>(ws);
  WorkspaceLayout L;
  L.bytes = o_pos + round256(t * 4);
  L.idx = reinterpret_cast<uint32_t*>(w);
  L.slot = reinterpret_cast<uint32_t*>(w + o_slot);
  L.live = reinterpret_cast<uint32_t*>(w + o_count);
  L.mem = reinterpret_cast<uint16_t*>(w + o_mem);
  L.kv = reinterpret_cast<uint16_t*>(w + o_kv);
  L.live_pos = reinterpret_cast<uint32_t*>(w + o_pos);
  L.stage_codes = w + o_kv;
  L.stage_scales = w + o_kv + t * ENGRAM_BUCKETS * ENGRAM_ROW;
  return L;
}

// The body of engram_forward, argument checks included (engram_api.cpp); the
// entry point without a workspace argument calls it with its own device buffer.
int forward_impl(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                 const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                 const engram_hash_params* params, const uint8_t* codes, const uint8_t* scales,
                 const uint16_t* wkv, const uint16_t* wkv_packed, const float* wqk, uint16_t* hidden,
                 int32_t H, int32_t hc, float eps, float dot_scale, void* ws, size_t ws_bytes,
                 float* gate_out, uint32_t* err_flags, hipEvent_t* stage_events, hipStream_t stream);

// Sets this thread's engram_last_error() text (with the HIP error's name when
// e != hipSuccess) and returns status.
int report(int status, const char* what, hipError_t e);

// ---------------------------------------------------------------- device helpers
// float32 -> bfloat16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ void set_err(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace engram
