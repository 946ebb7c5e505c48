// wkv projection: kv[T][N] = mem[T][6144] . wkv[N][6144]^T, N = (hc+1)*H.
//
// [zLLM] 第二步: the 6,144-wide vector goes through the wkv projection
// (25,600 x 6,144, BF16) to give the keys and the value the gate needs.
// [zLLM] AVX-512 BF16: prefill batches tokens so one weight load serves many
// tokens; a single decode token gets no such reuse.
// [vLLM] How it works: one key per hyper-connection branch plus one shared
// value.
//
// A dense contraction, so it runs on the matrix cores: gfx950
// v_mfma_f32_32x32x16_bf16 with FP32 accumulation. Both operands are
// K-contiguous, so every lane's MFMA fragment (8 consecutive K values of one
// row) is one 16-byte LDS read. Workgroups are renumbered so that the tiles
// in flight at one time form compact blocks: each XCD (which owns an L2)
// works on a small block of its own, and the XCDs' blocks sit side by side,
// so they share operands in the Infinity Cache.
//
// Two kernels:
//  - wave_tile_kernel (T > 256): 256 x 256 x 64 tiles, 4 waves of 128 x 128
//    each, loads staged through registers two K steps ahead and spread
//    between the MFMAs.
//  - skinny_kernel (T <= 256): the projection is a stream of wkv; the few mem
//    rows sit in LDS and wkv rows go straight into registers, read either
//    from wkv itself or from its packed decode layout (pack_wkv_kernel).
// Measured on the 25,600 x 6,144 wkv: the skinny kernel takes 78 / 95 / 104-117
// us at T = 64 / 128 / 160-256 on wkv and 51 / 62 / 78-91 us on the packed
// layout, where the 256 x 256 kernel takes 128-147 us; above T = 256 the
// 256 x 256 kernel wins (141-158 us at T = 384-512, where 128 x 128 tiles took
// 233-255 us).

#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int K = ENGRAM_MEM;
constexpr int BK = 64;
constexpr int kXcds = 8;
// Fourth word of a raw buffer resource on gfx9-family GPUs: a 32-bit data
// format, so the hardware accepts the buffer loads (raw loads with stride 0
// ignore the format otherwise).
constexpr int kRawBufferWord3 = 0x00020000;

// ---------------------------------------------------------------- wave-tile kernel
// Tile 256 x 256 x 64, 4 waves (one per SIMD), each owning a 128 x 128
// sub-tile: 16 accumulators of 32 x 32 fill the 256 accumulation registers,
// and every K16 step issues 16 MFMAs against 8 fragment reads, the lowest LDS
// traffic per MFMA a wave can have.
//
// Operands are staged through registers, two K steps ahead: in K step kt a
// thread writes its chunks of tile kt+1 from register set (kt+1) % 2 into the
// idle LDS buffer and then reloads that set with tile kt+3, so a global load
// has two whole K steps (~4,000 cycles) to return. Loads use buffer
// instructions whose row offsets sit in per-chunk registers and whose K
// position is a scalar offset. Each K step is cut into four K16 steps; the
// loads and LDS writes are spread between the MFMAs of the first three, every
// K16 step reads the next one's fragments first, and one barrier, before the
// last, publishes tile kt+1.
//
// LDS rows are 128 bytes (64 bf16 of K); 16-byte chunk c of row r is stored
// in slot c ^ swz(r), which keeps the 32-row fragment reads free of bank
// conflicts. The MFMA takes the wkv fragment as its first operand, so an
// accumulator holds a 32 x 32 block of kv transposed: each lane ends with
// four consecutive kv columns of one row, stored to LDS as one 8-byte write
// and then written out in 16-byte row chunks, with non-temporal stores (kv is
// read once, by the gate; 1.1% faster than ordinary stores).
constexpr int kWTBM = 256, kWTBN = 256;

// Tile order. Consecutive workgroup ids go to the XCDs in turn, so the 256
// workgroups in flight at once are ids 256w .. 256w + 255, 32 on each XCD.
// Such a group covers a block of kWTBand row tiles x (256 / kWTBand) column
// tiles (column-major inside a band of kWTBand row tiles), and each XCD gets
// a kWTSubRows x (32 / kWTSubRows) sub-block of it. Inside one XCD's L2 its
// 32 tiles share 4 row slices of mem and 8 column slices of wkv per K step;
// across the XCDs the group shares 16 + 16, so an L2 miss mostly finds its
// line in the Infinity Cache, brought in by another XCD, instead of in HBM.
// Against contiguous per-XCD tile ranges (4-row-tile groups) this is 5-6%
// faster on the 50,032 x 25,600 x 6,144 projection (interleaved A/B runs on
// three boxes). A last partial group of fewer than 256 tiles keeps the plain
// order.
constexpr int kWTBand = 16, kWTSubRows = 4;
__device__ __forceinline__ void wt_tile_of(int pid, int m_tiles, int n_tiles, int& m0, int& n0) {
  constexpr int kSubCols = 32 / kWTSubRows, kSubsPerBand = kWTBand / kWTSubRows;
  static_assert(kXcds == 8 && kSubsPerBand * (256 / kWTBand) / kSubCols == kXcds, "group shape");
  const int total = m_tiles * n_tiles;
  const int full = total & ~255;
  const int xcd = pid % kXcds, lid = pid / kXcds, l = lid % 32;
  const int sr = (xcd % kSubsPerBand) * kWTSubRows + l % kWTSubRows;
  const int sc = (xcd / kSubsPerBand) * kSubCols + l / kWTSubRows;
  const int logical = pid < full ? (lid / 32) * 256 + sc * kWTBand + sr : pid;
  const int span = kWTBand * n_tiles;
  const int first_m = (logical / span) * kWTBand;
  const int gm = (m_tiles - first_m) < kWTBand ? (m_tiles - first_m) : kWTBand;
  const int ing = logical % span;
  m0 = (first_m + ing % gm) * kWTBM;
  n0 = (ing / gm) * kWTBN;
}

__device__ __forceinline__ int wt_swz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Order inside one K16 step: 16 MFMAs; the NR fragment reads for the next
// K16 step go first, two per MFMA slot, then from slot 5 on the LDS writes and
// the global loads alternate (writes on odd slots, loads on even ones);
// nothing crosses the step. LDS returns a wave's operations in order, so a
// fragment read issued behind this step's 16-byte writes waits for them: with
// the reads in the back half, the next step's first MFMAs stalled on reads
// queued behind writes, and reads first is 4-6% faster on the 50,032 x 25,600
// x 6,144 projection (interleaved A/B runs on three boxes; four or eight reads
// per slot, or writes from slot 2 or 3, measured slower). Spacing the writes
// keeps the LDS write-data queue from filling, which would stall MFMA issue.
template <int NW, int NV, int NR>
__device__ __forceinline__ void wt_interleave() {
  constexpr int kFirstWrite = 5;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                               // MFMA
    if (q < NR / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);               // DS read x 2
    if (q >= kFirstWrite) {
      const int o = q - kFirstWrite;
      if ((o & 1) == 0 && o / 2 < NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // DS write
      if ((o & 1) == 1 && o / 2 < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // VMEM read
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// live_rows, when given, holds the number of rows of A that count (M is then
// only an upper bound from the host): tiles at or past it stop after their
// first loads, and rows past it are not stored.
__global__ __launch_bounds__(256) void wave_tile_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        uint16_t* __restrict__ C, int M,
                                                        const uint32_t* __restrict__ live_rows,
                                                        int N, int m_tiles, int n_tiles) {
  constexpr int BM = kWTBM, BN = kWTBN, ROWB = 128;
  constexpr int STAGE_A = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int TM = 4, TN = 4;
  constexpr int KT = K / BK;
  static_assert(KT % 2 == 0, "K steps come in pairs");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STAGE];

  int m0, n0;
  wt_tile_of(blockIdx.x, m_tiles, n_tiles, m0, n0);
  // a scalar load; it has returned by the end of the prologue's first LDS wait
  const int m_live = live_rows != nullptr ? (int)min(*live_rows, (uint32_t)M) : M;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Staging: thread t owns chunks (row (t >> 3) + 32 i, chunk t & 7), i < 8,
  // of both operands; swz(row) does not depend on i. Rows past the edge of A
  // or B re-read its last row (their products are never stored), so every
  // address stays inside the operands.
  const int rowsA = (M - m0) < BM ? (M - m0) : BM;
  const int rowsB = (N - n0) < BN ? (N - n0) : BN;
  const auto rsA = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A) + (int64_t)m0 * K, 0,
                                                    rowsA * K * 2, kRawBufferWord3);
  const auto rsB = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(B) + (int64_t)n0 * K, 0,
                                                    rowsB * K * 2, kRawBufferWord3);
  const int gr = tid >> 3, gc = tid & 7;
  int voffA[8], voffB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = gr + 32 * i;
    voffA[i] = (r < rowsA ? r : rowsA - 1) * (K * 2) + gc * 16;
    voffB[i] = (r < rowsB ? r : rowsB - 1) * (K * 2) + gc * 16;
  }
  const uint32_t soff0 = gr * ROWB + ((gc ^ wt_swz(gr)) << 4);

  i32x4 ra[2][8], rb[2][8];
  auto gload = [&](int set, int kt, int i0, int cnt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < i0 || i >= i0 + cnt) continue;
      ra[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rsA, voffA[i], kt * (BK * 2), 0);
      rb[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rsB, voffB[i], kt * (BK * 2), 0);
    }
  };
  auto swrite = [&](int set, int buf, int i0, int cnt) {
    unsigned char* st = lds + buf * STAGE + soff0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < i0 || i >= i0 + cnt) continue;
      *reinterpret_cast<i32x4*>(st + i * 4096) = ra[set][i];
      *reinterpret_cast<i32x4*>(st + STAGE_A + i * 4096) = rb[set][i];
    }
  };

  // Fragments: lane reads row (lane & 31) of a 32-row block, chunk 2u + (lane >> 5)
  // for K16 step u; swz depends on row bits 0..3 only, so the blocks are 4 KB
  // apart and u flips bits 5-6 of the address.
  const int hi = lane >> 5;
  const int fra0 = wm * 128 + (lane & 31), frb0 = wn * 128 + (lane & 31);
  const uint32_t fa0 = fra0 * ROWB + ((hi ^ wt_swz(fra0)) << 4);
  const uint32_t fb0 = STAGE_A + frb0 * ROWB + ((hi ^ wt_swz(frb0)) << 4);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
  bf16x8 fa[2][TM], fb[2][TN];
  auto load_frags = [&](int buf, int u, int fbuf) {
    const unsigned char* st = lds + buf * STAGE;
    const uint32_t x = (uint32_t)u << 5;
    const unsigned char* pa = st + (fa0 ^ x);
    const unsigned char* pb = st + (fb0 ^ x);
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[fbuf][i] = *reinterpret_cast<const bf16x8*>(pa + i * 4096);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[fbuf][j] = *reinterpret_cast<const bf16x8*>(pb + j * 4096);
  };
  auto mfmas = [&](int fbuf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fbuf][j], fa[fbuf][i], acc[i][j], 0, 0, 0);
  };

  // Prologue: tile 0 into LDS buffer 0, tiles 1 and 2 into register sets 1 and 0.
  gload(0, 0, 0, 8);
  swrite(0, 0, 0, 8);
  gload(1, 1, 0, 8);
  gload(0, 2, 0, 8);
  lds_barrier();
  if (m0 >= m_live) {   // no live row in this tile (the same in every wave)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }
  load_frags(0, 0, 0);

  // K step kt (LDS buffer kt & 1, register set (kt+1) & 1; the set is a
  // compile-time index, hence the loop over pairs of steps).
#define WT_K16(SET, U, I0, CNT)                          \
  mfmas((U) & 1);                                        \
  load_frags(cur, (U) + 1, ((U) + 1) & 1);               \
  swrite(SET, nxt, I0, CNT);                             \
  gload(SET, ktn, I0, CNT);                              \
  wt_interleave<2 * (CNT), 2 * (CNT), 8>();
#define WT_KSTEP(KTV, SET)                                        \
  {                                                               \
    const int cur = (KTV) & 1, nxt = cur ^ 1;                     \
    const int ktn = (KTV) + 3 < KT ? (KTV) + 3 : KT - 1;          \
    WT_K16(SET, 0, 0, 3)                                          \
    WT_K16(SET, 1, 3, 3)                                          \
    WT_K16(SET, 2, 6, 2)                                          \
    lds_barrier();                                                \
    mfmas(1);                                                     \
    load_frags(nxt, 0, 0);                                        \
    wt_interleave<0, 0, 8>();                                     \
  }
  for (int kt = 0; kt < KT; kt += 2) {
    WT_KSTEP(kt, 1)
    WT_KSTEP(kt + 1, 0)
  }
#undef WT_KSTEP
#undef WT_K16

  // Epilogue. The accumulators are read with explicit v_accvgpr_read (which
  // keeps the compiler from copying them out of the accumulation registers
  // inside the loop); the nops cover the last MFMAs' result latency.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __syncthreads();
  // kv tile in LDS: [256 rows][512 bytes], 16-byte chunk c of row r at c ^ (r & 15).
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wm * 128 + i * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[i][j][4 * g + e]));
        const uint32_t w0 = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
        const uint32_t w1 = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
        const int chunk = (wn * 16 + j * 4 + g) ^ (row & 15);
        *reinterpret_cast<uint2*>(lds + row * 512 + chunk * 16 + hi * 8) = make_uint2(w0, w1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  __syncthreads();
  for (int ch = tid; ch < BM * 32; ch += 256) {
    const int row = ch >> 5, cc = ch & 31;
    const int grow = m0 + row, gcol = n0 + cc * 8;
    if (grow < m_live && gcol < N) {
      const uint4 q = *reinterpret_cast<const uint4*>(lds + row * 512 + ((cc ^ (row & 15)) << 4));
      const u32x4 v = {q.x, q.y, q.z, q.w};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + (int64_t)grow * N + gcol));
    }
  }
}

// Shared by the skinny kernel below.
__device__ __forceinline__ void slot_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* gptr_t;


// ---------------------------------------------------------------- skinny kernel (T <= 256)
// Decode-sized T: the projection streams the 315 MB of wkv once and is bound
// by HBM, so the kernel is built to keep many wkv bytes in flight and to read
// each wkv row in long contiguous runs.
//
// vmcnt retires loads in order, so a wave that mixed a deep HBM stream with
// short L2 loads would drain the stream at every short wait; the work is
// split between waves. In each workgroup wave 0 copies the mem rows (16*MT
// padded rows) into an LDS ring of R stages with DMA; waves 1..NC each own 16
// wkv rows and load them straight into registers as 16x16x32 MFMA B
// fragments, U super-steps ahead. One barrier per super-step tells the
// consumers that a mem stage has landed and the loader that the consumers
// are done with the stage it refills.
//
// A super-step covers SK values of K (J = SK/32 MFMA K-steps). The K order
// inside a super-step is permuted identically for both operands, which leaves
// the sums unchanged: for K-step j, lane group g (lane >> 4) supplies chunk
// g*J + j (8 values). So each lane reads SK/4 contiguous bytes of its row per
// super-step and a wave asks for 16 rows x 2*SK contiguous bytes at once. In
// LDS, chunk c of mem row r sits in slot c ^ wt_swz(r) (the wave-tile
// kernel's swizzle): a 16-row fragment read then covers all sixteen 16-byte
// bank groups of a 256-byte span, since rows r and r + 8 take different
// slots. With slot c ^ (r & 7) those two rows shared banks, a 2-way conflict
// on every read, which cost 18% at T = 256 and 11% at T = 128 (same results).
//
// Read from wkv itself, each load instruction of a wave asks for 64 bytes of
// each of 16 rows 12 KB apart, and the stream runs at about 4 TB/s. PK reads
// the packed decode layout instead (pack_wkv_kernel), in which the 1 KB that
// one load instruction of a wave takes is contiguous and a wave's whole tile
// is one contiguous run, read with non-temporal loads (wkv is read once per
// call): on its own that stream reaches 6.8 TB/s against 5.0 for the strided
// one (no-compute probes, 315 MB, cold cache), and the kernel at T = 64 goes
// from 78 to 51 us with bit-identical results (same fragments, same order).
//
// On the packed layout a super-step may also span two packed super-steps (SK
// = 128): rows of 256 bytes in LDS (slot c ^ (r & 15)), half the barriers,
// and the same MFMAs in the same order, so the same bits; at T = 128 it takes
// 60 us against 66 (it gains nothing at T = 64 or at 192-256).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS slot swizzle of a mem row with CH 16-byte chunks per stage: the 16
// rows of a fragment read land in 16 distinct 16-byte bank groups.
template <int CH>
__device__ __forceinline__ int sk_swz(int r) {
  static_assert(CH == 8 || CH == 16, "rows of 128 or 256 bytes");
  if constexpr (CH == 8) return wt_swz(r);
  else return r & 15;
}

template <int MT, int NC, int R, int U, int SK, bool PK>
__global__ __launch_bounds__(64 * (NC + 1)) void skinny_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ B,
                                                               uint16_t* __restrict__ C, int M,
                                                               int N, int RW) {
  constexpr int KS = K / SK;                 // super-steps
  constexpr int J = SK / 32;                 // MFMA K-steps per super-step
  constexpr int CH = SK / 8;                 // 16-byte chunks per row per super-step
  constexpr int ROWS = MT * 16;
  constexpr int ROWB = SK * 2;               // LDS bytes per mem row per stage
  constexpr int STAGE = ROWS * ROWB;
  constexpr int INSTR = STAGE / 1024;        // 1 KB DMA instructions per stage
  static_assert(CH >= 8 && KS % U == 0 && KS > U, "super-step shape");
  static_assert(!PK || SK == kPackSK || SK == 2 * kPackSK,
                "a super-step spans one or two packed super-steps");
  constexpr int P = PK ? SK / kPackSK : 1;   // packed super-steps per super-step
  static_assert(R >= 2 && R <= 4 && (R - 2) * INSTR <= 63, "ring depth vs vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[R * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  if (wave == 0) {
    // ---- mem loader
    uint32_t off[INSTR];
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int q = i * 64 + lane, r = q / CH, sl = q % CH;
      const int c = sl ^ sk_swz<CH>(r);
      const int rr = r < M ? r : M - 1;
      off[i] = (uint32_t)rr * (K * 2) + c * 16;
    }
    const unsigned char* Ab = reinterpret_cast<const unsigned char*>(A);
    auto issue = [&](int ks) {
      unsigned char* st = lds + (ks % R) * STAGE;
#pragma unroll
      for (int i = 0; i < INSTR; ++i)
        __builtin_amdgcn_global_load_lds((gptr_t)(Ab + ks * ROWB + off[i]),
                                         (lds_ptr_t)(st + i * 1024), 16, 0, 0);
    };
#pragma unroll
    for (int ks = 0; ks < R - 1; ++ks) issue(ks);
    for (int ks = 0; ks < KS; ++ks) {
      // stages ks+1 .. ks+R-2 may stay in flight
      const int newer = (KS - 1 - ks) < (R - 2) ? (KS - 1 - ks) : (R - 2);
      if constexpr (R == 4) {
        if (newer == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * INSTR) : "memory");
        else if (newer == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INSTR) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else if constexpr (R == 3) {
        if (newer == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INSTR) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      slot_barrier();
      if (ks + R - 1 < KS) issue(ks + R - 1);
    }
    return;
  }

  // ---- consumers
  // Workgroup w owns wkv rows [w*RW, w*RW + RW); rows of its last 16-row
  // tile past that range re-read its last row (same lines: no extra HBM
  // traffic) and are not stored.
  const int base = blockIdx.x * RW;
  const int lim = (base + RW) < N ? (base + RW) : N;
  const int n0 = base + (wave - 1) * 16;
  const int arow = lane & 15, g = lane >> 4;
  // B offsets of this lane's chunks: k-step j of super-step ks is at
  // bp + ks * kstride + j * jstride (wkv's rows), or at bp + (P * ks + j / 2)
  // * kstride + (j % 2) * jstride (packed layout: kstride spans one packed
  // super-step).
  const uint16_t* bp;
  int jstride, kstride;
  if constexpr (PK) {
    // Tile of t_rows rows at n0, laid out [super-step][j][g][row][8 values]
    // (pack_wkv_kernel). A wave whose tile lies past the group (small N)
    // reads the group's last tile again and stores nothing: the loads stay
    // unconditional, so the compiler keeps the U super-steps of loads in
    // flight (a branch around them made it drain them at every step).
    const int lt = base + ((lim - base - 1) & ~15);   // the group's last tile
    const int tn = n0 < lim ? n0 : lt;
    const int t_rows = lim - tn < 16 ? lim - tn : 16;
    const int prow = arow < t_rows ? arow : t_rows - 1;
    bp = B + (int64_t)tn * K + (g * t_rows + prow) * 8;
    jstride = 4 * t_rows * 8;
    kstride = 2 * jstride;
  } else {
    int nr = n0 + arow;
    nr = nr < lim ? nr : lim - 1;
    bp = B + (int64_t)nr * K + g * J * 8;   // this lane's SK/4-value span
    jstride = 8;
    kstride = SK;
  }
  auto load_b = [&](int ks, int j) -> bf16x8 {
    if constexpr (PK)
      return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(
          bp + (P * ks + (j >> 1)) * kstride + (j & 1) * jstride));
    else return *reinterpret_cast<const bf16x8*>(bp + ks * kstride + j * jstride);
  };
  // LDS chunk of mem holding the K values of k-step j for lane group g: the
  // same K order as the B fragments above.
  auto chunk_of = [&](int j) -> int {
    if constexpr (PK) return (j >> 1) * 8 + g * 2 + (j & 1);
    else return g * J + j;
  };
  bf16x8 bq[U][J];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < J; ++j) bq[u][j] = load_b(u, j);
  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int ks, const bf16x8 (&b)[J]) {
    slot_barrier();
    const unsigned char* st = lds + (ks % R) * STAGE;
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int r = i * 16 + arow;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + r * ROWB + ((chunk_of(j) ^ sk_swz<CH>(r)) << 4));
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i], 0, 0, 0);
      }
    }
  };
  // Steady state: consume super-step ks from ring slot u, refill it with ks + U.
  for (int ks0 = 0; ks0 < KS - U; ks0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u;
      step(ks, bq[u]);
#pragma unroll
      for (int j = 0; j < J; ++j) bq[u][j] = load_b(ks + U, j);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) step(KS - U + u, bq[u]);

  // 16x16 accumulator layout: lane holds column lane & 15 and rows 4*(lane >> 4) + jj.
  const int col = n0 + arow;
  if (col < lim) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = i * 16 + g * 4 + jj;
        if (row < M) C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][jj]);
      }
  }
}

// One workgroup per CU, each with an equal share of wkv rows (100 of 25,600
// on 256 CUs): workgroups of a fixed 16*NC rows left CUs idle or doubly
// loaded (25,600 rows are 6.25 tiles of 16 per CU), which cost 8-22%. The
// packed layout fixes its groups (pack_group_rows: 256 groups, one per CU of
// an MI355X), so on it the workgroups are its groups.
template <int MT, int NC, int R, int U, int SK, bool PK>
hipError_t run_skinny(const uint16_t* mem, int64_t T, const uint16_t* wkv, int32_t N, uint16_t* kv,
                      hipStream_t st) {
  static_assert(16 * NC == kPackMaxGroupRows, "a workgroup holds the largest packed group");
  int rw = 0;
  if constexpr (PK) {
    rw = pack_group_rows(N);
  } else {
    int n_cu = 0;
    hipError_t e = cu_count(&n_cu);
    if (e != hipSuccess) return e;
    rw = (N + n_cu - 1) / n_cu;
    rw = rw < 16 ? 16 : (rw > 16 * NC ? 16 * NC : rw);
  }
  const int blocks = (N + rw - 1) / rw;
  skinny_kernel<MT, NC, R, U, SK, PK><<<blocks, 64 * (NC + 1), 0, st>>>(mem, wkv, kv, (int)T, N, rw);
  return hipGetLastError();
}

hipError_t run_wave_tile(const uint16_t* mem, int64_t T, const uint32_t* live_rows,
                         const uint16_t* wkv, int32_t N, uint16_t* kv, hipStream_t st) {
  const int m_tiles = (int)((T + kWTBM - 1) / kWTBM);
  const int n_tiles = (N + kWTBN - 1) / kWTBN;
  wave_tile_kernel<<<m_tiles * n_tiles, 256, 0, st>>>(mem, wkv, kv, (int)T, live_rows, N, m_tiles,
                                                      n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project(const uint16_t* mem, int64_t T, const uint32_t* live_rows,
                          const uint16_t* wkv, const uint16_t* wkv_packed, int32_t N, uint16_t* kv,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  // <MT, NC, R, U, SK> chosen by sweeps on the 25,600 x 6,144 wkv stream
  // (interleaved runs, 4 rotating copies of wkv so that none is cached).
  if (T <= kSkinnyMaxTokens && wkv_packed != nullptr) {
    const uint16_t* P = wkv_packed;
    if (T <= 16) return run_skinny<1, 7, 4, 4, 64, true>(mem, T, P, N, kv, st);
    if (T <= 32) return run_skinny<2, 7, 4, 4, 64, true>(mem, T, P, N, kv, st);
    if (T <= 64) return run_skinny<4, 7, 4, 4, 64, true>(mem, T, P, N, kv, st);
    if (T <= 128) return run_skinny<8, 7, 3, 2, 128, true>(mem, T, P, N, kv, st);
    if (T <= 192) return run_skinny<12, 7, 4, 4, 64, true>(mem, T, P, N, kv, st);
    return run_skinny<16, 7, 3, 3, 64, true>(mem, T, P, N, kv, st);
  }
  if (T <= 16) return run_skinny<1, 7, 4, 8, 64, false>(mem, T, wkv, N, kv, st);
  if (T <= 32) return run_skinny<2, 7, 4, 8, 64, false>(mem, T, wkv, N, kv, st);
  if (T <= 64) return run_skinny<4, 7, 4, 8, 64, false>(mem, T, wkv, N, kv, st);
  if (T <= 128) return run_skinny<8, 7, 4, 8, 64, false>(mem, T, wkv, N, kv, st);
  if (T <= 192) return run_skinny<12, 7, 4, 8, 64, false>(mem, T, wkv, N, kv, st);
  if (T <= kSkinnyMaxTokens) return run_skinny<16, 7, 3, 8, 64, false>(mem, T, wkv, N, kv, st);
  return run_wave_tile(mem, T, live_rows, wkv, N, kv, st);
}

// ---------------------------------------------------------------- packed decode layout
// One thread per 16-byte chunk (8 values) of wkv: chunk q of row n holds
// k = 8q .. 8q+7, which is super-step s = q / 8, lane group g = (q % 8) / 2 and
// k-step j = q % 2 of the skinny kernel's K order. Row n sits in group
// n / G (G = pack_group_rows(N)), in that group's 16-row tile starting at
// n0, which has t_rows rows (16, or fewer for a group's last tile); the chunk
// goes to value offset n0 * 6144 + (((s * 2 + j) * 4 + g) * t_rows + i) * 8 of
// the packed buffer, i = n - n0. Reads are coalesced, writes are 16-byte
// pieces of 1 KB runs; it runs once per weight load.
__global__ __launch_bounds__(256) void pack_wkv_kernel(const uint16_t* __restrict__ wkv,
                                                       uint16_t* __restrict__ out, int N, int G) {
  constexpr int QR = K / 8;   // chunks per row
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)N * QR) return;
  const int n = (int)(c / QR), q = (int)(c - (int64_t)n * QR);
  const int grp = n / G, lr = n - grp * G;
  const int glim = (N - grp * G) < G ? (N - grp * G) : G;   // rows in this group
  const int t0 = lr & ~15, i = lr & 15;
  const int t_rows = (glim - t0) < 16 ? (glim - t0) : 16;
  const int s = q >> 3, g = (q & 7) >> 1, j = q & 1;
  const int64_t n0 = (int64_t)grp * G + t0;
  const int64_t dst = n0 * K + (int64_t)((((s * 2 + j) * 4 + g) * t_rows + i) * 8);
  const uint4 v = *reinterpret_cast<const uint4*>(wkv + c * 8);
  *reinterpret_cast<uint4*>(out + dst) = v;
}

hipError_t launch_pack_wkv(const uint16_t* wkv, int32_t N, uint16_t* out, hipStream_t st) {
  static_assert(kPackSK == 64, "pack_wkv_kernel cuts K in super-steps of 64 values");
  if (N <= 0) return hipSuccess;
  const int64_t chunks = (int64_t)N * (K / 8);
  const unsigned blocks = (unsigned)((chunks + 255) / 256);
  pack_wkv_kernel<<<blocks, 256, 0, st>>>(wkv, out, N, pack_group_rows(N));
  return hipGetLastError();
}

}  // namespace engram
