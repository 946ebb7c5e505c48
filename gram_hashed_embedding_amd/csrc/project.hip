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
// row) is one 16-byte LDS read. The workgroup tile is BM x BN x 64 with 4
// waves in a 2 x 2 grid; tiles are double-buffered in LDS with one barrier
// per K step. Workgroups are renumbered so that each XCD (which owns an L2)
// receives a contiguous range of tiles, and tiles are visited in groups of
// kGroupM row-tiles so concurrently running workgroups share both operands
// in L2.

#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int K = ENGRAM_MEM;
constexpr int BK = 64;
constexpr int kPad = 8;                 // bf16 elements of row padding in LDS
constexpr int kLds = BK + kPad;         // LDS row stride (elements)
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void project_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ B,
                                                           uint16_t* __restrict__ C, int M, int N,
                                                           int m_tiles, int n_tiles) {
  constexpr int TM = BM / 64;           // 32x32 MFMA tiles per wave along M
  constexpr int TN = BN / 64;           // ... along N
  constexpr int A_CH = BM * (BK / 8) / kThreads;   // 16-byte chunks per thread per K step
  constexpr int B_CH = BN * (BK / 8) / kThreads;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * kLds];

  // ---- tile assignment: XCD-contiguous, then grouped along M
  const int total = m_tiles * n_tiles;
  const int pid = blockIdx.x;
  const int per = total / kXcds, rem = total % kXcds;
  const int x = pid % kXcds, l = pid / kXcds;
  const int logical = x * per + (x < rem ? x : rem) + l;
  const int group_span = kGroupM * n_tiles;
  const int first_m = (logical / group_span) * kGroupM;
  const int gm = (m_tiles - first_m) < kGroupM ? (m_tiles - first_m) : kGroupM;
  const int in_group = logical % group_span;
  const int m0 = (first_m + in_group % gm) * BM;
  const int n0 = (in_group / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  uint4 ra[A_CH], rb[B_CH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int ch = tid + i * kThreads, row = ch >> 3, kc = ch & 7;
      const int gr = m0 + row;
      ra[i] = gr < M ? *reinterpret_cast<const uint4*>(A + (int64_t)gr * K + kt * BK + kc * 8)
                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int ch = tid + i * kThreads, row = ch >> 3, kc = ch & 7;
      const int gr = n0 + row;
      rb[i] = gr < N ? *reinterpret_cast<const uint4*>(B + (int64_t)gr * K + kt * BK + kc * 8)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int ch = tid + i * kThreads, row = ch >> 3, kc = ch & 7;
      *reinterpret_cast<uint4*>(&sA[buf][row * kLds + kc * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int ch = tid + i * kThreads, row = ch >> 3, kc = ch & 7;
      *reinterpret_cast<uint4*>(&sB[buf][row * kLds + kc * 8]) = rb[i];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  constexpr int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(
            &sA[cur][(wm * (BM / 2) + i * 32 + frag_row) * kLds + kk * 16 + frag_k]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(
            &sB[cur][(wn * (BN / 2) + j * 32 + frag_row) * kLds + kk * 16 + frag_k]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 32x32 accumulator layout: lane holds column lane%32 and
  // rows 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / 2) + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M && col < N) C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
      }
    }
}

template <int BM, int BN>
hipError_t run(const uint16_t* mem, int64_t T, const uint16_t* wkv, int32_t N, uint16_t* kv,
               hipStream_t st) {
  const int m_tiles = (int)((T + BM - 1) / BM);
  const int n_tiles = (N + BN - 1) / BN;
  project_kernel<BM, BN><<<m_tiles * n_tiles, kThreads, 0, st>>>(mem, wkv, kv, (int)T, N,
                                                                  m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project(const uint16_t* mem, int64_t T, const uint16_t* wkv, int32_t N,
                          uint16_t* kv, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (T <= 64) return run<64, 64>(mem, T, wkv, N, kv, st);
  return run<128, 128>(mem, T, wkv, N, kv, st);
}

}  // namespace engram
