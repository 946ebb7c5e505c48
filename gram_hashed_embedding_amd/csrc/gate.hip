// Context gate and residual update at the layer entry.
//
// [zLLM] 第三步: per mHC branch, hidden and key each get a normalisation
// factor, their weighted dot gives the relevance score, then
//   gate = sigmoid(copysign(sqrt(max(abs(dot), 1e-6)), dot)),
//   hidden += gate * value;
// the q and k elementwise weights are stored premultiplied.
// [zLLM] 第四步 / [vLLM] How it works: positions outside the n-grams (image
// spans, DEAD) are masked and pass through unchanged.
//
// HBM-bound: per token it reads hc branches of hidden and keys plus the value
// (5 x 10 KB at H = 5,120) and writes hidden back. At H = 5,120 a persistent
// workgroup of 640 threads per CU walks the tokens, one 16-byte chunk of 8
// values per thread and branch. Each thread keeps its hidden and value chunks
// in registers, forms the 3*hc sums (sum h^2, sum k^2, sum h*k*w per branch),
// reduces them across the wave with cross-lane adds and across waves through
// LDS, then writes bf16(h + g*v) from registers, with the next token's loads
// already in flight. Streamed data uses non-temporal accesses; the norm
// weights (hc*H floats, shared by all tokens) stay in L2.

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kMaxHc = 8;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void unpack8(const uint4& q, float* f) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float gate_of(float ss_h, float ss_k, float hkw, float inv_h, float eps,
                                         float dot_scale) {
  const float r_h = 1.0f / sqrtf(ss_h * inv_h + eps);
  const float r_k = 1.0f / sqrtf(ss_k * inv_h + eps);
  const float dot = dot_scale * r_h * r_k * hkw;
  const float z = copysignf(sqrtf(fmaxf(fabsf(dot), 1e-6f)), dot);
  return 1.0f / (1.0f + expf(-z));
}

// Reduce 3*HC per-thread sums to per-branch gates in g_sh (all threads read it after).
template <int HC, int WAVES>
__device__ __forceinline__ void reduce_gates(float (&s)[3 * HC], float* red, float* g_sh, int H,
                                             float eps, float dot_scale, float* gate_out, int64_t t) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int q = 0; q < 3 * HC; ++q) {
    const float v = wave_sum(s[q]);
    if (lane == 0) red[q * WAVES + wave] = v;
  }
  __syncthreads();
  if (tid < HC) {
    float a = 0.f, k2 = 0.f, d = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      a += red[(3 * tid) * WAVES + w];
      k2 += red[(3 * tid + 1) * WAVES + w];
      d += red[(3 * tid + 2) * WAVES + w];
    }
    const float g = gate_of(a, k2, d, 1.0f / (float)H, eps, dot_scale);
    g_sh[tid] = g;
    if (gate_out != nullptr) gate_out[t * HC + tid] = g;
  }
  __syncthreads();
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte accesses: hidden and k/v are touched once.
__device__ __forceinline__ uint4 nt_load(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store(uint16_t* p, uint32_t a, uint32_t b, uint32_t c,
                                         uint32_t d) {
  const u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Register-resident, persistent variant for H = 8 * THREADS: one workgroup
// per CU walks the tokens blockIdx.x, blockIdx.x + gridDim.x, ...; thread i
// owns chunk i of every branch. While token t is reduced across the
// workgroup, the keys of its next token are already loading, and that
// token's hidden and value loads are issued right after t's stores, so the
// HBM queue stays full through the barriers (one workgroup per token, which
// idles its loads at every reduction, was 10-14% slower).
//
// The loads are never behind a branch: making them conditional cost 20%, as
// the waits at the joins drained the queue. A DEAD token, or a position past
// the end, reads the norm-weight array instead (80 KB that stay in L2), so it
// moves no HBM bytes; its sums are discarded and its hidden is not stored.
//
// kv_row, when given, maps a position to its row of kv (the projection then
// ran over the live positions only); otherwise position t reads row t. With
// live_pos and live_count as well (the live positions in order and their
// number), the workgroups walk the live rows i < *live_count instead, each
// reading kv row i and hidden position live_pos[i], so DEAD positions cost
// no steps (a DEAD step moves no HBM bytes but still waits on the
// workgroup's reduction: about 60% of a live step's time), and a last light
// pass writes their zero gates. On the multimodal prefill's 65,536-position
// chunks (56% DEAD) the gate went from 1.39 to 0.77 ms.
template <int HC, int THREADS>
__global__ __launch_bounds__(THREADS) void gate_stream_kernel(
    uint16_t* __restrict__ hidden, const uint16_t* __restrict__ kv, const float* __restrict__ wqk,
    const uint32_t* __restrict__ tok, const uint32_t* __restrict__ kv_row,
    const uint32_t* __restrict__ live_pos, const uint32_t* __restrict__ live_count, int64_t T,
    float eps, float dot_scale, float* __restrict__ gate_out) {
  constexpr int WAVES = THREADS / 64;
  constexpr int H = THREADS * 8;
  static_assert((HC + 1) * H * 2 <= HC * H * 4, "stand-in rows must fit in the norm weights");
  const int tid = threadIdx.x;
  __shared__ float red[3 * HC * WAVES];
  __shared__ float g_sh[HC];
  const uint16_t* stand_in = reinterpret_cast<const uint16_t*>(wqk);
  uint4 hq[HC], kq[HC], vq;
  const int64_t G = gridDim.x;
  auto load_k = [&](int64_t kr, bool l) {
    const uint16_t* kv_t = (l ? kv + kr * (int64_t)(HC + 1) * H : stand_in) + tid * 8;
#pragma unroll
    for (int b = 0; b < HC; ++b) kq[b] = nt_load(kv_t + b * H);
  };
  auto load_hv = [&](int64_t tt, int64_t kr, bool l) {
    const uint16_t* kv_t = (l ? kv + kr * (int64_t)(HC + 1) * H : stand_in) + tid * 8;
    const uint16_t* h_t = (l ? hidden + tt * (int64_t)HC * H : stand_in) + tid * 8;
    vq = nt_load(kv_t + HC * H);
#pragma unroll
    for (int b = 0; b < HC; ++b) hq[b] = nt_load(h_t + b * H);
  };
  // The workgroup's walk is w = blockIdx.x + it * G, over positions, or over
  // live rows (live mode). Liveness, kv row and hidden position of its steps,
  // 64 at a time: lane i of `flags`, `rows` and `hpos` holds step k0 + i
  // (0 past the end).
  const bool live_mode = live_pos != nullptr && live_count != nullptr;
  const int64_t n_walk = live_mode ? min((int64_t)*live_count, T) : T;
  const int lane = tid & 63;
  uint32_t flags = 0, rows = 0, hpos = 0;
  auto load_meta = [&](int64_t k0) {
    const int64_t w = blockIdx.x + (k0 + lane) * G;
    const bool in = w < n_walk;
    if (live_mode) {
      flags = in ? 1u : 0u;
      rows = in ? (uint32_t)w : 0u;
      hpos = in ? min(live_pos[w], (uint32_t)(T - 1)) : 0u;
    } else {
      flags = (in && (tok == nullptr || tok[w] != ENGRAM_DEAD_TOKEN)) ? 1u : 0u;
      // (clamped: a DEAD position's map entry is never used, and no entry
      // may leave kv)
      rows = kv_row == nullptr ? (uint32_t)w : (in ? min(kv_row[w], (uint32_t)(T - 1)) : 0u);
      hpos = (uint32_t)w;
    }
  };
  load_meta(0);
  auto live_at = [&](int64_t it) -> bool {
    return __builtin_amdgcn_readlane(flags, (int)(it & 63)) != 0;
  };
  auto row_at = [&](int64_t it) -> int64_t {
    return (int64_t)(uint32_t)__builtin_amdgcn_readlane(rows, (int)(it & 63));
  };
  auto pos_at = [&](int64_t it) -> int64_t {
    return (int64_t)(uint32_t)__builtin_amdgcn_readlane(hpos, (int)(it & 63));
  };

  int64_t it = 0;
  bool lv = live_at(0);
  bool lvn = live_at(1);
  int64_t kr = row_at(0), krn = row_at(1);
  int64_t t = pos_at(0), tn = pos_at(1);
  load_hv(t, kr, lv);
  load_k(kr, lv);
  for (int64_t w = blockIdx.x; w < n_walk; w += G, ++it) {
    if (((it + 2) & 63) == 0) load_meta(it + 2);
    const bool lvnn = live_at(it + 2);
    const int64_t krnn = row_at(it + 2);
    const int64_t tnn = pos_at(it + 2);
    float s[3 * HC];
#pragma unroll
    for (int b = 0; b < HC; ++b) {
      const float4 w0 = *reinterpret_cast<const float4*>(wqk + b * H + tid * 8);
      const float4 w1 = *reinterpret_cast<const float4*>(wqk + b * H + tid * 8 + 4);
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float h[8], k[8];
      unpack8(hq[b], h);
      unpack8(kq[b], k);
      s[3 * b] = s[3 * b + 1] = s[3 * b + 2] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s[3 * b] = fmaf(h[i], h[i], s[3 * b]);
        s[3 * b + 1] = fmaf(k[i], k[i], s[3 * b + 1]);
        s[3 * b + 2] = fmaf(h[i] * k[i], w[i], s[3 * b + 2]);
      }
    }
    load_k(krn, lvn);
    reduce_gates<HC, WAVES>(s, red, g_sh, H, eps, dot_scale, lv ? gate_out : nullptr, t);
    if (lv) {
      float v[8];
      unpack8(vq, v);
      uint16_t* h_t = hidden + t * (int64_t)HC * H + tid * 8;
#pragma unroll
      for (int b = 0; b < HC; ++b) {
        const float g = g_sh[b];
        float h[8];
        unpack8(hq[b], h);
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = f32_to_bf16_rne(fmaf(g, v[2 * i], h[2 * i])) |
                 (f32_to_bf16_rne(fmaf(g, v[2 * i + 1], h[2 * i + 1])) << 16);
        nt_store(h_t + b * H, o[0], o[1], o[2], o[3]);
      }
    } else if (gate_out != nullptr && tid < HC && w < T) {
      gate_out[t * HC + tid] = 0.0f;
    }
    load_hv(tn, krn, lvn);
    lv = lvn;
    lvn = lvnn;
    krn = krnn;
    t = tn;
    tn = tnn;
    __syncthreads();   // keeps the waves of the workgroup on the same token
  }
  if (live_mode && gate_out != nullptr && tok != nullptr) {
    // the DEAD positions, which the walk skipped: gate 0
    for (int64_t q = (int64_t)blockIdx.x * THREADS + tid; q < T; q += G * THREADS)
      if (tok[q] == ENGRAM_DEAD_TOKEN) {
#pragma unroll
        for (int b = 0; b < HC; ++b) gate_out[q * HC + b] = 0.0f;
      }
  }
}

// Small-T variant for H = 8 * CPT * THREADS: one workgroup per (token,
// branch), so a decode batch of 64 tokens fills 256 workgroups instead of 64.
// Each branch's gate needs only that branch's hidden and key (and every
// branch the shared value, read once per branch). Thread i owns chunks i,
// i + THREADS, ...; the sums are formed per chunk and reduced per wave in the
// same order as in gate_stream_kernel (chunk c's wave sums land where the
// 640-thread layout's waves c * WAVES + w put theirs), so the kernels give
// identical bits. CPT = 2 (320 threads) is for grids of more than three
// 640-thread workgroups per CU, which would run in two rounds: at T = 256,
// hc = 4 it takes 10.2 us against 12.0 (1,024 workgroups); at T <= 128 the
// 640-thread form is faster (5.3 against 5.5 us at T = 64, 6.7 against 7.6
// at T = 128).
template <int THREADS, int CPT>
__global__ __launch_bounds__(THREADS) void gate_branch_kernel(
    uint16_t* __restrict__ hidden, const uint16_t* __restrict__ kv, const float* __restrict__ wqk,
    const uint32_t* __restrict__ tok, const uint32_t* __restrict__ kv_row, int hc, float eps,
    float dot_scale, float* __restrict__ gate_out) {
  constexpr int WAVES = THREADS / 64;
  constexpr int H = THREADS * 8 * CPT;
  const int64_t t = blockIdx.x / hc;
  const int b = blockIdx.x - (int)t * hc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tok != nullptr && tok[t] == ENGRAM_DEAD_TOKEN) {
    if (gate_out != nullptr && tid == 0) gate_out[t * hc + b] = 0.0f;
    return;
  }
  uint16_t* h_b = hidden + (t * hc + b) * (int64_t)H;
  const int64_t T = gridDim.x / hc;
  const int64_t kr = kv_row == nullptr ? t : (int64_t)min(kv_row[t], (uint32_t)(T - 1));
  const uint16_t* kv_t = kv + kr * (int64_t)(hc + 1) * H;
  uint4 hq[CPT], kq[CPT], vq[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = (tid + c * THREADS) * 8;
    hq[c] = nt_load(h_b + e);
    kq[c] = nt_load(kv_t + b * H + e);
    vq[c] = nt_load(kv_t + hc * H + e);
  }
  __shared__ float red[3 * CPT * WAVES];
  __shared__ float g_sh[1];
  float h[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = (tid + c * THREADS) * 8;
    const float4 w0 = *reinterpret_cast<const float4*>(wqk + b * H + e);
    const float4 w1 = *reinterpret_cast<const float4*>(wqk + b * H + e + 4);
    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float k[8];
    unpack8(hq[c], h[c]);
    unpack8(kq[c], k);
    float s[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s[0] = fmaf(h[c][i], h[c][i], s[0]);
      s[1] = fmaf(k[i], k[i], s[1]);
      s[2] = fmaf(h[c][i] * k[i], w[i], s[2]);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const float v = wave_sum(s[q]);
      if (lane == 0) red[q * CPT * WAVES + c * WAVES + wave] = v;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float a = 0.f, k2 = 0.f, d = 0.f;
#pragma unroll
    for (int w = 0; w < CPT * WAVES; ++w) {
      a += red[0 * CPT * WAVES + w];
      k2 += red[1 * CPT * WAVES + w];
      d += red[2 * CPT * WAVES + w];
    }
    const float g = gate_of(a, k2, d, 1.0f / (float)H, eps, dot_scale);
    g_sh[0] = g;
    if (gate_out != nullptr) gate_out[t * hc + b] = g;
  }
  __syncthreads();
  const float g = g_sh[0];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    float v[8];
    unpack8(vq[c], v);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = f32_to_bf16_rne(fmaf(g, v[2 * i], h[c][2 * i])) |
             (f32_to_bf16_rne(fmaf(g, v[2 * i + 1], h[c][2 * i + 1])) << 16);
    nt_store(h_b + (tid + c * THREADS) * 8, o[0], o[1], o[2], o[3]);
  }
}

// Generic variant (any H % 64 == 0, hc <= 8): 256 threads, strided chunks,
// hidden and value re-read (from L2) for the residual.
constexpr int kGenThreads = 256;
__global__ __launch_bounds__(kGenThreads) void gate_generic_kernel(
    uint16_t* __restrict__ hidden, const uint16_t* __restrict__ kv, const float* __restrict__ wqk,
    const uint32_t* __restrict__ tok, const uint32_t* __restrict__ kv_row, int H, int hc, float eps,
    float dot_scale, float* __restrict__ gate_out) {
  constexpr int WAVES = kGenThreads / 64;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tok != nullptr && tok[t] == ENGRAM_DEAD_TOKEN) {
    if (gate_out != nullptr && tid < hc) gate_out[t * hc + tid] = 0.0f;
    return;
  }
  const int chunks = H / 8;
  uint16_t* h_t = hidden + t * (int64_t)hc * H;
  const int64_t kr = kv_row == nullptr ? t : (int64_t)min(kv_row[t], (uint32_t)(gridDim.x - 1));
  const uint16_t* kv_t = kv + kr * (int64_t)(hc + 1) * H;
  float s[3 * kMaxHc];
#pragma unroll
  for (int q = 0; q < 3 * kMaxHc; ++q) s[q] = 0.0f;
  for (int c = tid; c < chunks; c += kGenThreads) {
#pragma unroll
    for (int b = 0; b < kMaxHc; ++b) {
      if (b >= hc) break;
      float h[8], k[8];
      unpack8(*reinterpret_cast<const uint4*>(h_t + b * H + c * 8), h);
      unpack8(*reinterpret_cast<const uint4*>(kv_t + b * H + c * 8), k);
      const float4 w0 = *reinterpret_cast<const float4*>(wqk + b * H + c * 8);
      const float4 w1 = *reinterpret_cast<const float4*>(wqk + b * H + c * 8 + 4);
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s[3 * b] = fmaf(h[i], h[i], s[3 * b]);
        s[3 * b + 1] = fmaf(k[i], k[i], s[3 * b + 1]);
        s[3 * b + 2] = fmaf(h[i] * k[i], w[i], s[3 * b + 2]);
      }
    }
  }
  __shared__ float red[3 * kMaxHc * WAVES];
  __shared__ float g_sh[kMaxHc];
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int q = 0; q < 3 * kMaxHc; ++q) {
    if (q >= 3 * hc) break;
    const float v = wave_sum(s[q]);
    if (lane == 0) red[q * WAVES + wave] = v;
  }
  __syncthreads();
  if (tid < hc) {
    float a = 0.f, k2 = 0.f, d = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      a += red[(3 * tid) * WAVES + w];
      k2 += red[(3 * tid + 1) * WAVES + w];
      d += red[(3 * tid + 2) * WAVES + w];
    }
    const float g = gate_of(a, k2, d, 1.0f / (float)H, eps, dot_scale);
    g_sh[tid] = g;
    if (gate_out != nullptr) gate_out[t * hc + tid] = g;
  }
  __syncthreads();
  const uint16_t* v_t = kv_t + (int64_t)hc * H;
  for (int c = tid; c < chunks; c += kGenThreads) {
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(v_t + c * 8), v);
#pragma unroll
    for (int b = 0; b < kMaxHc; ++b) {
      if (b >= hc) break;
      const float g = g_sh[b];
      uint4* hp = reinterpret_cast<uint4*>(h_t + b * H + c * 8);
      float h[8];
      unpack8(*hp, h);
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16_rne(fmaf(g, v[2 * i], h[2 * i])) |
               (f32_to_bf16_rne(fmaf(g, v[2 * i + 1], h[2 * i + 1])) << 16);
      *hp = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

}  // namespace

hipError_t launch_gate(uint16_t* hidden, const uint16_t* kv, const float* wqk,
                       const uint32_t* tok, const uint32_t* kv_row, const uint32_t* live_pos,
                       const uint32_t* live_count, int64_t T, int32_t H, int32_t hc, float eps,
                       float dot_scale, float* gate_out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (H == 5120) {
    int n_cu = 0;
    hipError_t e = cu_count(&n_cu);
    if (e != hipSuccess) return e;
    if ((hc != 4 || T * hc <= 4 * (int64_t)n_cu) && T * hc <= (int64_t)INT32_MAX) {
      // decode-sized batches (and other branch counts): a workgroup per (token, branch)
      const unsigned grid = (unsigned)(T * hc);
      if (T * hc > 3 * (int64_t)n_cu)
        gate_branch_kernel<320, 2><<<grid, 320, 0, st>>>(hidden, kv, wqk, tok, kv_row, hc, eps,
                                                         dot_scale, gate_out);
      else
        gate_branch_kernel<640, 1><<<grid, 640, 0, st>>>(hidden, kv, wqk, tok, kv_row, hc, eps,
                                                         dot_scale, gate_out);
      return hipGetLastError();
    }
    if (hc == 4) {
      // one resident workgroup per CU (the kernel keeps two tokens' loads in
      // registers, so a second workgroup would not fit beside it)
      const unsigned grid = (unsigned)(T < n_cu ? T : n_cu);
      gate_stream_kernel<4, 640><<<grid, 640, 0, st>>>(hidden, kv, wqk, tok, kv_row, live_pos,
                                                       live_count, T, eps, dot_scale, gate_out);
      return hipGetLastError();
    }
  }
  gate_generic_kernel<<<(unsigned)T, kGenThreads, 0, st>>>(hidden, kv, wqk, tok, kv_row, H, hc,
                                                           eps, dot_scale, gate_out);
  return hipGetLastError();
}

}  // namespace engram
