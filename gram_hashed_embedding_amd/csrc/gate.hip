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
// and writes hidden back. One workgroup per token. Pass 1 forms the 3*hc
// sums (sum h^2, sum k^2, sum h*k*w per branch) with 16-byte loads; they are
// reduced across each wave with cross-lane moves, then across waves in LDS.
// Pass 2 re-reads h and v (now in L2) and writes bf16(h + g*v).

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
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

__global__ __launch_bounds__(kThreads) void gate_kernel(
    uint16_t* __restrict__ hidden, const uint16_t* __restrict__ kv, const float* __restrict__ wqk,
    const uint32_t* __restrict__ tok, int H, int hc, float eps, float dot_scale,
    float* __restrict__ gate_out) {
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool dead = tok != nullptr && tok[t] == ENGRAM_DEAD_TOKEN;
  if (dead) {
    if (gate_out != nullptr && tid < hc) gate_out[t * hc + tid] = 0.0f;
    return;
  }
  const int N = (hc + 1) * H;
  const int chunks = H / 8;
  uint16_t* h_t = hidden + t * (int64_t)hc * H;
  const uint16_t* kv_t = kv + t * (int64_t)N;

  float s_hh[kMaxHc], s_kk[kMaxHc], s_hk[kMaxHc];
#pragma unroll
  for (int b = 0; b < kMaxHc; ++b) s_hh[b] = s_kk[b] = s_hk[b] = 0.0f;

  for (int c = tid; c < chunks; c += kThreads) {
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
        s_hh[b] = fmaf(h[i], h[i], s_hh[b]);
        s_kk[b] = fmaf(k[i], k[i], s_kk[b]);
        s_hk[b] = fmaf(h[i] * k[i], w[i], s_hk[b]);
      }
    }
  }

  __shared__ float red[3 * kMaxHc][kWaves];
  __shared__ float g_sh[kMaxHc];
#pragma unroll
  for (int b = 0; b < kMaxHc; ++b) {
    if (b >= hc) break;
    const float a = wave_sum(s_hh[b]), k2 = wave_sum(s_kk[b]), d = wave_sum(s_hk[b]);
    if (lane == 0) {
      red[3 * b][wave] = a;
      red[3 * b + 1][wave] = k2;
      red[3 * b + 2][wave] = d;
    }
  }
  __syncthreads();
  if (tid < hc) {
    const int b = tid;
    float a = 0.f, k2 = 0.f, d = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      a += red[3 * b][w];
      k2 += red[3 * b + 1][w];
      d += red[3 * b + 2][w];
    }
    const float inv_h = 1.0f / (float)H;
    const float r_h = 1.0f / sqrtf(a * inv_h + eps);
    const float r_k = 1.0f / sqrtf(k2 * inv_h + eps);
    const float dot = dot_scale * r_h * r_k * d;
    const float z = copysignf(sqrtf(fmaxf(fabsf(dot), 1e-6f)), dot);
    const float g = 1.0f / (1.0f + expf(-z));
    g_sh[b] = g;
    if (gate_out != nullptr) gate_out[t * hc + b] = g;
  }
  __syncthreads();

  const uint16_t* v_t = kv_t + (int64_t)hc * H;
  for (int c = tid; c < chunks; c += kThreads) {
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
                       const uint32_t* tok, int64_t T, int32_t H, int32_t hc, float eps,
                       float dot_scale, float* gate_out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  gate_kernel<<<(unsigned)T, kThreads, 0, st>>>(hidden, kv, wqk, tok, H, hc, eps, dot_scale,
                                                gate_out);
  return hipGetLastError();
}

}  // namespace engram
