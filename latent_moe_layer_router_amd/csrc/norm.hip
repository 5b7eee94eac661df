// The two normalization passes of the block.
//
// pool_norm — the pooled input is RMS-normalized before the experts run (LMSYS
// blog, "MoE with pooler, unpooler and per-expert normalization"): one workgroup
// per token reads the fp32 pooler output row, reduces its sum of squares and
// writes xp = P / sqrt(mean(P^2) + eps) * g_pool in the expert GEMM's input type
// to each of the token's k rows in the experts' sorted order.
//
// combine — the finalize step of the blog's "AMD support" section (unpermute +
// per-expert RMSNorm + weighted sum in one kernel). One workgroup per token
// gathers the token's k expert rows from their sorted positions, scales each by
// w_j / sqrt(mean(y^2) + eps) — the mean coming from the down GEMM's per-64-column
// partial sums of squares of the stored values ("Fused per-expert post-norm") —
// and by that expert's gamma, and sums in fp32 in slot order j = 0..k-1 ("Miles"
// RL backend: FP32 weighted sum).
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace lmoe {

namespace {

constexpr int kThreads = 256;

__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Store 8 consecutive values as bf16 (one 16-byte store) or fp32 (two).
__device__ __forceinline__ void store8(bf16_t* dst, const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store8(float* dst, const float (&v)[8]) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
// Load 8 consecutive fp32 values.
__device__ __forceinline__ void load8(const float* src, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// load8 with a non-temporal hint: for rows read exactly once, so that they do
// not displace lines that are read again (the experts' gammas in the combine).
__device__ __forceinline__ void load8_once(const bf16_t* src, float (&v)[8]) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8_once(const float* src, float (&v)[8]) {
  typedef __attribute__((ext_vector_type(4))) float f32x4v;
  const f32x4v a = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(src));
  const f32x4v b = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(src) + 1);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The normalized row goes to the token's k rows of the sorted (expert-major)
// order, inv[t*k + j], so that the expert GEMMs read their rows contiguously.
template <typename T>
__global__ __launch_bounds__(kThreads) void pool_norm_kernel(const float* __restrict__ P,
                                                             const float* __restrict__ g, int Dp,
                                                             float eps, const int32_t* __restrict__ inv,
                                                             int k, T* __restrict__ xp) {
  __shared__ float red[kThreads / kWave];
  const int t = blockIdx.x;
  const float* row = P + (int64_t)t * Dp;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < Dp; c += kThreads * 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)Dp + eps);
  for (int c = threadIdx.x * 8; c < Dp; c += kThreads * 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
      const float4 x = *reinterpret_cast<const float4*>(row + c + i);
      const float4 gg = *reinterpret_cast<const float4*>(g + c + i);
      v[i] = x.x * r * gg.x;
      v[i + 1] = x.y * r * gg.y;
      v[i + 2] = x.z * r * gg.z;
      v[i + 3] = x.w * r * gg.w;
    }
    for (int j = 0; j < k; ++j) store8(xp + (int64_t)inv[t * k + j] * Dp + c, v);
  }
}

// Quantize 32 values held by one thread to an MXFP8 E4M3 block: 32 code bytes
// (two 16-byte stores) and one E8M0 scale byte.
__device__ __forceinline__ void mx_store_block(const float (&v)[32], uint8_t* codes, uint8_t* scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_e4m3_exponent(amax);
  uint32_t w[8];
#pragma unroll
  for (int d = 0; d < 8; ++d)
    w[d] = (uint32_t)mx_e4m3_code(v[4 * d], X) | ((uint32_t)mx_e4m3_code(v[4 * d + 1], X) << 8) |
           ((uint32_t)mx_e4m3_code(v[4 * d + 2], X) << 16) | ((uint32_t)mx_e4m3_code(v[4 * d + 3], X) << 24);
  reinterpret_cast<uint4*>(codes)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  reinterpret_cast<uint4*>(codes)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  *scale = mx_scale_code(X);
}

// MX variant of pool_norm (MXFP4-expert path): the normalized row is quantized
// to MXFP8 E4M3 blocks of 32 (codes [T][Dp], scales [T][Dp/32]) as the experts'
// input. One thread per block after the row's sum of squares.
__global__ __launch_bounds__(kThreads) void pool_norm_mx_kernel(const float* __restrict__ P,
                                                                const float* __restrict__ g, int Dp,
                                                                float eps, const int32_t* __restrict__ inv,
                                                                int k, uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
  __shared__ float red[kThreads / kWave];
  const int t = blockIdx.x;
  const float* row = P + (int64_t)t * Dp;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < Dp; c += kThreads * 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)Dp + eps);
  for (int b = threadIdx.x; b < Dp / 32; b += kThreads) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float4 x = *reinterpret_cast<const float4*>(row + 32 * b + i);
      const float4 gg = *reinterpret_cast<const float4*>(g + 32 * b + i);
      v[i] = x.x * r * gg.x;
      v[i + 1] = x.y * r * gg.y;
      v[i + 2] = x.z * r * gg.z;
      v[i + 3] = x.w * r * gg.w;
    }
    // one quantization, stored to the token's k sorted rows
    uint8_t* c0 = codes + (int64_t)inv[t * k] * Dp + 32 * b;
    uint8_t* s0 = scales + (int64_t)inv[t * k] * (Dp / 32) + b;
    mx_store_block(v, c0, s0);
    for (int j = 1; j < k; ++j) {
      const int64_t pos = inv[t * k + j];
      reinterpret_cast<uint4*>(codes + pos * Dp + 32 * b)[0] = reinterpret_cast<const uint4*>(c0)[0];
      reinterpret_cast<uint4*>(codes + pos * Dp + 32 * b)[1] = reinterpret_cast<const uint4*>(c0)[1];
      scales[pos * (Dp / 32) + b] = *s0;
    }
  }
}

// Stand-alone MXFP8 E4M3 quantization of n fp32 values (n a multiple of 32).
__global__ __launch_bounds__(kThreads) void mx_quant_kernel(const float* __restrict__ x, int64_t nb,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nb) return;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    const float4 q = *reinterpret_cast<const float4*>(x + 32 * b + i);
    v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
  }
  mx_store_block(v, codes + 32 * b, scales + b);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  __shared__ float scale[16];
  __shared__ int pos[16];
  __shared__ int eid[16];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nss = p.Dp / 64;
  // Slot j's scale: one wave reduces the row's partial sums of squares (lane q
  // takes partials q, q + 64, ...; then a butterfly over the wave).
  for (int j = wave; j < p.k; j += kThreads / kWave) {
    const int a = t * p.k + j;
    const int ps = p.inv[a];
    const float* ss = p.ss + (int64_t)ps * nss;
    float s = 0.f;
    for (int q = lane; q < nss; q += kWave) s += ss[q];
    s = wave_sum(s);
    if (lane == 0) {
      scale[j] = p.w[a] / sqrtf(s / (float)p.Dp + p.eps);
      pos[j] = ps;
      eid[j] = p.ids[a];
    }
  }
  __syncthreads();
  const T* y = static_cast<const T*>(p.y);
  T* u = static_cast<T*>(p.u) + (int64_t)t * p.Dp;
  // 8 consecutive columns per thread; the loads of up to 8 slots are issued
  // before any is used, then the terms are added in slot order j = 0..k-1.
  for (int c = threadIdx.x * 8; c < p.Dp; c += kThreads * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < p.k; j0 += 8) {
      float yv[8][8], gv[8][8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj < p.k) {
          load8_once(y + (int64_t)pos[j0 + jj] * p.Dp + c, yv[jj]);
          load8(p.g_expert + (int64_t)eid[j0 + jj] * p.Dp + c, gv[jj]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj < p.k) {
          const float sj = scale[j0 + jj];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += sj * gv[jj][i] * yv[jj][i];
        }
      }
    }
    store8(u + c, acc);
  }
}

}  // namespace

hipError_t launch_pool_norm(const float* P, const float* g, int T, int Dp, float eps, const int32_t* inv,
                            int k, void* xp, bool bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(pool_norm_kernel<bf16_t>, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps, inv, k,
                       static_cast<bf16_t*>(xp));
  else
    hipLaunchKernelGGL(pool_norm_kernel<float>, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps, inv, k,
                       static_cast<float*>(xp));
  return hipGetLastError();
}

hipError_t launch_pool_norm_mx(const float* P, const float* g, int T, int Dp, float eps, const int32_t* inv,
                               int k, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_norm_mx_kernel, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps, inv, k, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant(const float* x, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nb = n / 32;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)((nb + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     x, nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(p.T), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(p.T), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace lmoe
