// The two normalization passes of the block.
//
// pool_norm — the pooled input is RMS-normalized before the experts run (LMSYS
// blog, "MoE with pooler, unpooler and per-expert normalization"): one workgroup
// per token reads the fp32 pooler output row, reduces its sum of squares and
// writes xp = P / sqrt(mean(P^2) + eps) * g_pool in the expert GEMM's input type.
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

template <typename T>
__global__ __launch_bounds__(kThreads) void pool_norm_kernel(const float* __restrict__ P,
                                                             const float* __restrict__ g, int Dp,
                                                             float eps, T* __restrict__ xp) {
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
  T* out = xp + (int64_t)t * Dp;
  for (int c = threadIdx.x * 4; c < Dp; c += kThreads * 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + c);
    const float4 gg = *reinterpret_cast<const float4*>(g + c);
    out[c + 0] = Elem<T>::from_f32(v.x * r * gg.x);
    out[c + 1] = Elem<T>::from_f32(v.y * r * gg.y);
    out[c + 2] = Elem<T>::from_f32(v.z * r * gg.z);
    out[c + 3] = Elem<T>::from_f32(v.w * r * gg.w);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  __shared__ float scale[16];
  __shared__ int pos[16];
  __shared__ int eid[16];
  const int t = blockIdx.x;
  const int nss = p.Dp / 64;
  if (threadIdx.x < p.k) {
    const int j = threadIdx.x;
    const int a = t * p.k + j;
    const int ps = p.inv[a];
    const float* ss = p.ss + (int64_t)ps * nss;
    float s = 0.f;
    for (int q = 0; q < nss; ++q) s += ss[q];
    scale[j] = p.w[a] / sqrtf(s / (float)p.Dp + p.eps);
    pos[j] = ps;
    eid[j] = p.ids[a];
  }
  __syncthreads();
  const T* y = static_cast<const T*>(p.y);
  T* u = static_cast<T*>(p.u) + (int64_t)t * p.Dp;
  for (int c = threadIdx.x * 4; c < p.Dp; c += kThreads * 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.k; ++j) {
      const T* yr = y + (int64_t)pos[j] * p.Dp + c;
      const float4 gg = *reinterpret_cast<const float4*>(p.g_expert + (int64_t)eid[j] * p.Dp + c);
      const float s = scale[j];
      acc[0] += s * gg.x * Elem<T>::to_f32(yr[0]);
      acc[1] += s * gg.y * Elem<T>::to_f32(yr[1]);
      acc[2] += s * gg.z * Elem<T>::to_f32(yr[2]);
      acc[3] += s * gg.w * Elem<T>::to_f32(yr[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) u[c + i] = Elem<T>::from_f32(acc[i]);
  }
}

}  // namespace

hipError_t launch_pool_norm(const float* P, const float* g, int T, int Dp, float eps, void* xp,
                            bool bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(pool_norm_kernel<bf16_t>, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps,
                       static_cast<bf16_t*>(xp));
  else
    hipLaunchKernelGGL(pool_norm_kernel<float>, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps,
                       static_cast<float*>(xp));
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
