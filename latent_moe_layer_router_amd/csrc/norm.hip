// The two normalization passes of the block.
//
// pool_norm — the pooled input is RMS-normalized before the experts run (LMSYS
// blog, "MoE with pooler, unpooler and per-expert normalization"): one workgroup
// per token reads the fp32 pooler output row, reduces its sum of squares and
// writes xp = P / sqrt(mean(P^2) + eps) * g_pool in the expert GEMM's input type,
// one row per token (the expert GEMMs gather the rows of their assignments).
//
// combine — the finalize step of the blog's "AMD support" section (unpermute +
// per-expert RMSNorm + weighted sum, one kernel). Each slot's scale is
// w_j / sqrt(mean(y^2) + eps), the mean coming from the down GEMM's
// per-64-column partial sums of squares of the stored values ("Fused per-expert
// post-norm"). A workgroup takes 1024 columns of one token: it computes the
// token's k slot scales, gathers its k expert rows from their sorted positions,
// multiplies each by its scale and that expert's gamma, and sums in fp32 in
// slot order j = 0..k-1 ("Miles" RL backend: FP32 weighted sum).
#include "common.h"
#include "kernels.h"
#include "mx.h"
#include "route.h"

namespace lmoe {

namespace {

constexpr int kThreads = 256;

template <int NT = kThreads>
__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) s += red[i];
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
// Store 4 consecutive values as bf16 (one 8-byte store) or fp32 (one 16-byte).
__device__ __forceinline__ void store4(bf16_t* dst, const float4& v) {
  *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                                              (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16));
}
__device__ __forceinline__ void store4(float* dst, const float4& v) { *reinterpret_cast<float4*>(dst) = v; }

// Rows of up to 4 NT kRowChunks values stay in registers between the sum of
// squares and the scaling, so P is read once: thread i holds the 16-byte chunks
// i + NT j of the row, in the order the sum of squares takes them either way.
constexpr int kRowChunks = 8;

// Normalize one fp32 row of P (the calling workgroup's NT threads) into xp.
template <int NT, typename T>
__device__ __forceinline__ void pool_norm_row(const float* __restrict__ row, const float* __restrict__ g,
                                              int Dp, float eps, T* __restrict__ out, float* red) {
  if (Dp <= 4 * NT * kRowChunks) {
    float4 v[kRowChunks];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
      const int c = 4 * (threadIdx.x + NT * j);
      if (c < Dp) {
        v[j] = *reinterpret_cast<const float4*>(row + c);
        ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
      }
    }
    ss = block_sum<NT>(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)Dp + eps);
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
      const int c = 4 * (threadIdx.x + NT * j);
      if (c < Dp) {
        const float4 gg = *reinterpret_cast<const float4*>(g + c);
        store4(out + c, make_float4(v[j].x * r * gg.x, v[j].y * r * gg.y, v[j].z * r * gg.z, v[j].w * r * gg.w));
      }
    }
    return;
  }
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < Dp; c += NT * 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum<NT>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)Dp + eps);
  for (int c = threadIdx.x * 8; c < Dp; c += NT * 8) {
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
    store8(out + c, v);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void pool_norm_kernel(const float* __restrict__ P,
                                                             const float* __restrict__ g, int Dp,
                                                             float eps, T* __restrict__ xp) {
  __shared__ float red[kThreads / kWave];
  const int t = blockIdx.x;
  pool_norm_row<kThreads>(P + (int64_t)t * Dp, g, Dp, eps, xp + (int64_t)t * Dp, red);
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
    w[d] = mx_e4m3_code4(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3], X);
  reinterpret_cast<uint4*>(codes)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  reinterpret_cast<uint4*>(codes)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  *scale = mx_scale_code(X);
}

// MX variant of pool_norm (MXFP4-expert path): the normalized row is quantized
// to MXFP8 E4M3 blocks of 32 (codes [T][Dp], scales [T][Dp/32]) as the experts'
// input. One thread per block after the row's sum of squares.
template <int NT>
__device__ __forceinline__ void pool_norm_mx_row(const float* __restrict__ row, const float* __restrict__ g,
                                                 int Dp, float eps, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, float* red) {
  if (Dp <= 4 * NT * kRowChunks) {
    // the row in registers as in pool_norm_row; an MXFP8 block of 32 values is
    // the chunks of 8 consecutive lanes (NT j is a multiple of 8 and Dp of
    // 32, so a block's 8 lanes are active together): its largest magnitude
    // over those lanes, then each lane's 4 codes in one 32-bit store
    float4 v[kRowChunks];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
      const int c = 4 * (threadIdx.x + NT * j);
      if (c < Dp) {
        v[j] = *reinterpret_cast<const float4*>(row + c);
        ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
      }
    }
    ss = block_sum<NT>(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)Dp + eps);
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
      const int c = 4 * (threadIdx.x + NT * j);
      if (c < Dp) {
        const float4 gg = *reinterpret_cast<const float4*>(g + c);
        const float x0 = v[j].x * r * gg.x, x1 = v[j].y * r * gg.y, x2 = v[j].z * r * gg.z, x3 = v[j].w * r * gg.w;
        float amax = fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3)));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        const int X = mx_e4m3_exponent(amax);
        *reinterpret_cast<uint32_t*>(codes + c) = mx_e4m3_code4(x0, x1, x2, x3, X);
        if ((threadIdx.x & 7) == 0) scales[c / 32] = mx_scale_code(X);
      }
    }
    return;
  }
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < Dp; c += NT * 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum<NT>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)Dp + eps);
  for (int b = threadIdx.x; b < Dp / 32; b += NT) {
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
    mx_store_block(v, codes + 32 * b, scales + b);
  }
}

__global__ __launch_bounds__(kThreads) void pool_norm_mx_kernel(const float* __restrict__ P,
                                                                const float* __restrict__ g, int Dp,
                                                                float eps, uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
  __shared__ float red[kThreads / kWave];
  const int t = blockIdx.x;
  pool_norm_mx_row<kThreads>(P + (int64_t)t * Dp, g, Dp, eps, codes + (int64_t)t * Dp,
                             scales + (int64_t)t * (Dp / 32), red);
}

// Small batches (router + pooler by split-K): one workgroup per token adds the
// token's split-K partials in slice order (the pooler columns to P, the router
// columns plus bias to the logits), then normalizes its P row into xp — the
// reduction, the pooled norm and (MXFP4 experts) the quantization in one pass.
// 1024 threads, so that the token's columns take about one pass of 4 per
// thread, with the slice loads of a pass in flight together. The barrier
// after the reduction orders the P columns before the norm reads them.
constexpr int kSplitNormThreads = 1024;

template <int MODE>   // 0: bf16 xp, 2: MXFP8 codes + scales
__global__ __launch_bounds__(kSplitNormThreads) void splitk_pool_norm_kernel(DenseStreamParams d, int part_ld,
                                                                            const float* __restrict__ g,
                                                                            float eps, void* xp,
                                                                            uint8_t* __restrict__ scales,
                                                                            TopkOut tk) {
  constexpr int NT = kSplitNormThreads;
  __shared__ float red[NT / kWave];
  // With the top-k, workgroups T .. 2T - 1 take the logit columns and the
  // top-k of token blockIdx.x - T, beside the pooled-row workgroups (the two
  // run at once instead of one after the other).
  const bool topk_role = tk.ids && (int)blockIdx.x >= d.T;
  const int t = topk_role ? blockIdx.x - d.T : blockIdx.x;
  const int lo = topk_role ? d.n_split : 0, hi = (tk.ids && !topk_role) ? d.n_split : d.N;
  const int64_t plane = (int64_t)d.T * part_ld;
  float* P = static_cast<float*>(d.out0) + (int64_t)t * d.ldo0;
  for (int n0 = lo + threadIdx.x * 4; n0 < hi; n0 += NT * 4) {
    const float* src = d.part + (int64_t)t * part_ld + n0;
    float4 s = *reinterpret_cast<const float4*>(src);
#pragma unroll 8
    for (int sl = 1; sl < d.slices; ++sl) {
      const float4 v = *reinterpret_cast<const float4*>(src + sl * plane);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = n0 + e;
      if (n >= hi) break;
      if (n < d.n_split) {
        P[n] = sv[e];
      } else {
        const int c = n - d.n_split;
        d.out1[(int64_t)t * d.ldo1 + c] = sv[e] + (d.bias1 ? d.bias1[c] : 0.f);
      }
    }
  }
  __syncthreads();                           // (uniform: a workgroup has one role)
  if (topk_role) {
    // the token's top-k on the logits this workgroup wrote before the barrier
    if (threadIdx.x < kWave)
      topk_token(d.out1 + (int64_t)t * d.ldo1, t, d.N - d.n_split, tk.k, tk.ids, tk.w, tk.chunk_masks);
    return;
  }
  const int Dp = d.n_split;
  if (MODE == 2)
    pool_norm_mx_row<NT>(P, g, Dp, eps, static_cast<uint8_t*>(xp) + (int64_t)t * Dp,
                         scales + (int64_t)t * (Dp / 32), red);
  else
    pool_norm_row<NT>(P, g, Dp, eps, static_cast<bf16_t*>(xp) + (int64_t)t * Dp, red);
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

// One workgroup per (1024-column chunk, token). With the first y words in
// flight, it computes the token's k slot scales, w_j / sqrt(mean(y_j^2) + eps), the mean from the row's partial
// sums of squares: 16 threads per slot, thread q adding partials q, q + 16, ...,
// then a butterfly over the 16; the scales go through LDS. A thread then sums 8
// consecutive columns over the k slots in slot order. The workgroups of one
// token are adjacent (its partials are read from L2 after the first), token t
// starting at chunk t mod (Dp / 1024): the rows being read at any time spread
// over all column offsets (and so over all HBM channels; all workgroups on one
// chunk measured 10% slower).
constexpr int kCombineThreads = 128, kCombineCols = kCombineThreads * 8, kMaxSlots = 16;

// The slots' loads are all issued before any is used: raw 16-byte words per
// slot (converted to fp32 only when summed, so each load keeps registers of its
// own and stays in flight).
__device__ __forceinline__ uint4 load16_once(const void* src) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  return make_uint4(q.x, q.y, q.z, q.w);
}
__device__ __forceinline__ void widen8(const uint4& q, float (&v)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// 8 columns of up to 8 slots j0 .. j0 + 7: the y words and the experts' gammas.
template <typename T>
struct SlotWords {
  uint4 y[8][8 * sizeof(T) / 16];
  float4 g0[8], g1[8];
};

template <typename T>
__device__ __forceinline__ void combine_load(const CombineParams& p, int t, int c, int j0, SlotWords<T>& w) {
  constexpr int VW = 16 / sizeof(T);       // values per 16-byte word of y
  const T* y = static_cast<const T*>(p.y);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    if (j0 + jj < p.k) {
      const int pos = p.inv[t * p.k + j0 + jj], eid = p.ids[t * p.k + j0 + jj];
      const T* yrow = y + (int64_t)pos * p.Dp + c;
#pragma unroll
      for (int h = 0; h < 8 / VW; ++h) w.y[jj][h] = load16_once(yrow + h * VW);
      const float4* gp = reinterpret_cast<const float4*>(p.g_expert + (int64_t)eid * p.Dp + c);
      w.g0[jj] = gp[0];
      w.g1[jj] = gp[1];
    }
  }
}

template <typename T>
__device__ __forceinline__ void combine_add(const CombineParams& p, const float* sc, int j0, const SlotWords<T>& w,
                                            float (&acc)[8]) {
  constexpr int VW = 16 / sizeof(T);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    if (j0 + jj < p.k) {
      const float sj = sc[j0 + jj];
      float yv[8];
      if constexpr (VW == 8) {
        widen8(w.y[jj][0], yv);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          yv[4 * h] = __uint_as_float(w.y[jj][h].x);
          yv[4 * h + 1] = __uint_as_float(w.y[jj][h].y);
          yv[4 * h + 2] = __uint_as_float(w.y[jj][h].z);
          yv[4 * h + 3] = __uint_as_float(w.y[jj][h].w);
        }
      }
      const float gv[8] = {w.g0[jj].x, w.g0[jj].y, w.g0[jj].z, w.g0[jj].w,
                           w.g1[jj].x, w.g1[jj].y, w.g1[jj].z, w.g1[jj].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += sj * gv[i] * yv[i];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineParams p) {
  __shared__ float sc[kMaxSlots];
  const int nchunk = (p.Dp + kCombineCols - 1) / kCombineCols;
  const int t = blockIdx.x / nchunk, chunk = (blockIdx.x + t) % nchunk;
  const int tid = threadIdx.x, nss = p.Dp / 64;
  const int c = chunk * kCombineCols + tid * 8;
  SlotWords<T> w;
  if (c < p.Dp) combine_load<T>(p, t, c, 0, w);   // in flight while the scales are computed
  for (int j0 = 0; j0 < p.k; j0 += kCombineThreads / 16) {
    const int j = j0 + (tid >> 4), q0 = tid & 15;
    float s = 0.f;
    if (j < p.k) {
      const int a = t * p.k + j;
      const float* ss = p.ss + (int64_t)p.inv[a] * nss;
      for (int q = q0; q < nss; q += 16) s += ss[q];
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (j < p.k && q0 == 0) sc[j] = p.w[t * p.k + j] / sqrtf(s / (float)p.Dp + p.eps);
  }
  __syncthreads();
  if (c >= p.Dp) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < p.k; j0 += 8) {
    if (j0) combine_load<T>(p, t, c, j0, w);
    combine_add<T>(p, sc, j0, w, acc);
  }
  store8(static_cast<T*>(p.u) + (int64_t)t * p.Dp + c, acc);
}

}  // namespace

hipError_t launch_pool_norm(const float* P, const float* g, int T, int Dp, float eps, void* xp, bool bf16,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(pool_norm_kernel<bf16_t>, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps,
                       static_cast<bf16_t*>(xp));
  else
    hipLaunchKernelGGL(pool_norm_kernel<float>, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps,
                       static_cast<float*>(xp));
  return hipGetLastError();
}

hipError_t launch_pool_norm_mx(const float* P, const float* g, int T, int Dp, float eps, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_norm_mx_kernel, dim3(T), dim3(kThreads), 0, s, P, g, Dp, eps, codes, scales);
  return hipGetLastError();
}

hipError_t launch_splitk_pool_norm(const DenseStreamParams& d, const float* g, float eps, void* xp, int mode,
                                   uint8_t* scales, const TopkOut& tk, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  if (d.out0_bf16 || d.n_split % 64 || d.N < d.n_split || (mode == 2 && !scales)) return hipErrorInvalidValue;
  if (tk.ids && (d.ldo1 != d.N - d.n_split || !tk.w || !tk.chunk_masks)) return hipErrorInvalidValue;
  const int ld = dense_stream_part_ld(d.N);
  if (mode == 0)
    hipLaunchKernelGGL(splitk_pool_norm_kernel<0>, dim3(tk.ids ? 2 * d.T : d.T), dim3(kSplitNormThreads), 0, s, d,
                       ld, g, eps, xp, scales, tk);
  else if (mode == 2)
    hipLaunchKernelGGL(splitk_pool_norm_kernel<2>, dim3(tk.ids ? 2 * d.T : d.T), dim3(kSplitNormThreads), 0, s, d,
                       ld, g, eps, xp, scales, tk);
  else
    return hipErrorInvalidValue;
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
  if (p.k > kMaxSlots || p.Dp % 64) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)((p.Dp + kCombineCols - 1) / kCombineCols) * p.T;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3((unsigned)grid), dim3(kCombineThreads), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)grid), dim3(kCombineThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace lmoe
