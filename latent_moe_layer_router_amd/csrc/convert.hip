// Load-time re-encoding of NVFP4 expert weights as MXFP4.
//
// NVFP4 (LMSYS blog, "NVFP4 as a third MMA type"): dense E2M1 values with one
// UE4M3 block scale per 16 elements, and one FP32 scale per weight matrix in a
// stored checkpoint. gfx950's block-scaled MFMA takes E8M0 scales per 32, and
// the blog's "AMD support" section serves the NVFP4 checkpoint on MI355X
// through the MXFP4 path ("NVFP4 Requant"). Each 32-element block is decoded to
// FP32 (e2m1 * ue4m3 is exact, the product with the matrix scale rounds to
// nearest-even) and MX-quantized (OCP Microscaling v1.0): shared exponent
// X = floor(log2(amax)) - 2, clamped to [-127, 127] (-127 for an all-zero
// block); elements v / 2^X rounded to the E2M1 grid, ties to even, saturated
// at 6. A block with a NaN scale (UE4M3 0x7F; the byte's top bit is ignored), a
// non-finite matrix scale or an FP32 overflow gets the E8M0 NaN scale 0xFF and
// zero codes.
//
// One thread per block: 16 code bytes and 2 scale bytes in, 16 code bytes and
// one scale byte out, so consecutive threads touch consecutive bytes. A thread
// reads its whole block before it writes, which lets the output codes overwrite
// the input codes in place.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

// Twice the E2M1 magnitude of code m (0..7) is the integer 0, 1, 2, 3, 4, 6, 8
// or 12: one byte permute picks it from two constant words.
__device__ __forceinline__ float e2m1_twice(uint32_t m) {
  return (float)(__builtin_amdgcn_perm(0x0C080604u, 0x03020100u, m) & 0xFFu);
}

// Unsigned E4M3 (bias 7; code 0x7F is NaN, handled by the caller).
__device__ __forceinline__ float ue4m3_value(uint32_t s) {
  const uint32_t e = (s >> 3) & 15u, m = s & 7u;
  if (e == 0) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude code of q in [0, 8): nearest, ties to even, saturating at 6.
// Below 1 the grid step is 0.5, so the code is rint(2q) (0, 1 or 2). From 1 up
// the code is the float's exponent and top mantissa bit, so rounding q's bit
// pattern to one mantissa bit (ties to even) gives it directly; 8 and above
// saturate to code 7 (6.0).
__device__ __forceinline__ uint32_t e2m1_mag_code(float q) {
  const uint32_t b = __float_as_uint(q);
  const uint32_t hi = ((b + 0x1FFFFFu + ((b >> 22) & 1u)) >> 22) - 252u;
  const uint32_t lo = (uint32_t)__builtin_rintf(q + q);
  return q < 1.f ? lo : (hi > 7u ? 7u : hi);
}

__global__ __launch_bounds__(256) void nvfp4_to_mxfp4_kernel(const uint8_t* codes, const uint8_t* scales16,
                                                             const float* __restrict__ gscale, int64_t rows,
                                                             int64_t nb, int64_t total, uint8_t* out_codes,
                                                             uint8_t* __restrict__ out_scales) {
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < total;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = b / (rows * nb);
    const float g = gscale[m];
    const uint4 cw = *reinterpret_cast<const uint4*>(codes + 16 * b);
    const uint32_t s2 = *reinterpret_cast<const uint16_t*>(scales16 + 2 * b);
    const uint32_t s0 = s2 & 0x7Fu, s1 = (s2 >> 8) & 0x7Fu;
    bool bad = !(fabsf(g) <= 3.402823466e38f) || s0 == 0x7Fu || s1 == 0x7Fu;
    // half the block scales: e2m1 * ue4m3 = (2 e2m1) * (ue4m3 / 2), both exact
    const float hsc[2] = {0.5f * ue4m3_value(s0), 0.5f * ue4m3_value(s1)};
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t c = (w[i >> 3] >> (4 * (i & 7))) & 15u;
      const float mag = e2m1_twice(c & 7u) * hsc[i >> 4];
      const float p = __uint_as_float(__float_as_uint(mag) ^ ((c & 8u) << 28));
      v[i] = p * g;
      amax = fmaxf(amax, fabsf(v[i]));
    }
    if (!(amax <= 3.402823466e38f)) bad = true;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    uint8_t scale = 0xFF;
    if (!bad) {
      int X = -127;
      if (amax > 0.f) {
        const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF);
        X = (e == 0 ? -127 : e - 127) - 2;
        X = X < -127 ? -127 : X;
      }
      scale = (uint8_t)(X + 127);
      // 2^-X for X in [-127, 125] is a normal float; |v| * 2^-X is exact (or far
      // below the grid's first step)
      const float inv = __uint_as_float((uint32_t)(127 - X) << 23);
#pragma unroll
      for (int i = 0; i < 32; ++i)
        o[i >> 3] |= (e2m1_mag_code(fabsf(v[i]) * inv) | (v[i] < 0.f ? 8u : 0u)) << (4 * (i & 7));
    }
    *reinterpret_cast<uint4*>(out_codes + 16 * b) = uint4{o[0], o[1], o[2], o[3]};
    out_scales[b] = scale;
  }
}

}  // namespace

hipError_t launch_nvfp4_to_mxfp4(const uint8_t* codes, const uint8_t* scales16, const float* gscale,
                                 int64_t n_mats, int64_t rows, int64_t cols, uint8_t* out_codes,
                                 uint8_t* out_scales, hipStream_t s) {
  const int64_t nb = cols / 32, total = n_mats * rows * nb;
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(nvfp4_to_mxfp4_kernel, dim3(grid), dim3(256), 0, s, codes, scales16, gscale, rows, nb,
                     total, out_codes, out_scales);
  return hipGetLastError();
}

}  // namespace lmoe
