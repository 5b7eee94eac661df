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
//
// The E2M1 steps use gfx950's scaled FP4 conversions. With a scale of 1 the
// FP4 -> FP32 conversion gives the signed E2M1 values (two per instruction);
// with a power-of-two scale 2^X the FP32 -> FP4 conversion gives v / 2^X
// rounded to the E2M1 grid, ties to even, saturating at 6: on the device this
// matched that rule on every value tried (dense sweeps over [0, 8] with
// scales 2^-127 .. 2^127, both neighbours of every tie, infinities, FP32
// subnormals). Both conversions take only the exponent of the scale, so the
// UE4M3 block scale is applied by a multiply. The conversion keeps the sign of
// a negative zero (code 8) where the rule above gives code 0 (a sign bit only
// for values below zero), so negative zeros are cleared first.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

// Unsigned E4M3 (bias 7; code 0x7F is NaN, handled by the caller).
__device__ __forceinline__ float ue4m3_value(uint32_t s) {
  const uint32_t e = (s >> 3) & 15u, m = s & 7u;
  if (e == 0) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

// The two E2M1 values of byte S of w (low nibble first) as floats.
template <int S>
__device__ __forceinline__ f32x2_t fp4_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, S);
}
// w with byte S replaced by the E2M1 codes of a / sx (low nibble) and b / sx.
template <int S>
__device__ __forceinline__ uint32_t fp4_put(uint32_t w, float a, float b, float sx) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, sx, S);
}

__global__ __launch_bounds__(256) void nvfp4_to_mxfp4_kernel(const uint8_t* codes, const uint8_t* scales16,
                                                             const float* __restrict__ gscale, int64_t n_mats,
                                                             int64_t per_mat, uint8_t* out_codes,
                                                             uint8_t* __restrict__ out_scales) {
  // matrices over grid rows, each matrix's blocks over the grid's columns
  for (int64_t m = blockIdx.y; m < n_mats; m += gridDim.y) {
  const float g = gscale[m];
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < per_mat;
       bi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = m * per_mat + bi;
    // every byte is read and written once: non-temporal accesses
    const u32x4_t cwv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(codes + 16 * b));
    const uint4 cw = {cwv.x, cwv.y, cwv.z, cwv.w};
    const uint32_t s2 = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(scales16 + 2 * b));
    const uint32_t s0 = s2 & 0x7Fu, s1 = (s2 >> 8) & 0x7Fu;
    bool bad = !(fabsf(g) <= 3.402823466e38f) || s0 == 0x7Fu || s1 == 0x7Fu;
    const float sc[2] = {ue4m3_value(s0), ue4m3_value(s1)};
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // elements 2i (low nibble) and 2i + 1 of byte i = 4j + t; e2m1 * ue4m3 is
      // exact, the product with g rounds once (an fma with +0, which also turns
      // a negative zero into +0)
      const f32x2_t e[4] = {fp4_pair<0>(w[j]), fp4_pair<1>(w[j]), fp4_pair<2>(w[j]), fp4_pair<3>(w[j])};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = 4 * j + t;
        v[2 * i] = fmaf(e[t].x * sc[i >> 3], g, 0.f);
        v[2 * i + 1] = fmaf(e[t].y * sc[i >> 3], g, 0.f);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
      }
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
      // 2^X as a float (2^-127 is the subnormal 0x00400000)
      const float sx = __uint_as_float(X == -127 ? 0x00400000u : (uint32_t)(X + 127) << 23);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[j] = fp4_put<0>(o[j], v[8 * j], v[8 * j + 1], sx);
        o[j] = fp4_put<1>(o[j], v[8 * j + 2], v[8 * j + 3], sx);
        o[j] = fp4_put<2>(o[j], v[8 * j + 4], v[8 * j + 5], sx);
        o[j] = fp4_put<3>(o[j], v[8 * j + 6], v[8 * j + 7], sx);
      }
    }
    __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4_t*>(out_codes + 16 * b));
    __builtin_nontemporal_store(scale, out_scales + b);
  }
  }
}

}  // namespace

hipError_t launch_nvfp4_to_mxfp4(const uint8_t* codes, const uint8_t* scales16, const float* gscale,
                                 int64_t n_mats, int64_t rows, int64_t cols, uint8_t* out_codes,
                                 uint8_t* out_scales, hipStream_t s) {
  const int64_t per = rows * (cols / 32);
  if (n_mats == 0 || per == 0) return hipSuccess;
  // about 16384 workgroups of 256 threads in all
  const int gy = (int)(n_mats < 16384 ? n_mats : 16384);
  const int64_t want_x = (per + 255) / 256, cap_x = (16384 + gy - 1) / gy;
  const int gx = (int)(want_x < cap_x ? want_x : cap_x);
  hipLaunchKernelGGL(nvfp4_to_mxfp4_kernel, dim3(gx, gy), dim3(256), 0, s, codes, scales16, gscale, n_mats, per,
                     out_codes, out_scales);
  return hipGetLastError();
}

}  // namespace lmoe
