// OCP Microscaling (MX) helpers for the MXFP4-expert path: MXFP8 E4M3
// quantization of activations (blocks of 32 values along the row, one E8M0
// scale each) and the gfx950 scaled-MFMA operand conventions.
//
// The MXFP4 format (E2M1 values with one UE8M0 scale per 32 elements) is the
// one the LMSYS Muse Spark Open blog names in "NVFP4 as a third MMA type"; the
// element and scale encodings follow OCP Microscaling Formats v1.0.
#pragma once

#include "common.h"

namespace lmoe {

// Shared exponent of a block of MXFP8 E4M3 values: floor(log2(amax)) minus the
// largest E4M3 exponent (8), clamped to [-127, 127]; an all-zero block takes
// -127. amax must be finite.
__device__ __forceinline__ int mx_e4m3_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF);   // biased exponent
  // floor(log2(amax)): e - 127 for normals; subnormals (e == 0) lie below
  // 2^-126, where the clamp below takes over anyway.
  int X = (e == 0 ? -127 : e - 127) - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// E4M3 code (OCP: bias 7, max 448, no infinities) of v / 2^X: nearest, ties to
// even, saturating. v / 2^X is formed exactly (a power-of-two scaling of a
// float whose result is either exact or far below the smallest E4M3 step).
// The codec's definition in plain arithmetic: the kernels call the packed
// hardware form below (mx_e4m3_code4), which was checked against this one.
__device__ __forceinline__ uint8_t mx_e4m3_code(float v, int X) {
  const float a = fabsf(v) * __uint_as_float((uint32_t)(127 - X) << 23 & 0x7F800000u);
  uint8_t code = 0;
  if (a > 0.f) {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;        // floor(log2 a) for normal a
    if (((__float_as_uint(a) >> 23) & 0xFF) == 0) e = -127;
    if (e < -6) e = -6;                                            // subnormal range: step 2^-9
    const float step = __uint_as_float((uint32_t)(e - 3 + 127) << 23);
    // a / step is a power-of-two scaling (exact either way): multiply by the
    // exact reciprocal instead of dividing
    const float inv_step = __uint_as_float((uint32_t)(3 - e + 127) << 23);
    float q = __builtin_rintf(a * inv_step) * step;                // ties to even
    if (q > 448.f) q = 448.f;
    if (q > 0.f) {
      const int qe = (int)((__float_as_uint(q) >> 23) & 0xFF) - 127;
      if (qe < -6) {
        code = (uint8_t)(int)(q * 512.f);                          // subnormal: q = m / 8 * 2^-6
      } else {
        const int m = (int)((__float_as_uint(q) >> 20) & 7);        // top 3 mantissa bits
        code = (uint8_t)(((qe + 7) << 3) | m);
      }
    }
  }
  return (uint8_t)(code | (v < 0.f ? 0x80 : 0));
}

// Four E4M3 codes of v0..v3 / 2^X, exactly as mx_e4m3_code gives them, packed
// into 32 bits (v0 in the low byte), by gfx950's packed fp8 conversion (OCP
// E4M3, to nearest, ties to even) of the scaled values with the codec's
// conventions applied first: a NaN codes as +0, magnitudes saturate at 448,
// and -0 codes as +0 (checked against mx_e4m3_code on 2^24 values at seven
// scales, edge values included).
__device__ __forceinline__ uint32_t mx_e4m3_code4(float v0, float v1, float v2, float v3, int X) {
  const float s = __uint_as_float((uint32_t)(127 - X) << 23 & 0x7F800000u);
  auto prep = [s](float v) {
    float a = v * s;
    a = (a == a) ? a : 0.f;
    return fminf(fmaxf(a, -448.f), 448.f) + 0.f;
  };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(prep(v0), prep(v1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(prep(v2), prep(v3), w, true);
  return (uint32_t)w;
}

// The scale argument of X: an E8M0 byte.
__device__ __forceinline__ uint8_t mx_scale_code(int X) { return (uint8_t)(X + 127); }

}  // namespace lmoe
