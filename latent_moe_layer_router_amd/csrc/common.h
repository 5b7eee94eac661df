// Shared device helpers of the HIP path (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

typedef uint16_t bf16_t;  // bfloat16 storage (bits)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Element type traits: T is float or bf16_t. Every row of a GEMM operand is
// read in 16-byte chunks (8 bf16 or 4 fp32 elements).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Value of an fp32 accumulator rounded to the storage type, back as float.
template <typename T> __device__ __forceinline__ float round_to(float v);
template <> __device__ __forceinline__ float round_to<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float v) {
  return bf16_to_f32(f32_to_bf16(v));
}

// Wave-wide sum (all 64 lanes receive the result).
// 16-byte load marked non-temporal: for data read exactly once (streamed
// weights), so it neither displaces reused lines from the caches nor waits on
// their allocation. On MI355X a plain streaming read reaches about 7.1 TB/s
// this way against about 6.2 TB/s with ordinary loads.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4*>(p)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace lmoe
