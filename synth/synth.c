/*
 * Seeded synthetic-input generator for the latent-MoE block.
 *
 * This file only draws random numbers; it holds none of the block's arithmetic.
 * Both the HIP path and the CPU oracle consume the arrays it writes, so the two
 * sides always see bit-identical inputs.
 *
 * Generator: counter-based. Every (seed, stream) pair names an independent
 * stream, and element i of a stream is a pure function of (seed, stream, i),
 * so any slice (one expert's weights, one token's row) can be regenerated on
 * its own and in parallel.
 *   - bits:    the SplitMix64 output function (Steele, Lea & Flood, "Fast
 *              splittable pseudorandom number generators", OOPSLA 2014) applied
 *              to a Weyl sequence keyed by (seed, stream);
 *   - normals: the Box-Muller transform (Box & Muller, 1958) on two 24-bit
 *              uniforms in (0, 1); pair p of a stream yields elements 2p, 2p+1;
 *   - bf16:    round-to-nearest-even of the fp32 value (NaN cannot occur).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Key of a stream: the seed and the stream id pass through the mixer separately
   so that nearby (seed, stream) pairs land far apart. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * SYNTH_GOLDEN + 0x2545F4914F6CDD1Dull) ^ mix64(stream + 0x632BE59BD9B4E019ull);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = { f };
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* 64 random bits for counter c of the stream with key `key`. */
uint64_t synth_bits(uint64_t seed, uint64_t stream, uint64_t c) {
  return mix64(stream_key(seed, stream) + (c + 1) * SYNTH_GOLDEN);
}

enum { SYNTH_CHUNK = 1024 };  /* pairs per work item; chunks start at multiples of this */

/* Normals for the pairs [p, p + SYNTH_CHUNK) of the stream with key `key`, into
   z[0 .. 2 * SYNTH_CHUNK). Every chunk is computed whole and chunk-aligned, so an
   element's value never depends on which slice of the stream was requested. The
   steps run as separate fixed-length loops so that each one vectorizes the same way. */
static void normal_chunk(uint64_t key, uint64_t p, float* z) {
  float u1[SYNTH_CHUNK], u2[SYNTH_CHUNK], r[SYNTH_CHUNK], c[SYNTH_CHUNK], s[SYNTH_CHUNK];
  const float two_pi = 6.283185307179586f;
  for (int q = 0; q < SYNTH_CHUNK; ++q) {
    uint64_t h = mix64(key + (p + (uint64_t)q + 1) * SYNTH_GOLDEN);
    u1[q] = ((float)(int32_t)(uint32_t)(h >> 40) + 0.5f) * 5.9604644775390625e-8f;   /* 2^-24 */
    u2[q] = two_pi * (((float)(int32_t)(uint32_t)((h >> 8) & 0xFFFFFFu) + 0.5f) * 5.9604644775390625e-8f);
  }
  for (int q = 0; q < SYNTH_CHUNK; ++q) r[q] = sqrtf(-2.0f * logf(u1[q]));
  for (int q = 0; q < SYNTH_CHUNK; ++q) c[q] = cosf(u2[q]);
  for (int q = 0; q < SYNTH_CHUNK; ++q) s[q] = sinf(u2[q]);
  for (int q = 0; q < SYNTH_CHUNK; ++q) {
    z[2 * q] = r[q] * c[q];
    z[2 * q + 1] = r[q] * s[q];
  }
}

/* Elements [first, first + n) of the N(shift, scale^2) stream (seed, stream).
   out_kind: 0 -> float32, 1 -> bfloat16 bits (uint16). */
void synth_normal(uint64_t seed, uint64_t stream, uint64_t first, size_t n,
                  float scale, float shift, int out_kind, void* out) {
  if (n == 0) return;
  const uint64_t key = stream_key(seed, stream);
  const uint64_t per = 2 * (uint64_t)SYNTH_CHUNK;          /* elements per chunk */
  const uint64_t c0 = first / per, c1 = (first + n + per - 1) / per;
#pragma omp parallel for schedule(static)
  for (long long ci = (long long)c0; ci < (long long)c1; ++ci) {
    float z[2 * SYNTH_CHUNK];
    uint64_t e0 = (uint64_t)ci * per;                       /* first element of the chunk */
    normal_chunk(key, e0 / 2, z);
    uint64_t lo = e0 < first ? first : e0;
    uint64_t hi = e0 + per > first + n ? first + n : e0 + per;
    for (uint64_t i = lo; i < hi; ++i) {
      float v = shift + scale * z[i - e0];
      if (out_kind == 0) ((float*)out)[i - first] = v;
      else ((uint16_t*)out)[i - first] = f32_to_bf16_rne(v);
    }
  }
}

/* Elements [first, first + n) of a uniform stream in [0, 1) with 53-bit resolution. */
void synth_uniform(uint64_t seed, uint64_t stream, uint64_t first, size_t n, double* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (long long q = 0; q < (long long)n; ++q) {
    uint64_t h = mix64(key + (first + (uint64_t)q + 1) * SYNTH_GOLDEN);
    out[q] = (double)(h >> 11) * 1.1102230246251565e-16; /* 2^-53 */
  }
}

/* Round an fp32 array to bf16 bits (RNE). */
void synth_f32_to_bf16(const float* in, size_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* E2M1 code of a magnitude a in [0, 8) (already divided by the block scale):
   nearest grid value of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code,
   saturating at 6. Written as exact float threshold tests. */
static uint8_t e2m1_code_of(float a) {
  if (a <= 0.25f) return 0;
  if (a < 0.75f) return 1;
  if (a <= 1.25f) return 2;
  if (a < 1.75f) return 3;
  if (a <= 2.5f) return 4;
  if (a < 3.5f) return 5;
  if (a <= 5.0f) return 6;
  return 7;
}

/* n normals N(0, scale^2) of stream (seed, stream), stored in MXFP4 form: one
   E8M0 scale per 32 consecutive values (shared exponent floor(log2(amax)) - 2)
   and E2M1 codes, element 2i in the low nibble of codes[i/2]. n % 32 == 0. */
void synth_mxfp4_normal(uint64_t seed, uint64_t stream, size_t n, float scale,
                        uint8_t* codes, uint8_t* scales) {
  float* v = (float*)malloc(sizeof(float) * n);
  synth_normal(seed, stream, 0, n, scale, 0.0f, 0, v);
#pragma omp parallel for schedule(static)
  for (long long b = 0; b < (long long)(n / 32); ++b) {
    const float* blk = v + 32 * b;
    uint32_t amax_bits = 0;
    for (int i = 0; i < 32; ++i) {
      union { float f; uint32_t u; } c = { blk[i] };
      uint32_t m = c.u & 0x7FFFFFFFu;
      if (m > amax_bits) amax_bits = m;
    }
    int X = (amax_bits == 0) ? -127 : (int)(amax_bits >> 23) - 127 - 2;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    scales[b] = (uint8_t)(X + 127);
    for (int i = 0; i < 32; i += 2) {
      uint8_t c0 = e2m1_code_of(ldexpf(fabsf(blk[i]), -X)) | (blk[i] < 0 ? 8 : 0);
      uint8_t c1 = e2m1_code_of(ldexpf(fabsf(blk[i + 1]), -X)) | (blk[i + 1] < 0 ? 8 : 0);
      codes[(32 * b + i) / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
  free(v);
}
