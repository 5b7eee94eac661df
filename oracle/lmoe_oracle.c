/*
 * CPU oracle for the latent mixture-of-experts block forward.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the plain, slow, obviously correct
 * definition that the GPU path is checked against. Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product path
 * never does. It shares no code, header or table with the HIP library.
 *
 * Source of the definition (the pages describing the model's MoE block):
 *  - LMSYS blog "SGLang and Miles Add Day-0 Support for Muse Spark Open", section
 *    "MoE with pooler, unpooler and per-expert normalization": a learned pooler
 *    narrows every token before the routed SwiGLU experts, the router chooses
 *    experts from the full-width representation, the pooled expert input is
 *    normalized before the experts run, each selected expert's output gets its
 *    own RMSNorm before it is scaled by its routing weight and summed, and the
 *    unpooler restores model width after the sum;
 *  - same blog, "Reinforcement learning" section: the weighted sum of expert
 *    outputs is formed in FP32;
 *  - vLLM day-0 summary, "Latent MoE": pooler 8192 x 4096 and unpooler learned
 *    projections shared by the layer's 256 experts; "Nvidia" backend notes: the
 *    router GEMM takes FP32 input and produces FP32 logits;
 *  - same blog, "NVFP4 as a third MMA type": MXFP4 = dense E2M1 values with one
 *    UE8M0 scale per 32 elements (used by the MXFP4-expert configuration).
 *
 * Arithmetic: every dot product accumulates in double. The router logits are
 * rounded to float once, because top-k selection is decided on FP32 logits; the
 * routing weights, norms and sums stay in double.
 *
 * Precision boundaries (flag `rnd`, used for the BF16 workloads): the pages fix
 * where a BF16 model holds BF16 values, and with rnd set the oracle rounds to
 * bfloat16 (nearest, ties to even) exactly there and nowhere else:
 *  - the normalized pooled input, i.e. the experts' GEMM input (BF16 expert
 *    layers; blog, "Kernel optimizations": BF16 expert loop of layers 0 and 61);
 *  - the SwiGLU output between the two expert GEMMs (same);
 *  - each expert's output row, whose RMS is taken from those BF16 values (blog,
 *    "Fused per-expert post-norm": the second GEMM's tile sums the squares of the
 *    BF16 values it holds);
 *  - the FP32 weighted sum, rounded once as the unpooler's BF16 GEMM input
 *    (blog, "Reinforcement learning": the sum itself is FP32).
 * The block output itself is not rounded. In MX mode the expert input and the
 * SwiGLU output are MXFP8-quantized at those points instead of rounded to BF16.
 *
 * Readings of points the pages leave open (each is a choice, stated once here):
 *  - routing weights are the softmax of the k selected logits;
 *  - top-k order is logit descending, ties to the lower expert index;
 *  - RMSNorm(v) = v / sqrt(mean(v^2) + eps) * gamma, mean over the vector's width;
 *  - SwiGLU(x) = silu(x . W_gate^T) * (x . W_up^T), gate = rows [0, F) of the
 *    packed gate/up matrix and up = rows [F, 2F);
 *  - no biases in the projections; an optional per-expert router bias is added to
 *    the logits and used for both selection and weights;
 *  - MX quantization (OCP Microscaling v1.0): per 32-element block the shared
 *    exponent is floor(log2(amax)) - emax_elem, clamped to [-127, 127]; elements
 *    are v / 2^X rounded to nearest-even and saturated; an all-zero block takes
 *    the smallest scale.
 *
 * Layouts: row-major; weights are [out][in] (K-contiguous). Element dtypes:
 * ORC_F32 (float), ORC_BF16 (bfloat16 bits), ORC_MXFP4 (two E2M1 codes per byte,
 * element 2i in the low nibble, plus uint8 E8M0 scales [rows][K/32]).
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_MXFP4 = 2 };

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Element i of a dense array of dtype dt, as double. */
static double ld(const void* p, int dt, size_t i) {
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  return bf16_to_double(((const uint16_t*)p)[i]);
}

/* Round a double to the nearest bfloat16 value (8 significant bits), ties to
   even; the result is returned as a double. Values here are far from the
   bfloat16 overflow and underflow limits. */
double orc_round_bf16(double v) {
  if (v == 0 || !isfinite(v)) return v;
  int ex;
  frexp(v, &ex);                               /* |v| in [2^(ex-1), 2^ex) */
  double step = ldexp(1.0, ex - 8);
  return nearbyint(v / step) * step;
}

/* ---------------------------------------------------------------------------
 * MX codec (OCP Microscaling Formats v1.0; MXFP4 per-32 UE8M0 as stated in the
 * blog's "NVFP4 as a third MMA type" section).
 * ------------------------------------------------------------------------- */

/* E8M0 scale code -> 2^(code - 127). Code 255 is NaN. */
double orc_e8m0_value(uint8_t code) {
  if (code == 255) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* E2M1 code (4 bits: sign, 2-bit exponent with bias 1, 1-bit mantissa). */
double orc_e2m1_value(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E4M3 code, OCP variant: bias 7, no infinities, S.1111.111 is NaN, max 448. */
double orc_e4m3_value(uint8_t code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Round |v| to the grid of a minifloat with `mbits` mantissa bits, minimum normal
   exponent `emin` and largest finite value `maxv`: nearest, ties to even,
   saturating. Returns the rounded magnitude. */
static double round_minifloat(double a, int mbits, int emin, double maxv) {
  if (!(a > 0)) return 0.0;
  int ex;
  frexp(a, &ex);                  /* a = f * 2^ex, f in [0.5, 1) -> floor(log2 a) = ex - 1 */
  int e = ex - 1;
  if (e < emin) e = emin;         /* subnormal range shares the minimum normal's step */
  double step = ldexp(1.0, e - mbits);
  double q = nearbyint(a / step) * step;   /* default rounding mode: ties to even */
  return q > maxv ? maxv : q;
}

/* Encode a magnitude already on the E4M3 grid (or zero) plus a sign into a code. */
static uint8_t e4m3_encode(double q, int neg) {
  uint8_t code = 0;
  if (q > 0) {
    int ex;
    frexp(q, &ex);
    int e = ex - 1;
    if (e < -6) {                               /* subnormal: q = m/8 * 2^-6 */
      code = (uint8_t)(int)nearbyint(q / ldexp(1.0, -9));
    } else {
      int m = (int)nearbyint((q / ldexp(1.0, e) - 1.0) * 8.0);
      code = (uint8_t)(((e + 7) << 3) | m);
    }
  }
  return (uint8_t)(code | (neg ? 0x80 : 0));
}

static uint8_t e2m1_encode(double q, int neg) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  uint8_t c = 0;
  for (uint8_t i = 0; i < 8; ++i)
    if (grid[i] == q) c = i;
  return (uint8_t)(c | (neg ? 0x8 : 0));
}

/* Shared exponent of one block: floor(log2(amax)) - emax_elem, clamped. */
static int mx_block_exponent(const double* v, int n, int emax_elem) {
  double amax = 0;
  for (int i = 0; i < n; ++i) amax = fmax(amax, fabs(v[i]));
  if (amax == 0) return -127;
  int ex;
  frexp(amax, &ex);
  int X = (ex - 1) - emax_elem;
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  return X;
}

/* Quantize n values (n a multiple of 32) to MXFP8 E4M3 blocks of 32.
   codes[n], scales[n/32] (E8M0). If deq != NULL it receives the dequantized values. */
void orc_mx_quant_e4m3(const double* v, int n, uint8_t* codes, uint8_t* scales, double* deq) {
  for (int b = 0; b < n / 32; ++b) {
    int X = mx_block_exponent(v + 32 * b, 32, 8);
    double s = ldexp(1.0, X);
    if (scales) scales[b] = (uint8_t)(X + 127);
    for (int i = 32 * b; i < 32 * b + 32; ++i) {
      double q = round_minifloat(fabs(v[i]) / s, 3, -6, 448.0);
      if (codes) codes[i] = e4m3_encode(q, v[i] < 0);
      if (deq) deq[i] = (v[i] < 0 ? -q : q) * s;
    }
  }
}

/* Quantize n values (n a multiple of 32) to MXFP4 E2M1 blocks of 32.
   packed[n/2] (element 2i in the low nibble), scales[n/32]. */
void orc_mx_quant_e2m1(const double* v, int n, uint8_t* packed, uint8_t* scales, double* deq) {
  for (int b = 0; b < n / 32; ++b) {
    int X = mx_block_exponent(v + 32 * b, 32, 2);
    double s = ldexp(1.0, X);
    if (scales) scales[b] = (uint8_t)(X + 127);
    for (int i = 32 * b; i < 32 * b + 32; ++i) {
      double q = round_minifloat(fabs(v[i]) / s, 1, 0, 6.0);
      uint8_t c = e2m1_encode(q, v[i] < 0);
      if (packed) {
        if (i % 2 == 0) packed[i / 2] = c;
        else packed[i / 2] = (uint8_t)(packed[i / 2] | (c << 4));
      }
      if (deq) deq[i] = (v[i] < 0 ? -q : q) * s;
    }
  }
}

/* ---------------------------------------------------------------------------
 * NVFP4 -> MXFP4 requantization of expert weights at load.
 *
 * NVFP4 (blog, "NVFP4 as a third MMA type"): dense E2M1 values with one UE4M3
 * block scale per 16 elements (instead of MXFP4's one UE8M0 per 32); a stored
 * checkpoint also carries one FP32 scale per weight matrix. The blog's "AMD
 * support" section serves the NVFP4 checkpoint on MI355X through the MXFP4
 * quantization path and reports an "NVFP4 Requant" accuracy column, i.e. the
 * NVFP4 weights are re-encoded as MXFP4 for the MI355X kernels.
 *
 * Reading (the pages give no formula): each element's NVFP4 value
 * e2m1(code) * ue4m3(scale16) * g is formed in FP32 (the product of the two
 * minifloats is exact; the multiplication by the FP32 matrix scale g rounds to
 * nearest-even), then every 32-element block is MX-quantized exactly as
 * orc_mx_quant_e2m1 does. The block-scale byte is unsigned (its top bit is
 * ignored). A block whose scales or g are NaN (UE4M3 0x7F, non-finite g), or
 * whose values overflow FP32, gets the E8M0 NaN scale 0xFF and zero codes.
 *
 * codes [n_mats][rows][cols/2] (element 2i in the low nibble), scales16
 * [n_mats][rows][cols/16], g [n_mats] -> out_codes [n_mats][rows][cols/2],
 * out_scales [n_mats][rows][cols/32]; cols a multiple of 32.
 * ------------------------------------------------------------------------- */
/* IEEE arithmetic whatever the host process's SSE modes are: a library loaded
   into the same process can switch it to flush-to-zero / denormals-are-zero
   (code linked with fast-math does), which would change FP32 products below
   2^-126. The modes are cleared for the call and restored after it. */
static unsigned ieee_begin(void) {
  const unsigned csr = _mm_getcsr();
  _mm_setcsr(csr & ~0x8040u);                 /* FTZ (bit 15), DAZ (bit 6) */
  return csr;
}
static void ieee_end(unsigned csr) { _mm_setcsr(csr); }

/* Timing hooks: the number of threads the parallel loops over tokens and
   assignments use (a CPU-baseline run single-threaded or on every core). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_get_threads(void) { return omp_get_max_threads(); }

/* Test hook: turn FTZ and DAZ on (1) or off (0) for the calling thread. */
void orc_set_flush_modes(int on) {
  const unsigned csr = _mm_getcsr();
  _mm_setcsr(on ? (csr | 0x8040u) : (csr & ~0x8040u));
}

void orc_nvfp4_to_mxfp4(const uint8_t* codes, const uint8_t* scales16, const float* g,
                        int64_t n_mats, int64_t rows, int64_t cols, uint8_t* out_codes,
                        uint8_t* out_scales) {
  const unsigned csr = ieee_begin();
  const int64_t nb = cols / 32;
  for (int64_t m = 0; m < n_mats; ++m) {
    const float gm = g[m];
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t row = m * rows + r;
      for (int64_t b = 0; b < nb; ++b) {
        double v[32];
        int bad = !isfinite(gm);
        for (int i = 0; i < 32; ++i) {
          const int64_t k = 32 * b + i;
          const uint8_t byte = codes[row * (cols / 2) + k / 2];
          const uint8_t c = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
          const uint8_t sc = scales16[row * (cols / 16) + k / 16] & 0x7F;
          if (sc == 0x7F) bad = 1;
          const float p = (float)orc_e2m1_value(c) * (float)orc_e4m3_value(sc);
          const float x = p * gm;
          if (!isfinite(x)) bad = 1;
          v[i] = (double)x;
        }
        uint8_t* oc = out_codes + row * (cols / 2) + 16 * b;
        if (bad) {
          for (int i = 0; i < 16; ++i) oc[i] = 0;
          out_scales[row * nb + b] = 0xFF;
        } else {
          orc_mx_quant_e2m1(v, 32, oc, out_scales + row * nb + b, NULL);
        }
      }
    }
  }
  ieee_end(csr);
}

/* Row r of an expert weight matrix with K columns, dequantized into out[K]. */
static void load_row(const void* w, const uint8_t* scales, int dt, size_t r, int K, double* out) {
  if (dt == ORC_MXFP4) {
    const uint8_t* row = (const uint8_t*)w + r * (size_t)(K / 2);
    const uint8_t* sc = scales + r * (size_t)(K / 32);
    for (int i = 0; i < K; ++i) {
      uint8_t c = (i % 2 == 0) ? (row[i / 2] & 0xF) : (row[i / 2] >> 4);
      out[i] = orc_e2m1_value(c) * orc_e8m0_value(sc[i / 32]);
    }
  } else {
    for (int i = 0; i < K; ++i) out[i] = ld(w, dt, r * (size_t)K + i);
  }
}

/* ---------------------------------------------------------------------------
 * Step 1 — router: logits = x . W_router^T (+ bias), from the full-width input
 * (blog, MoE section: the router picks experts from the full-width
 * representation; vLLM summary, Nvidia notes: FP32 router output).
 * x [T][D] (dt), wr [E][D] (dt), bias [E] float or NULL, logits [T][E] float.
 * ------------------------------------------------------------------------- */
void orc_router(const void* x, const void* wr, int dt, const float* bias,
                int T, int D, int E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double s = 0;
      for (int i = 0; i < D; ++i) s += ld(x, dt, (size_t)t * D + i) * ld(wr, dt, (size_t)e * D + i);
      if (bias) s += (double)bias[e];
      logits[(size_t)t * E + e] = (float)s;
    }
}

/* ---------------------------------------------------------------------------
 * Step 2 — top-k selection and routing weights (blog, "Kernel optimizations":
 * a top-k routing kernel emits expert ids and weights). Selection: the k largest
 * logits, ties to the lower index, listed in that order. Weights: softmax over
 * the k selected logits.
 *
 * Non-finite logits (the pages do not consider them; readings):
 *  - a logit's routing score is the logit itself, except that NaN scores as
 *    -inf: NaN ranks below every number and ties with -inf, so the k selected
 *    ids are always k distinct valid experts (ties still go to the lower index);
 *  - the weights are the softmax of the selected scores; when the largest
 *    selected score m is infinite (every selected score is -inf, or some are
 *    +inf) they are the softmax's limit as the logits equal to m move together
 *    without bound: equal shares among the slots whose score is m, 0 elsewhere.
 * ------------------------------------------------------------------------- */
static double route_score(float v) { return isnan(v) ? -INFINITY : (double)v; }

void orc_topk_softmax(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    int32_t* id = ids + (size_t)t * k;
    for (int j = 0; j < k; ++j) {            /* selection by repeated arg-max */
      int best = -1;
      for (int e = 0; e < E; ++e) {
        int taken = 0;
        for (int q = 0; q < j; ++q) taken |= (id[q] == e);
        if (taken) continue;
        /* strict '>' keeps the lower index on ties */
        if (best < 0 || route_score(l[e]) > route_score(l[best])) best = e;
      }
      id[j] = best;
    }
    double m = route_score(l[id[0]]);
    for (int j = 1; j < k; ++j) m = fmax(m, route_score(l[id[j]]));
    if (isinf(m)) {
      int n = 0;
      for (int j = 0; j < k; ++j) n += route_score(l[id[j]]) == m;
      for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = route_score(l[id[j]]) == m ? 1.0 / n : 0.0;
      continue;
    }
    double den = 0;
    for (int j = 0; j < k; ++j) den += exp(route_score(l[id[j]]) - m);
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = exp(route_score(l[id[j]]) - m) / den;
  }
}

/* ---------------------------------------------------------------------------
 * Step 3 — token-to-expert permutation (AMD notes on the blog: the expert sort
 * groups the (token, slot) assignments by expert; the finalize step undoes it).
 * Definition: assignment a = t*k + j; sorted order is (expert asc, token asc).
 * counts[E], offsets[E+1] (exclusive prefix sums), sorted_assign[T*k] (the a at
 * each sorted position), inv[T*k] (sorted position of each a).
 * ------------------------------------------------------------------------- */
void orc_permutation(const int32_t* ids, int T, int k, int E,
                     int32_t* counts, int32_t* offsets, int32_t* sorted_assign, int32_t* inv) {
  int32_t pos = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = pos;
    counts[e] = 0;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (ids[(size_t)t * k + j] == e) {
          sorted_assign[pos] = t * k + j;
          inv[t * k + j] = pos;
          ++pos;
          ++counts[e];
        }
  }
  offsets[E] = pos;
}

/* ---------------------------------------------------------------------------
 * Step 4 — pooler and pooled RMSNorm (blog, MoE section: the learned pooler
 * narrows each token to the expert width and the pooled expert input is
 * normalized before the experts run; vLLM summary: pooler 8192 x 4096).
 * x [T][D], wp [Dp][D], gp [Dp] -> xp [T][Dp] double.
 * If mx_act, xp is then quantized to MXFP8 E4M3 per 32 and dequantized (the
 * expert input of the MXFP4-expert configuration); else if rnd it is rounded
 * to bfloat16.
 * ------------------------------------------------------------------------- */
void orc_pool_norm(const void* x, const void* wp, int dt, const float* gp,
                   int T, int D, int Dp, double eps, int mx_act, int rnd, double* xp) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    double* p = xp + (size_t)t * Dp;
    double ss = 0;
    for (int c = 0; c < Dp; ++c) {
      double s = 0;
      for (int i = 0; i < D; ++i) s += ld(x, dt, (size_t)t * D + i) * ld(wp, dt, (size_t)c * D + i);
      p[c] = s;
      ss += s * s;
    }
    double r = 1.0 / sqrt(ss / Dp + eps);
    for (int c = 0; c < Dp; ++c) p[c] = p[c] * r * (double)gp[c];
    if (mx_act) orc_mx_quant_e4m3(p, Dp, NULL, NULL, p);
    else if (rnd)
      for (int c = 0; c < Dp; ++c) p[c] = orc_round_bf16(p[c]);
  }
}

/* ---------------------------------------------------------------------------
 * Step 5 — one selected expert on one token (blog, MoE section: routed SwiGLU
 * experts at the pooled width; each selected expert's output is RMS-normalized
 * with its own parameters before the routing weight is applied; "Fused
 * per-expert post-norm": the norm covers the whole expert output row).
 * xin [Dp] (the normalized pooled input), wgu [2F][Dp], wd [Dp][F], ge [Dp].
 * z [Dp] = RMSNorm_e(y) (gamma applied); *rms_unit = RMS of y / sqrt(ms + eps),
 * i.e. the normalized row before gamma. If mx_act, the SwiGLU output h is
 * quantized to MXFP8 E4M3 per 32 and dequantized before the down projection,
 * else if rnd it is rounded to bfloat16; if rnd the expert output y is rounded
 * to bfloat16 before its RMS is taken.
 * ------------------------------------------------------------------------- */
void orc_expert(const double* xin, int Dp, int F,
                const void* wgu, const uint8_t* sgu, const void* wd, const uint8_t* sd, int wdt,
                const float* ge, double eps, int mx_act, int rnd, double* z, double* rms_unit) {
  double* row = (double*)malloc(sizeof(double) * (size_t)(Dp > F ? Dp : F));
  double* h = (double*)malloc(sizeof(double) * (size_t)F);
  for (int f = 0; f < F; ++f) {
    double g = 0, u = 0;
    load_row(wgu, sgu, wdt, (size_t)f, Dp, row);
    for (int c = 0; c < Dp; ++c) g += xin[c] * row[c];
    load_row(wgu, sgu, wdt, (size_t)(F + f), Dp, row);
    for (int c = 0; c < Dp; ++c) u += xin[c] * row[c];
    h[f] = g / (1.0 + exp(-g)) * u;                    /* silu(g) * u */
  }
  if (mx_act) orc_mx_quant_e4m3(h, F, NULL, NULL, h);
  else if (rnd)
    for (int f = 0; f < F; ++f) h[f] = orc_round_bf16(h[f]);
  double ss = 0;
  for (int c = 0; c < Dp; ++c) {
    double y = 0;
    load_row(wd, sd, wdt, (size_t)c, F, row);
    for (int f = 0; f < F; ++f) y += h[f] * row[f];
    if (rnd) y = orc_round_bf16(y);
    z[c] = y;
    ss += y * y;
  }
  double r = 1.0 / sqrt(ss / Dp + eps);
  double su = 0;
  for (int c = 0; c < Dp; ++c) {
    double n = z[c] * r;
    su += n * n;
    z[c] = n * (double)ge[c];
  }
  if (rms_unit) *rms_unit = sqrt(su / Dp);
  free(row);
  free(h);
}

/* Step 5 for n (token, expert) assignments at once: assignment a runs token row
   tok[a] of xin [*][Dp] through expert ex[a], whose weights are found in the
   per-expert pointer arrays (sgu/sd NULL unless MXFP4). z [n][Dp], rms_unit [n]
   or NULL. Assignments are independent, so they run in parallel. */
void orc_expert_assign(const double* xin, int n, const int32_t* tok, const int32_t* ex, int Dp,
                       int F, const void* const* wgu, const uint8_t* const* sgu,
                       const void* const* wd, const uint8_t* const* sd, int wdt, const float* ge,
                       double eps, int mx_act, int rnd, double* z, double* rms_unit) {
#pragma omp parallel for schedule(dynamic)
  for (int a = 0; a < n; ++a) {
    int e = ex[a];
    orc_expert(xin + (size_t)tok[a] * Dp, Dp, F, wgu[e], sgu ? sgu[e] : NULL, wd[e],
               sd ? sd[e] : NULL, wdt, ge + (size_t)e * Dp, eps, mx_act, rnd, z + (size_t)a * Dp,
               rms_unit ? rms_unit + a : NULL);
  }
}

/* ---------------------------------------------------------------------------
 * Step 6 — weighted sum and unpooler (blog, MoE section: normalized expert
 * outputs are scaled by their routing weights and summed, then the unpooler
 * restores model width; "Reinforcement learning" section: the sum is FP32 or
 * wider, kept here in double, in slot order j = 0..k-1).
 * z [T][k][Dp], w [T][k], wun [D][Dp] -> out [T][D] double. If rnd, the sum
 * is rounded to bfloat16 before the unpooler.
 * ------------------------------------------------------------------------- */
void orc_combine_unpool(const double* z, const double* w, const void* wun, int dt,
                        int T, int k, int Dp, int D, int rnd, double* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    double* acc = (double*)calloc((size_t)Dp, sizeof(double));
    for (int j = 0; j < k; ++j)
      for (int c = 0; c < Dp; ++c) acc[c] += w[(size_t)t * k + j] * z[((size_t)t * k + j) * Dp + c];
    if (rnd)
      for (int c = 0; c < Dp; ++c) acc[c] = orc_round_bf16(acc[c]);
    for (int o = 0; o < D; ++o) {
      double s = 0;
      for (int c = 0; c < Dp; ++c) s += acc[c] * ld(wun, dt, (size_t)o * Dp + c);
      out[(size_t)t * D + o] = s;
    }
    free(acc);
  }
}
