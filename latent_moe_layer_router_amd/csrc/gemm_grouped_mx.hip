// Grouped expert GEMMs of the MXFP4-expert path for experts with many rows
// (prefill): MXFP8 E4M3 activations times MXFP4 (E2M1) weights, one E8M0 scale
// per 32 values along K on both sides, on gfx950's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), fp32 accumulation.
//   gate/up: H = silu(xq . Wg^T) * (xq . Wu^T), quantized again to MXFP8 E4M3
//            blocks of 32 (codes + scales) as the down GEMM's input;
//   down:    y = H . Wd^T in bf16 plus per-64-column sums of squares of the
//            stored values (for the per-expert RMSNorm in the combine).
// MXFP4 as the expert weight format with per-32 UE8M0 scales: LMSYS Muse Spark
// Open blog, "NVFP4 as a third MMA type"; encodings: OCP Microscaling v1.0.
//
// Scaled-MFMA operand layout (gfx950, 32x32x64; lane l: row r = l % 32 of the
// operand, group q = l / 32):
//   fp8 operand, 32 bytes: bytes 0..15 hold K [16q, 16q + 16), bytes 16..31 hold
//     K [32 + 16q, 32 + 16q + 16);
//   fp4 operand, 16 bytes: two E2M1 values per byte, low nibble first, holding
//     K [32q, 32q + 32);
//   scale: one E8M0 byte per lane, for K [32q, 32q + 32) of its row;
//   result: register v of lane l at row 8 (v / 4) + 4q + v % 4, column l % 32.
//
// Row tiles as in the bf16 grouped GEMM: up to 320 rows x 256 weight rows, each
// expert's rows split over ceil(rows / 320) tiles in whole units of 64 rows
// and each tile's rows between two wave rows. 512 threads = 8 wave64 in a 2 x 4 grid, each wave up
// to 160 x 64 = 5 x 2 MFMAs per K-step of 64 (160 accumulator registers, two
// waves per SIMD). With 256-row tiles, near-uniform routing (512 +- 23 rows per
// expert) gave half the experts a third row tile that loads the whole weight
// slice again (measured: 12% of the time).
//
// A stage holds two K-steps (128 columns): A 320 rows x 128 bytes (fp8), B 256
// rows x 64 bytes (fp4), moved by direct global-to-LDS buffer loads of whole
// 128- and 64-byte row segments; two stage buffers, the next stage loading
// while the current one is multiplied, one barrier per stage. The scales come
// in groups of 4 stages (512 columns = 16 bytes per row of A and of B) into one
// of two scale buffers. LDS: 2 x 56 KiB + 2 x 9 KiB = 130 KiB. The fragments of
// a K-step are read group by group just before their MFMAs (a scheduling
// barrier after each K-step keeps the next step's reads from being hoisted):
// the other wave of the SIMD covers the LDS latency, and a K-step's whole
// fragment set (48 registers) would not fit twice beside 160 accumulators.
//
// Tile order over the 8 XCDs: one index space (expert, n-tile, m-tile) cut into
// 8 contiguous chunks.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace lmoe {

namespace {

constexpr int XW = 8;                  // waves
constexpr int XNT = XW * 64;
constexpr int XBM = 320, XBN = 256;    // A rows (max), B rows per tile
constexpr int XMI = 5, XNI = 2;        // 32-row groups, 32-column groups per wave
constexpr int RA = 128;                // bytes per A row per stage (128 fp8)
constexpr int RBB = 64;                // bytes per B row per stage (128 fp4)
constexpr int XSA = XBM * RA, XSB = XBN * RBB;
constexpr int XSS = (XBM + XBN) * 16;  // scale group: A rows then B rows, 16 bytes each
constexpr int kBufWord3 = 0x00020000;  // raw buffer descriptor, fourth word (CDNA)
constexpr uint32_t kOutOfRange = 0x80000000u;   // past every extent used here

#define LMOE_AS3 __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// A DS instruction's immediate offset holds 16 bits, so the scale buffers, read
// at many constant offsets from one lane address (8 K-steps x up to 7 rows of
// bytes per group), must sit below 64 KiB: offsets past it each cost a
// register of their own, which with 160 accumulators made the compiler spill.
// Their larger alignment places them first (the LDS layout is sorted by
// alignment, then size).
__shared__ __attribute__((aligned(1024))) unsigned char xS0[XSS], xS1[XSS];
__shared__ __attribute__((aligned(16))) unsigned char xA0[XSA], xA1[XSA];
__shared__ __attribute__((aligned(16))) unsigned char xB0[XSB], xB1[XSB];

// A rows (eight 16-byte chunks): chunk c of row r at position c ^ fa(r).
__device__ __forceinline__ int fa(int r) { return ((r >> 1) ^ (r << 2)) & 7; }
// B rows (four chunks): chunk c of row r at position c ^ fb(r).
__device__ __forceinline__ int fb(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

__device__ __forceinline__ void mfma_mx(const uint4& a0, const uint4& a1, const uint4& b, int sa, int sb,
                                        f32x16_t& acc) {
  const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // A format 0 = fp8 E4M3, B format 4 = fp4 E2M1; scales in byte 0 of sa / sb.
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 4, 0, sa, 0, sb);
}

// Two fp32 values rounded to bf16 by the packed hardware conversion (to
// nearest, ties to even, as f32_to_bf16 rounds every finite value; a NaN stays
// a NaN), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, b16x2_t));
}

// silu(g) * u with the hardware exponential and reciprocal (a few ulp of fp32).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// s_waitcnt immediate: no vector-memory and no LDS operation outstanding.
constexpr int kAllIdle = 7 << 4;

__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int EPI>
__global__ __launch_bounds__(XNT, 1) void gemm_grouped_mx_kernel(GroupedMxParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // ---- tile of this workgroup (XCD-chunked order) --------------------------
  const int total = p.ntiles_n * p.mt_off[p.E];
  const int chunk = (total + 7) / 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int t = xcd * chunk + local;
  if (local >= chunk || t >= total) return;
  int lo = 0, hi = p.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.ntiles_n * p.mt_off[mid] <= t) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mt_e = p.mt_off[e + 1] - p.mt_off[e];
  const int tl = t - p.ntiles_n * p.mt_off[e];
  const int mi_t = tl % mt_e, cnt = p.offsets[e + 1] - p.offsets[e];
  const int ntile = tl / mt_e;
  // whole units of 64 rows per tile, as in the bf16 grouped GEMM
  const int G = (cnt + 63) >> 6;
  const int g0 = (int)((int64_t)G * mi_t / mt_e), g1 = (int)((int64_t)G * (mi_t + 1) / mt_e);
  const int m0 = p.offsets[e] + min(cnt, 64 * g0);
  const int m_end = p.offsets[e] + min(cnt, 64 * g1);
  const int n0 = ntile * (EPI == EPI_SWIGLU ? XBN / 2 : XBN);   // output column start
  const int K = p.K;
  // the tile's rows split between the wave rows: wm = 0 takes the first r_half
  // (a multiple of 32, at least half), wm = 1 the rest; at most 160 each
  const int tile_rows = m_end - m0;
  const int r_half = 32 * ((((tile_rows + 1) >> 1) + 31) >> 5);
  const int wrow0 = wm * r_half;
  const int mrows = wm == 0 ? min(r_half, tile_rows) : tile_rows - r_half;
  const int nmi = __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : (mrows >= 32 * XMI ? XMI : (mrows + 31) / 32));

  // ---- buffer descriptors and per-lane load offsets ------------------------
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A), (short)0, (int)p.a_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rAs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.As), (short)0, (int)p.as_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.B + (int64_t)e * p.N * (K / 2)), (short)0, p.N * (K / 2), kBufWord3);
  const __amdgpu_buffer_rsrc_t rBs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.Bs + (int64_t)e * p.N * (K / 32)), (short)0, p.N * (K / 32), kBufWord3);
  // Rows past the tile's end (tail rows) get offsets beyond every extent: their
  // loads read nothing from memory; they are never stored.
  auto a_live = [&](int r) { return m0 + r < m_end; };
  auto a_src = [&](int r) { return (uint32_t)(p.a_rows ? p.a_rows[m0 + r] : m0 + r); };   // gathered rows
  auto b_row = [&](int r) -> uint32_t {     // B row of tile row r
    return (EPI == EPI_SWIGLU) ? (uint32_t)((r < XBN / 2) ? (n0 + r) : (p.F + n0 + r - XBN / 2))
                               : (uint32_t)(n0 + r);
  };
  // A: 40 loads of 8 rows x 128 bytes per stage; wave w issues loads 5 w .. 5 w
  // + 4 (lane: row 8 j + lane / 8, position lane % 8).
  uint32_t ga[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int r = 8 * (5 * wave + i) + (lane >> 3);
    ga[i] = a_live(r) ? a_src(r) * (uint32_t)K + (uint32_t)(((lane & 7) ^ fa(r)) << 4) : kOutOfRange;
  }
  // B: 16 loads of 16 rows x 64 bytes per stage; wave w issues 2 w, 2 w + 1.
  uint32_t gb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * (2 * wave + i) + (lane >> 2);
    gb[i] = b_row(r) * (uint32_t)(K / 2) + (uint32_t)(((lane & 3) ^ fb(r)) << 4);
  }
  // Scales, per group of 4 stages: 9 loads of 64 rows x 16 bytes (5 for A, 4 for
  // B); wave w issues load w, and wave 0 also load 8.
  auto scale_off = [&](int s) -> uint32_t {
    const int r = 64 * (s < 5 ? s : s - 5) + lane;
    if (s < 5) return a_live(r) ? a_src(r) * (uint32_t)(K / 32) : kOutOfRange;
    return b_row(r) * (uint32_t)(K / 32);
  };
  const uint32_t gs0 = scale_off(wave), gs1 = scale_off(8);

#define LMOE_DATA(st, SA, SB)                                                                    \
  {                                                                                             \
    const int koa = (st) * RA, kob = (st) * RBB;                                                \
    _Pragma("unroll") for (int i = 0; i < 5; ++i)                                               \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (LMOE_AS3 void*)((SA) + 1024 * (5 * wave + i)), \
                                               16, (int)ga[i], koa, 0, 0);                      \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                               \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (LMOE_AS3 void*)((SB) + 1024 * (2 * wave + i)), \
                                               16, (int)gb[i], kob, 0, 0);                      \
  }
#define LMOE_SCALES(g, SS)                                                                       \
  {                                                                                             \
    const int kos = (g) * 16;                                                                   \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wave < 5 ? rAs : rBs,                              \
                                             (LMOE_AS3 void*)((SS) + 1024 * wave), 16, (int)gs0, kos, 0, 0); \
    if (wave == 0)                                                                              \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, (LMOE_AS3 void*)((SS) + 1024 * 8), 16, (int)gs1, kos, 0, 0); \
  }

  f32x16_t acc[XMI][XNI];
#pragma unroll
  for (int mi = 0; mi < XMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < XNI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  // ---- fragment addresses ---------------------------------------------------
  // Row r of the A fragment mi; rows of the B fragments (SwiGLU: gate ni = 0
  // and up ni = 1 of the same 32 output columns). For MFMA step s of a stage,
  // lane group q reads A chunks 4s + q and 4s + 2 + q, B chunk 2s + q.
  // (fa depends on a row's low 4 bits only, so group mi's offsets are group 0's
  // plus mi rows of 32.)
  const int l32 = lane & 31, q = lane >> 5;
  int aoff[2][2], boff[2][XNI], bsc[XNI];
  const int ar = wrow0 + l32;
  const int asc = ar * 16 + q;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    aoff[s2][0] = ar * RA + (((4 * s2 + q) ^ fa(ar)) << 4);
    aoff[s2][1] = ar * RA + (((4 * s2 + 2 + q) ^ fa(ar)) << 4);
  }
#pragma unroll
  for (int ni = 0; ni < XNI; ++ni) {
    const int r = (EPI == EPI_SWIGLU) ? (ni * (XBN / 2) + wn * 32 + l32) : (wn * 64 + ni * 32 + l32);
    bsc[ni] = XBM * 16 + r * 16 + q;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) boff[s2][ni] = r * RBB + (((2 * s2 + q) ^ fb(r)) << 4);
  }

  // One MFMA step: step S2 (0, 1) of the stage in SA/SB, whose scales are step
  // J (0..7) of its group in SS (bytes 2 J + q of each row's 16). NMI live
  // 32-row groups.
  // One 32-row group MI of a K-step: its fragment reads, then its two MFMAs. The
  // empty asm statement takes the two accumulators and clobbers memory, so the
  // MFMAs stay here and the next group's reads stay below them: only one
  // group's fragments are live beside the 160 accumulators. (Without it the
  // compiler read a whole stage's fragments ahead and spilled them.)
#define LMOE_GROUP(MI, SA, SS, S2, J)                                                             \
  {                                                                                             \
    const uint4 a0_ = *reinterpret_cast<const uint4*>((SA) + aoff[S2][0] + (MI) * 32 * RA);     \
    const uint4 a1_ = *reinterpret_cast<const uint4*>((SA) + aoff[S2][1] + (MI) * 32 * RA);     \
    const int sa_ = (int)(SS)[asc + (MI) * 32 * 16 + 2 * (J)];                                   \
    mfma_mx(a0_, a1_, fb0_, sa_, sb0_, acc[MI][0]);                                             \
    mfma_mx(a0_, a1_, fb1_, sa_, sb1_, acc[MI][1]);                                             \
    asm volatile("" : "+v"(acc[MI][0]), "+v"(acc[MI][1]) : : "memory");                          \
  }
#define LMOE_KSTEP(NMI, SA, SB, SS, S2, J)                                                        \
  if ((NMI) > 0) {                                                                              \
    const uint4 fb0_ = *reinterpret_cast<const uint4*>((SB) + boff[S2][0]);                     \
    const uint4 fb1_ = *reinterpret_cast<const uint4*>((SB) + boff[S2][1]);                     \
    const int sb0_ = (int)(SS)[bsc[0] + 2 * (J)];                                                \
    const int sb1_ = (int)(SS)[bsc[1] + 2 * (J)];                                                \
    LMOE_GROUP(0, SA, SS, S2, J)                                                                \
    if ((NMI) > 1) LMOE_GROUP(1, SA, SS, S2, J)                                                 \
    if ((NMI) > 2) LMOE_GROUP(2, SA, SS, S2, J)                                                 \
    if ((NMI) > 3) LMOE_GROUP(3, SA, SS, S2, J)                                                 \
    if ((NMI) > 4) LMOE_GROUP(XMI - 1, SA, SS, S2, J)                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
  // Stage k (buffers SA/SB, the P-th of its scale group in SS): both MFMA steps;
  // then each wave waits for its loads (stage k + 1) and LDS reads and passes
  // the barrier, after which no wave reads stage k's buffers any more: the
  // loads of stage k + 2 go into them (past the last stage: a harmless repeat
  // of the last one), and at the last stage of a scale group the scales of the
  // group after next go into the buffer of the group that just ended.
#define LMOE_STAGE(NMI, k, P, SA, SB, SS, SFREE)                                                  \
  {                                                                                             \
    LMOE_KSTEP(NMI, SA, SB, SS, 0, 2 * (P))                                                     \
    LMOE_KSTEP(NMI, SA, SB, SS, 1, 2 * (P) + 1)                                                 \
    __builtin_amdgcn_s_waitcnt(kAllIdle);                                                       \
    bar();                                                                                      \
    LMOE_DATA(((k) + 2 < nst ? (k) + 2 : nst - 1), SA, SB)                                      \
    if ((P) == 3) {                                                                             \
      const int g_ = ((k) + 1) / 4 + 1;                                                         \
      LMOE_SCALES((g_ < ng ? g_ : ng - 1), SFREE)                                               \
    }                                                                                           \
  }
  // Eight stages: two scale groups (buffers xS0, xS1), the stage buffers
  // alternating.
#define LMOE_KLOOP(NMI)                                                                          \
  {                                                                                             \
    for (int k0_ = 0; k0_ < nst; k0_ += 8) {                                                    \
      LMOE_STAGE(NMI, k0_ + 0, 0, xA0, xB0, xS0, xS1)                                           \
      LMOE_STAGE(NMI, k0_ + 1, 1, xA1, xB1, xS0, xS1)                                           \
      LMOE_STAGE(NMI, k0_ + 2, 2, xA0, xB0, xS0, xS1)                                           \
      LMOE_STAGE(NMI, k0_ + 3, 3, xA1, xB1, xS0, xS0)                                           \
      LMOE_STAGE(NMI, k0_ + 4, 0, xA0, xB0, xS1, xS0)                                           \
      LMOE_STAGE(NMI, k0_ + 5, 1, xA1, xB1, xS1, xS0)                                           \
      LMOE_STAGE(NMI, k0_ + 6, 2, xA0, xB0, xS1, xS0)                                           \
      LMOE_STAGE(NMI, k0_ + 7, 3, xA1, xB1, xS1, xS1)                                           \
    }                                                                                           \
  }

  // Prologue: scale groups 0 and 1, stage 0; wait for them; start stage 1.
  const int nst = K / 128;                   // a multiple of 8 (K % 1024 == 0)
  const int ng = nst / 4;
  LMOE_SCALES(0, xS0)
  LMOE_SCALES((ng > 1 ? 1 : 0), xS1)
  LMOE_DATA(0, xA0, xB0)
  __builtin_amdgcn_s_waitcnt(kAllIdle);
  bar();
  LMOE_DATA((nst > 1 ? 1 : 0), xA1, xB1)
  if (nmi > 4) {
    LMOE_KLOOP(5)
  } else if (nmi > 2) {
    LMOE_KLOOP(4)
  } else if (nmi > 0) {
    LMOE_KLOOP(2)
  } else {
    LMOE_KLOOP(0)
  }
#undef LMOE_KLOOP
#undef LMOE_STAGE
#undef LMOE_KSTEP
#undef LMOE_GROUP
#undef LMOE_SCALES
#undef LMOE_DATA
  __syncthreads();   // every load has landed and every wave has finished reading

  // ---- epilogue, by wave row (up to 160 rows each) ---------------------------
  // The staging area spans the two A stage buffers: rows [80 b, 80 b + 80) of
  // the half live in buffer b, 512 bytes per row (128 fp32 or 256 bf16).
  auto srow = [&](int r) -> unsigned char* { return (r < 80 ? xA0 : xA1) + (r < 80 ? r : r - 80) * 512; };
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int mi = 0; mi < XMI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          // rows r and r + 1 (v, v + 1); both have the same bit 2
          const int r = mi * 32 + 8 * (v >> 2) + 4 * q + (v & 3);
          unsigned char* row = srow(r);
          unsigned char* row1 = srow(r + 1);
          if (EPI == EPI_SWIGLU) {
            // fp32 h at column c (0..127), 16-byte chunk c / 4 stored at
            // position (c / 4) ^ (r & 7) of the row
            const int c = wn * 32 + l32;
            *reinterpret_cast<float*>(row + ((((c >> 2) ^ (r & 7)) << 4) | ((c & 3) << 2))) =
                swiglu(acc[mi][0][v], acc[mi][1][v]);
            *reinterpret_cast<float*>(row1 + ((((c >> 2) ^ ((r + 1) & 7)) << 4) | ((c & 3) << 2))) =
                swiglu(acc[mi][0][v + 1], acc[mi][1][v + 1]);
          } else {
            // bf16 y at column c (0..255), byte b of row r at b ^ ((r & 4) << 4):
            // the two half-waves write rows four apart, 64 bytes apart
            const int sw = (r & 4) << 4;
#pragma unroll
            for (int ni = 0; ni < XNI; ++ni) {
              const uint32_t pk = pack_bf16x2(acc[mi][ni][v], acc[mi][ni][v + 1]);
              const int b = ((wn * 64 + ni * 32 + l32) * 2) ^ sw;
              *reinterpret_cast<bf16_t*>(row + b) = static_cast<bf16_t>(pk);
              *reinterpret_cast<bf16_t*>(row1 + b) = static_cast<bf16_t>(pk >> 16);
            }
          }
        }
    }
    __syncthreads();
    // rows of this half: tile rows [half r_half, half r_half + hrows)
    const int hrows = half == 0 ? min(r_half, tile_rows) : tile_rows - r_half;
    const int mh = m0 + half * r_half;
    if (EPI == EPI_SWIGLU) {
      // MXFP8 E4M3 blocks of 32 values: 8 lanes per (row, block), 4 values
      // (one 16-byte chunk) each; the block's largest magnitude over the 8
      // lanes, then each lane's 4 codes in one 32-bit store. Whole 8-lane sets
      // are active together (the bound is a multiple of 32).
      for (int i = tid; i < hrows * 32; i += XNT) {
        const int r = i >> 5, blk = (i >> 3) & 3, sub = i & 7;
        const float4 f = *reinterpret_cast<const float4*>(srow(r) + (((blk * 8 + sub) ^ (r & 7)) << 4));
        float amax = fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w)));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        const int X = mx_e4m3_exponent(amax);
        const uint32_t w = mx_e4m3_code4(f.x, f.y, f.z, f.w, X);
        uint8_t* dst = static_cast<uint8_t*>(p.out) + (int64_t)(mh + r) * p.ldo + n0 + 32 * blk + 4 * sub;
        *reinterpret_cast<uint32_t*>(dst) = w;
        if (sub == 0) p.out_scales[(int64_t)(mh + r) * p.ldos + n0 / 32 + blk] = mx_scale_code(X);
      }
    } else {
      // 16-byte stores of the bf16 rows, then the sums of squares of the stored
      // values per row and 64-column group: 8 lanes per (row, group), 16 bytes
      // each (a row's groups on consecutive lanes), then a sum over the 8 lanes
      for (int i = tid; i < hrows * (XBN / 8); i += XNT) {
        const int r = i / (XBN / 8), c = i % (XBN / 8);
        *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)(mh + r) * p.ldo + n0 + 8 * c) =
            *reinterpret_cast<const uint4*>(srow(r) + ((c * 16) ^ ((r & 4) << 4)));
      }
      for (int i = tid; i < hrows * 32; i += XNT) {
        const int r = i >> 5, grp = (i >> 3) & 3, sub = i & 7;
        const uint4 qv = *reinterpret_cast<const uint4*>(srow(r) + ((grp * 128 + sub * 16) ^ ((r & 4) << 4)));
        float ssq = 0.f;
        for (uint32_t w : {qv.x, qv.y, qv.z, qv.w}) {
          const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
          ssq += lo * lo;
          ssq += hi * hi;
        }
        ssq += __shfl_xor(ssq, 1);
        ssq += __shfl_xor(ssq, 2);
        ssq += __shfl_xor(ssq, 4);
        if (sub == 0) p.ss_out[(int64_t)(mh + r) * p.ss_ld + n0 / 64 + grp] = ssq;
      }
    }
    __syncthreads();   // the half is read out before the next one is staged
  }
}

}  // namespace

int gemm_grouped_mx_tile_m() { return XBM; }

hipError_t launch_gemm_grouped_mx(const GroupedMxParams& p, EpiKind epi, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (p.K % 1024 != 0) return hipErrorInvalidValue;
  const int grid = ((p.max_tiles + 7) / 8) * 8;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm_grouped_mx_kernel<EPI_SWIGLU>, dim3(grid), dim3(XNT), 0, s, p);
  else if (epi == EPI_DOWN)
    hipLaunchKernelGGL(gemm_grouped_mx_kernel<EPI_DOWN>, dim3(grid), dim3(XNT), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lmoe
