// Large-tile grouped GEMM of the MXFP4-expert path: MXFP8 E4M3 activations
// times MXFP4 (E2M1) expert weights, both with one E8M0 scale per 32 values
// along K, on gfx950's block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4),
// fp32 accumulation. The two expert GEMMs of the block:
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
//   result: as the other 32x32 MFMAs (register v of lane l: row 8 (v / 4) +
//     4q + v % 4, column l % 32).
//
// Tile 256 x 256 (A rows x B rows), 4 waves of 128 x 128 = 4 x 4 MFMAs per
// MFMA K-step of 64. A stage holds two K-steps (128 columns): A 256 rows x 128
// bytes (fp8), B 256 rows x 64 bytes (fp4), moved by direct global-to-LDS
// buffer loads that cover 128 and 64 contiguous bytes of a row (narrower
// segments cost a full 64-byte request each, which halves the load rate). Two
// stage buffers: the next stage loads while the current one is multiplied,
// with one barrier per stage. The scales come in groups of 4 stages (512
// columns = 16 bytes per row of A and of B) into one of two scale buffers.
// LDS: 2 x 48 KiB + 2 x 8 KiB = 112 KiB.
//
// Tile order over the 8 XCDs as in the bf16 256-tile GEMM: one index space
// (expert, n-tile, m-tile) cut into 8 contiguous chunks.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace lmoe {

namespace {

constexpr int BM = 256, BNB = 256;
constexpr int NT = 256;
constexpr int RA = 128;               // bytes per A row per stage (128 fp8)
constexpr int RBB = 64;               // bytes per B row per stage (128 fp4)
constexpr int kBufWord3 = 0x00020000;   // raw buffer descriptor, fourth word (CDNA)
// A buffer offset past every extent used here (all below 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;

#define LMOE_AS3 __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

__shared__ __attribute__((aligned(16))) unsigned char mA0[BM * RA], mA1[BM * RA];
__shared__ __attribute__((aligned(16))) unsigned char mB0[BNB * RBB], mB1[BNB * RBB];
// scale buffers: A scales [256 rows][16 B] then B scales [256 rows][16 B]
__shared__ __attribute__((aligned(16))) unsigned char mS0[2 * 256 * 16], mS1[2 * 256 * 16];

// A rows (eight 16-byte chunks): chunk c of row r at position c ^ fa(r). Any 8
// consecutive rows (from a multiple of 8) then put one chunk index on 8
// distinct 16-byte bank slots of a 128-byte bank line, and any 16 (from a
// multiple of 16) on 16 distinct slots of 256 bytes.
__device__ __forceinline__ int fa(int r) { return ((r >> 1) ^ (r << 2)) & 7; }
// B rows (four chunks): chunk c of row r at position c ^ fb(r), the same
// property for 64-byte rows.
__device__ __forceinline__ int fb(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

__device__ __forceinline__ void mfma_mx(const uint4& a0, const uint4& a1, const uint4& b, int sa, int sb,
                                        f32x16_t& acc) {
  const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // A format 0 = fp8 E4M3, B format 4 = fp4 E2M1; scales in byte 0 of sa / sb.
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 4, 0, sa, 0, sb);
}

// s_waitcnt immediate: no vector-memory and no LDS operation outstanding.
constexpr int kAllIdle = 7 << 4;

__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm256_mx_kernel(Gemm256MxParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

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
  // Row tiles of 256 from the expert's first row; the last may be short. (An
  // even split over the tiles, as in the bf16 GEMM, costs time here: a tile of
  // about 170 rows keeps one wave at full MFMA work behind the stage barriers,
  // so three such tiles take longer than two full ones and a short tail.)
  const int ntile = tl / mt_e, mtile = tl % mt_e;
  const int m0 = p.offsets[e] + mtile * BM;
  const int m_end = p.offsets[e + 1];
  const int n0 = ntile * (EPI == EPI_SWIGLU ? BNB / 2 : BNB);   // output column start
  const int K = p.K;

  // ---- buffer descriptors and per-lane load offsets ------------------------
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A), (short)0, (int)p.a_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rAs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.As), (short)0, (int)p.as_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.B + (int64_t)e * p.N * (K / 2)), (short)0, p.N * (K / 2), kBufWord3);
  const __amdgpu_buffer_rsrc_t rBs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.Bs + (int64_t)e * p.N * (K / 32)), (short)0, p.N * (K / 32), kBufWord3);
  // A row (sorted position) of tile row r. Rows past the end (tail tiles) get
  // offsets beyond every extent: their loads read nothing from memory; they are
  // never stored.
  auto a_live = [&](int r) { return m0 + r < m_end; };
  auto b_row = [&](int r) -> uint32_t {     // B row of tile row r
    return (EPI == EPI_SWIGLU) ? (uint32_t)((r < BNB / 2) ? (n0 + r) : (p.F + n0 + r - BNB / 2))
                               : (uint32_t)(n0 + r);
  };
  // A: load j moves rows wave*64 + 8 j + lane/8, lane position lane % 8.
  uint32_t ga[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + 8 * j + (lane >> 3);
    ga[j] = a_live(r) ? (uint32_t)(m0 + r) * (uint32_t)K + (uint32_t)(((lane & 7) ^ fa(r)) << 4) : kOutOfRange;
  }
  // B: load j moves rows wave*64 + 16 j + lane/4, lane position lane % 4.
  uint32_t gb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 64 + 16 * j + (lane >> 2);
    gb[j] = b_row(r) * (uint32_t)(K / 2) + (uint32_t)(((lane & 3) ^ fb(r)) << 4);
  }
  // Scales: one load each for A and B, row wave*64 + lane, 16 bytes per group.
  const uint32_t gsa = a_live(wave * 64 + lane) ? (uint32_t)(m0 + wave * 64 + lane) * (uint32_t)(K / 32) : kOutOfRange;
  const uint32_t gsb = b_row(wave * 64 + lane) * (uint32_t)(K / 32);

#define LMOE_DATA(st, SA, SB)                                                                    \
  {                                                                                             \
    const int koa = (st) * RA, kob = (st) * RBB;                                                \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                               \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (LMOE_AS3 void*)((SA) + wave * 8192 + 1024 * j), \
                                               16, (int)ga[j], koa, 0, 0);                      \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                               \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (LMOE_AS3 void*)((SB) + wave * 4096 + 1024 * j), \
                                               16, (int)gb[j], kob, 0, 0);                      \
  }
#define LMOE_SCALES(g, SS)                                                                       \
  {                                                                                             \
    const int kos = (g) * 16;                                                                   \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rAs, (LMOE_AS3 void*)((SS) + wave * 1024), 16,      \
                                             (int)gsa, kos, 0, 0);                              \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, (LMOE_AS3 void*)((SS) + 4096 + wave * 1024), 16, \
                                             (int)gsb, kos, 0, 0);                              \
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  // ---- fragment addresses ---------------------------------------------------
  // Row r of the A fragment mi, row of the B fragment ni; for MFMA step s of a
  // stage, lane group q reads A chunks 4s + q and 4s + 2 + q, B chunk 2s + q.
  const int l32 = lane & 31, q = lane >> 5;
  int aoff[2][4][2], boff[2][4], asc[4], bsc[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int r = wm * 128 + mi * 32 + l32;
    asc[mi] = r * 16 + q;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      aoff[s2][mi][0] = r * RA + (((4 * s2 + q) ^ fa(r)) << 4);
      aoff[s2][mi][1] = r * RA + (((4 * s2 + 2 + q) ^ fa(r)) << 4);
    }
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    // SwiGLU: gate (ni = 0, 1) and up (ni = 2, 3) of the same 64 output columns
    const int r = (EPI == EPI_SWIGLU) ? ((ni >> 1) * (BNB / 2) + wn * 64 + (ni & 1) * 32 + l32)
                                      : (wn * 128 + ni * 32 + l32);
    bsc[ni] = 4096 + r * 16 + q;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) boff[s2][ni] = r * RBB + (((2 * s2 + q) ^ fb(r)) << 4);
  }
  const int mrows = m_end - (m0 + wm * 128);
  const int nmi = __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : (mrows >= 128 ? 4 : (mrows + 31) / 32));

  // Fragment registers: x for the first MFMA step of a stage, y for the second.
  uint4 xa[4][2], xb[4], ya[4][2], yb[4];
  int xsa[4], xsb[4], ysa[4], ysb[4];

  // Reads of MFMA step S2 (0, 1) of a stage in SA/SB whose scales are step J
  // (0..7) of its scale group in SS (bytes 2 J + q of each row's 16). NMI live
  // 32-row groups.
#define LMOE_READ(NMI, SA, SB, SS, S2, J, PA, PB, PSA, PSB)                                       \
  if ((NMI) > 0) {                                                                              \
    _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) {                                          \
      PB[ni] = *reinterpret_cast<const uint4*>((SB) + boff[S2][ni]);                            \
      PSB[ni] = (int)(SS)[bsc[ni] + 2 * (J)];                                                    \
    }                                                                                           \
    _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) if (mi < (NMI)) {                          \
      PA[mi][0] = *reinterpret_cast<const uint4*>((SA) + aoff[S2][mi][0]);                      \
      PA[mi][1] = *reinterpret_cast<const uint4*>((SA) + aoff[S2][mi][1]);                      \
      PSA[mi] = (int)(SS)[asc[mi] + 2 * (J)];                                                    \
    }                                                                                           \
  }
#define LMOE_MFMA(NMI, PA, PB, PSA, PSB)                                                          \
  _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) if (mi < (NMI)) {                            \
    _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                            \
      mfma_mx(PA[mi][0], PA[mi][1], PB[ni], PSA[mi], PSB[ni], acc[mi][ni]);                     \
  }
  // Stage k (buffers SA/SB, the k-th of its scale group: position P = k % 4 in
  // buffer SS; stage k + 1 in NA/NB with scales NS). On entry the x registers
  // hold stage k's first step and every wave has passed the barrier after
  // which stage k is visible. The stage reads its second step (y), runs the
  // first step's MFMAs, waits for its own loads (stage k + 1) and LDS reads and
  // passes the barrier; then no wave reads stage k's buffers any more, so the
  // loads of stage k + 2 go into them (past the last stage: a harmless repeat
  // of the last one), and at the last stage of a scale group the scales of the
  // group after next go into the buffer of the group that just ended. Then it
  // reads stage k + 1's first step (x) and runs its own second step's MFMAs (y).
#define LMOE_STAGE(NMI, k, P, SA, SB, SS, NA, NB, NS, SFREE)                                      \
  {                                                                                             \
    LMOE_READ(NMI, SA, SB, SS, 1, 2 * (P) + 1, ya, yb, ysa, ysb)                                \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, xa, xb, xsa, xsb)                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    __builtin_amdgcn_s_waitcnt(kAllIdle);                                                       \
    bar();                                                                                      \
    LMOE_DATA(((k) + 2 < nst ? (k) + 2 : nst - 1), SA, SB)                                      \
    if ((P) == 3) {                                                                             \
      const int g_ = ((k) + 1) / 4 + 1;                                                         \
      LMOE_SCALES((g_ < ng ? g_ : ng - 1), SFREE)                                               \
    }                                                                                           \
    LMOE_READ(NMI, NA, NB, NS, 0, (2 * ((P) + 1)) & 7, xa, xb, xsa, xsb)                        \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, ya, yb, ysa, ysb)                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
  // Eight stages: two scale groups (buffers mS0, mS1), the stage buffers
  // alternating.
#define LMOE_KLOOP(NMI)                                                                          \
  {                                                                                             \
    LMOE_READ(NMI, mA0, mB0, mS0, 0, 0, xa, xb, xsa, xsb)                                       \
    for (int k0_ = 0; k0_ < nst; k0_ += 8) {                                                    \
      LMOE_STAGE(NMI, k0_ + 0, 0, mA0, mB0, mS0, mA1, mB1, mS0, mS1)                            \
      LMOE_STAGE(NMI, k0_ + 1, 1, mA1, mB1, mS0, mA0, mB0, mS0, mS1)                            \
      LMOE_STAGE(NMI, k0_ + 2, 2, mA0, mB0, mS0, mA1, mB1, mS0, mS1)                            \
      LMOE_STAGE(NMI, k0_ + 3, 3, mA1, mB1, mS0, mA0, mB0, mS1, mS0)                            \
      LMOE_STAGE(NMI, k0_ + 4, 0, mA0, mB0, mS1, mA1, mB1, mS1, mS0)                            \
      LMOE_STAGE(NMI, k0_ + 5, 1, mA1, mB1, mS1, mA0, mB0, mS1, mS0)                            \
      LMOE_STAGE(NMI, k0_ + 6, 2, mA0, mB0, mS1, mA1, mB1, mS1, mS0)                            \
      LMOE_STAGE(NMI, k0_ + 7, 3, mA1, mB1, mS1, mA0, mB0, mS0, mS1)                            \
    }                                                                                           \
  }

  // Prologue: scale groups 0 and 1, stage 0; wait for them; start stage 1.
  const int nst = K / 128;                   // a multiple of 8 (K % 1024 == 0)
  const int ng = nst / 4;
  LMOE_SCALES(0, mS0)
  LMOE_SCALES((ng > 1 ? 1 : 0), mS1)
  LMOE_DATA(0, mA0, mB0)
  __builtin_amdgcn_s_waitcnt(kAllIdle);
  bar();
  LMOE_DATA((nst > 1 ? 1 : 0), mA1, mB1)
  if (nmi > 2) {
    LMOE_KLOOP(4)
  } else if (nmi > 0) {
    LMOE_KLOOP(2)
  } else {
    LMOE_KLOOP(0)
  }
#undef LMOE_KLOOP
#undef LMOE_STAGE
#undef LMOE_MFMA
#undef LMOE_READ
#undef LMOE_SCALES
#undef LMOE_DATA
  __syncthreads();   // every load has landed and every wave has finished reading

  // ---- epilogue, in two halves of 128 rows (waves wm = 0, then wm = 1) ------
  // The staging area spans the two A stage buffers: rows [64 b, 64 b + 64) of
  // the half live in buffer b, 512 bytes per row.
  auto srow = [&](int r) -> unsigned char* { return ((r >> 6) ? mA1 : mA0) + (r & 63) * 512; };
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = mi * 32 + 8 * (v >> 2) + 4 * q + (v & 3);
          unsigned char* row = srow(r);
          if (EPI == EPI_SWIGLU) {
            // fp32 h at column c (0..127), 16-byte chunk c / 4 stored at
            // position (c / 4) ^ (r & 7) of the row
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float g = acc[mi][h][v], u = acc[mi][2 + h][v];
              const int c = wn * 64 + h * 32 + l32;
              *reinterpret_cast<float*>(row + ((((c >> 2) ^ (r & 7)) << 4) | ((c & 3) << 2))) =
                  g / (1.0f + __expf(-g)) * u;
            }
          } else {
            // bf16 y at column c (0..255)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
              reinterpret_cast<bf16_t*>(row)[wn * 128 + ni * 32 + l32] = f32_to_bf16(acc[mi][ni][v]);
          }
        }
    }
    __syncthreads();
    if (EPI == EPI_SWIGLU) {
      // one thread per (row, block of 32 columns): quantize to MXFP8 E4M3
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int item = it * NT + tid;
        const int r = item & 127, blk = item >> 7;
        const int m = m0 + half * 128 + r;
        if (m < m_end) {
          const unsigned char* row = srow(r);
          float v[32];
#pragma unroll
          for (int c4 = 0; c4 < 8; ++c4) {
            const float4 f = *reinterpret_cast<const float4*>(row + (((blk * 8 + c4) ^ (r & 7)) << 4));
            v[4 * c4] = f.x; v[4 * c4 + 1] = f.y; v[4 * c4 + 2] = f.z; v[4 * c4 + 3] = f.w;
          }
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
          const int X = mx_e4m3_exponent(amax);
          uint32_t w[8];
#pragma unroll
          for (int d = 0; d < 8; ++d)
            w[d] = (uint32_t)mx_e4m3_code(v[4 * d], X) | ((uint32_t)mx_e4m3_code(v[4 * d + 1], X) << 8) |
                   ((uint32_t)mx_e4m3_code(v[4 * d + 2], X) << 16) |
                   ((uint32_t)mx_e4m3_code(v[4 * d + 3], X) << 24);
          uint8_t* dst = static_cast<uint8_t*>(p.out) + (int64_t)m * p.ldo + n0 + 32 * blk;
          reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
          reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
          p.out_scales[(int64_t)m * p.ldos + n0 / 32 + blk] = mx_scale_code(X);
        }
      }
    } else {
      // 16-byte stores of the bf16 rows, then the sums of squares of the stored
      // values per row and 64-column group
      for (int i = tid; i < 128 * (BNB / 8); i += NT) {
        const int r = i / (BNB / 8), c = (i % (BNB / 8)) * 8;
        const int m = m0 + half * 128 + r;
        if (m >= m_end) continue;
        *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)m * p.ldo + n0 + c) =
            *reinterpret_cast<const uint4*>(srow(r) + 2 * c);
      }
      for (int i = tid; i < 128 * (BNB / 64); i += NT) {
        const int r = i / (BNB / 64), grp = i % (BNB / 64);
        const int m = m0 + half * 128 + r;
        if (m >= m_end) continue;
        const bf16_t* row = reinterpret_cast<const bf16_t*>(srow(r)) + grp * 64;
        float ssq = 0.f;
        for (int j = 0; j < 64; ++j) {
          const float y = bf16_to_f32(row[j]);
          ssq += y * y;
        }
        p.ss_out[(int64_t)m * p.ss_ld + (n0 + grp * 64) / 64] = ssq;
      }
    }
    __syncthreads();   // the half is read out before the next one is staged
  }
}

}  // namespace

int gemm256_mx_tile_m() { return BM; }

hipError_t launch_gemm256_mx(const Gemm256MxParams& p, EpiKind epi, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  const int grid = ((p.max_tiles + 7) / 8) * 8;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm256_mx_kernel<EPI_SWIGLU>, dim3(grid), dim3(NT), 0, s, p);
  else if (epi == EPI_DOWN)
    hipLaunchKernelGGL(gemm256_mx_kernel<EPI_DOWN>, dim3(grid), dim3(NT), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lmoe
