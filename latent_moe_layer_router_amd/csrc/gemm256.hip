// Large-tile grouped GEMM for experts with many rows (prefill): the two expert
// GEMMs of the block (gate/up with the SwiGLU epilogue, down with the bf16
// output and per-64-column sums of squares).
//
// Tile 256 x 256 (A rows x B rows), K-step 64 bf16 (128 bytes per row), LDS
// double-buffered (2 x 64 KiB), 256 threads = 4 wave64 in a 2 x 2 grid, each
// wave a 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 bf16 (the accumulators live
// in AGPRs). Per K-step a wave reads 8 operand chunks from LDS for 16 MFMAs,
// which keeps LDS traffic well under its bandwidth.
//
// Scheduling for the 8 XCDs: the tiles of all experts form one index space
// ordered (expert, n-tile, m-tile); it is cut into 8 contiguous chunks and
// workgroup b (dispatched to XCD b % 8) takes tile (b % 8) * chunk + b / 8. So
// the CUs of one XCD work on the same expert at the same time and share its
// weight slices and token rows in their L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

constexpr int BM = 256, BNB = 256;   // A rows, B rows per tile
constexpr int NT = 256;
constexpr int ROWB = 128;
constexpr int CH = 8;
constexpr int STAGE_A = BM * ROWB, STAGE_B = BNB * ROWB;

__device__ __forceinline__ int swz(int row, int c) { return row * ROWB + ((c ^ (row & 7)) << 4); }

__device__ __forceinline__ void mfma32(const uint4& a, const uint4& b, f32x16_t& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm256_kernel(Gemm256Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * (STAGE_A + STAGE_B)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile of this workgroup (XCD-chunked order) --------------------------
  const int total = p.ntiles_n * p.mt_off[p.E];
  const int chunk = (total + 7) / 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int t = xcd * chunk + local;
  if (local >= chunk || t >= total) return;
  int lo = 0, hi = p.E;                      // expert e: ntiles_n*mt_off[e] <= t < ntiles_n*mt_off[e+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.ntiles_n * p.mt_off[mid] <= t) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mt_e = p.mt_off[e + 1] - p.mt_off[e];
  const int tl = t - p.ntiles_n * p.mt_off[e];
  const int ntile = tl / mt_e, mtile = tl % mt_e;
  const int row0 = p.offsets[e];
  const int m0 = row0 + mtile * BM;
  const int m_end = p.offsets[e + 1];
  const int n0 = ntile * (EPI == EPI_SWIGLU ? BNB / 2 : BNB);   // output column start

  // ---- global load addresses: thread loads chunk tid % 8 of rows tid/8 + 32 i
  const int lc = tid % CH, r0 = tid / CH;
  const bf16_t* Be = static_cast<const bf16_t*>(p.B) + (int64_t)e * p.b_expert_stride;
  auto a_row = [&](int r) -> const unsigned char* {
    int m = m0 + r;
    if (m >= m_end) m = m_end - 1;
    const int64_t src = (EPI == EPI_SWIGLU) ? (int64_t)p.a_gather[m] : (int64_t)m;
    return reinterpret_cast<const unsigned char*>(static_cast<const bf16_t*>(p.A) + src * p.lda) + lc * 16;
  };
  auto b_row = [&](int r) -> const unsigned char* {
    const int n = (EPI == EPI_SWIGLU) ? ((r < BNB / 2) ? (n0 + r) : (p.F + n0 + r - BNB / 2)) : (n0 + r);
    return reinterpret_cast<const unsigned char*>(Be + (int64_t)n * p.ldb) + lc * 16;
  };
#define LMOE_PTRS(X, f)                                                               \
  const unsigned char *X##0 = f(r0), *X##1 = f(r0 + 32), *X##2 = f(r0 + 64), *X##3 = f(r0 + 96), \
                      *X##4 = f(r0 + 128), *X##5 = f(r0 + 160), *X##6 = f(r0 + 192),              \
                      *X##7 = f(r0 + 224);
  LMOE_PTRS(pa, a_row)
  LMOE_PTRS(pb, b_row)
#undef LMOE_PTRS
  const int so = swz(r0, lc);                 // rows r0 + 32 i keep the same swizzle (32 % 8 == 0)

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  uint4 xa0, xa1, xa2, xa3, xa4, xa5, xa6, xa7, xb0, xb1, xb2, xb3, xb4, xb5, xb6, xb7;
#define LMOE_LD(off)                                                                       \
  xa0 = *reinterpret_cast<const uint4*>(pa0 + (off)); xa1 = *reinterpret_cast<const uint4*>(pa1 + (off)); \
  xa2 = *reinterpret_cast<const uint4*>(pa2 + (off)); xa3 = *reinterpret_cast<const uint4*>(pa3 + (off)); \
  xa4 = *reinterpret_cast<const uint4*>(pa4 + (off)); xa5 = *reinterpret_cast<const uint4*>(pa5 + (off)); \
  xa6 = *reinterpret_cast<const uint4*>(pa6 + (off)); xa7 = *reinterpret_cast<const uint4*>(pa7 + (off)); \
  xb0 = *reinterpret_cast<const uint4*>(pb0 + (off)); xb1 = *reinterpret_cast<const uint4*>(pb1 + (off)); \
  xb2 = *reinterpret_cast<const uint4*>(pb2 + (off)); xb3 = *reinterpret_cast<const uint4*>(pb3 + (off)); \
  xb4 = *reinterpret_cast<const uint4*>(pb4 + (off)); xb5 = *reinterpret_cast<const uint4*>(pb5 + (off)); \
  xb6 = *reinterpret_cast<const uint4*>(pb6 + (off)); xb7 = *reinterpret_cast<const uint4*>(pb7 + (off));
#define LMOE_ST(as, bs)                                                                    \
  *reinterpret_cast<uint4*>((as) + so) = xa0;                                              \
  *reinterpret_cast<uint4*>((as) + so + 32 * ROWB) = xa1;                                  \
  *reinterpret_cast<uint4*>((as) + so + 64 * ROWB) = xa2;                                  \
  *reinterpret_cast<uint4*>((as) + so + 96 * ROWB) = xa3;                                  \
  *reinterpret_cast<uint4*>((as) + so + 128 * ROWB) = xa4;                                 \
  *reinterpret_cast<uint4*>((as) + so + 160 * ROWB) = xa5;                                 \
  *reinterpret_cast<uint4*>((as) + so + 192 * ROWB) = xa6;                                 \
  *reinterpret_cast<uint4*>((as) + so + 224 * ROWB) = xa7;                                 \
  *reinterpret_cast<uint4*>((bs) + so) = xb0;                                              \
  *reinterpret_cast<uint4*>((bs) + so + 32 * ROWB) = xb1;                                  \
  *reinterpret_cast<uint4*>((bs) + so + 64 * ROWB) = xb2;                                  \
  *reinterpret_cast<uint4*>((bs) + so + 96 * ROWB) = xb3;                                  \
  *reinterpret_cast<uint4*>((bs) + so + 128 * ROWB) = xb4;                                 \
  *reinterpret_cast<uint4*>((bs) + so + 160 * ROWB) = xb5;                                 \
  *reinterpret_cast<uint4*>((bs) + so + 192 * ROWB) = xb6;                                 \
  *reinterpret_cast<uint4*>((bs) + so + 224 * ROWB) = xb7;

  // LDS rows of this lane's MFMA operands: A rows wm*128 + 32 mi + l32; B rows:
  // SwiGLU pairs gate (ni = 0, 1) and up (ni = 2, 3) of the same 64 columns.
  const int l32 = lane & 31, half = lane >> 5;
  const int abase = wm * 128 + l32;
  auto brow_of = [&](int ni) {
    return (EPI == EPI_SWIGLU) ? ((ni >> 1) * (BNB / 2) + wn * 64 + (ni & 1) * 32 + l32)
                               : (wn * 128 + ni * 32 + l32);
  };
  const int bb0 = brow_of(0), bb1 = brow_of(1), bb2 = brow_of(2), bb3 = brow_of(3);
  // rows of this wave that hold real tokens (tail tiles skip empty 32-row groups)
  const int mrows = m_end - (m0 + wm * 128);
  const int nmi = mrows <= 0 ? 0 : (mrows >= 128 ? 4 : (mrows + 31) / 32);

  const int nk = p.K * 2 / ROWB;
  LMOE_LD(0)
  LMOE_ST(lds, lds + STAGE_A)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t off = (int64_t)(kt + 1) * ROWB;
      LMOE_LD(off)
    }
    const unsigned char* as = lds + st * (STAGE_A + STAGE_B);
    const unsigned char* bs = as + STAGE_A;
#pragma unroll
    for (int s = 0; s < CH / 2; ++s) {
      const int c = 2 * s + half;
      const uint4 b0 = *reinterpret_cast<const uint4*>(bs + swz(bb0, c));
      const uint4 b1 = *reinterpret_cast<const uint4*>(bs + swz(bb1, c));
      const uint4 b2 = *reinterpret_cast<const uint4*>(bs + swz(bb2, c));
      const uint4 b3 = *reinterpret_cast<const uint4*>(bs + swz(bb3, c));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if (mi < nmi) {
          const uint4 a = *reinterpret_cast<const uint4*>(as + swz(abase + mi * 32, c));
          mfma32(a, b0, acc[mi][0]);
          mfma32(a, b1, acc[mi][1]);
          mfma32(a, b2, acc[mi][2]);
          mfma32(a, b3, acc[mi][3]);
        }
      }
    }
    if (more) {
      unsigned char* an = lds + (st ^ 1) * (STAGE_A + STAGE_B);
      LMOE_ST(an, an + STAGE_A)
    }
    __syncthreads();
  }
#undef LMOE_LD
#undef LMOE_ST

  // ---- epilogue: stage [256][OBN] bf16 in LDS, 16-byte stores ----------------
  constexpr int OBN = (EPI == EPI_SWIGLU) ? BNB / 2 : BNB;
  bf16_t* stile = reinterpret_cast<bf16_t*>(lds);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 128 + mi * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float g = acc[mi][h][v], u = acc[mi][2 + h][v];
          stile[r * OBN + wn * 64 + h * 32 + l32] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) stile[r * OBN + wn * 128 + ni * 32 + l32] = f32_to_bf16(acc[mi][ni][v]);
      }
    }
  __syncthreads();
  constexpr int CPR = OBN / 8;
  for (int i = tid; i < BM * CPR; i += NT) {
    const int r = i / CPR, c = (i % CPR) * 8;
    const int m = m0 + r;
    if (m >= m_end) continue;
    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)m * p.ldo + n0 + c) =
        *reinterpret_cast<const uint4*>(stile + r * OBN + c);
  }
  if (EPI == EPI_DOWN) {
    // sums of squares of the stored bf16 values, per row and 64-column group
    for (int i = tid; i < BM * (BNB / 64); i += NT) {
      const int r = i / (BNB / 64), grp = i % (BNB / 64);
      const int m = m0 + r;
      if (m >= m_end) continue;
      const bf16_t* row = stile + r * OBN + grp * 64;
      float ssq = 0.f;
      for (int j = 0; j < 64; ++j) {
        const float y = bf16_to_f32(row[j]);
        ssq += y * y;
      }
      p.ss_out[(int64_t)m * p.ss_ld + (n0 + grp * 64) / 64] = ssq;
    }
  }
}

}  // namespace

int gemm256_tile_m() { return BM; }

hipError_t launch_gemm256(const Gemm256Params& p, EpiKind epi, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  const int grid = ((p.max_tiles + 7) / 8) * 8;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm256_kernel<EPI_SWIGLU>, dim3(grid), dim3(NT), 0, s, p);
  else if (epi == EPI_DOWN)
    hipLaunchKernelGGL(gemm256_kernel<EPI_DOWN>, dim3(grid), dim3(NT), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lmoe
