// MFMA GEMM engine: C = A . B^T with both operands K-contiguous ("NT"), fp32
// accumulation, for the four GEMMs of the block:
//   router + pooler (one launch, two B matrices)        -> EPI_F32
//   gate/up, grouped per expert, A rows gathered          -> EPI_SWIGLU
//   down, grouped per expert                              -> EPI_DOWN
//   unpooler                                              -> EPI_ACT
//
// Block tile 128 x 128, 256 threads = 4 wave64 in a 2 x 2 grid, each wave a
// 64 x 64 sub-tile made of 2 x 2 MFMA 32x32 tiles. A K-step stages 128 bytes of
// every tile row (64 bf16 or 32 fp32) in LDS, double-buffered; rows are split
// in 16-byte chunks placed at (chunk ^ (row & 7)) so that the 32 rows an MFMA
// operand read touches spread over all banks.
//
// MFMA operand layout (CDNA3/CDNA4 32x32 family): lane l supplies row (or
// column) l % 32 and its half l / 32 of the K-slice; the 32x32 result leaves
// register v of lane l at row 8*(v/4) + 4*(l/32) + v%4, column l % 32. Each lane
// reads one 16-byte chunk per row and K-slice; A and B pair their elements the
// same way, so the order of K inside an instruction never matters.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

constexpr int BM = kGemmBM, BN = kGemmBN;
constexpr int NT = 256;          // threads per block
constexpr int ROWB = 128;        // bytes per tile row per K-step
constexpr int CH = ROWB / 16;    // 16-byte chunks per tile row

__device__ __forceinline__ int swz(int row, int c) { return row * ROWB + ((c ^ (row & 7)) << 4); }

// One 32x32 MFMA step on a 16-byte chunk of A and of B.
template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  __device__ static void step(const uint4& a, const uint4& b, f32x16_t& acc) {
    bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
    bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  __device__ static void step(const uint4& a, const uint4& b, f32x16_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

template <typename T, int EPI>
__global__ __launch_bounds__(NT) void gemm_nt_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * (BM + BN) * ROWB];
  unsigned char* As = lds;
  unsigned char* Bs = lds + 2 * BM * ROWB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool kGrouped = (EPI == EPI_SWIGLU || EPI == EPI_DOWN);

  // ---- tile coordinates -------------------------------------------------
  int m0, m_end, expert = 0;
  if (kGrouped) {
    const int slot = blockIdx.x;
    if (slot >= *p.n_tiles) return;
    expert = p.tiles[2 * slot];
    m0 = p.tiles[2 * slot + 1];
    m_end = p.offsets[expert + 1];
  } else {
    m0 = blockIdx.x * BM;
    m_end = p.M;
  }
  const int n0 = blockIdx.y * (EPI == EPI_SWIGLU ? BN / 2 : BN);

  // ---- per-thread row pointers for the global loads ---------------------
  // Thread t loads chunk t % 8 of tile rows t / 8 + 32 * i, i = 0..3, of both
  // operands. Four named pointers (not an array) keep everything in registers.
  const int lc = tid % CH;                 // chunk this thread loads
  const T* Bbase = static_cast<const T*>(p.B0);
  if (kGrouped) Bbase += (int64_t)expert * p.b_expert_stride;
  auto a_row = [&](int r) -> const unsigned char* {
    int m = m0 + r;
    if (m >= m_end) m = m_end - 1;          // rows past the end load a valid row; never stored
    if (p.a_rows) m = p.a_rows[m];          // gathered rows (gate/up: the assignment's token)
    return reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.A) + (int64_t)m * p.lda) + lc * 16;
  };
  auto b_row = [&](int r) -> const unsigned char* {
    const T* brow;
    if (EPI == EPI_SWIGLU) {
      const int f = (r < BN / 2) ? (n0 + r) : (p.F + n0 + r - BN / 2);
      brow = Bbase + (int64_t)f * p.ldb;
    } else {
      // Columns past N load row 0 of B0 (a valid row) and are never stored.
      const int n = n0 + r;
      if (EPI == EPI_F32 && n >= p.n_split)
        brow = (n < p.N) ? static_cast<const T*>(p.B1) + (int64_t)(n - p.n_split) * p.ldb : Bbase;
      else
        brow = Bbase + (int64_t)(n < p.N ? n : 0) * p.ldb;
    }
    return reinterpret_cast<const unsigned char*>(brow) + lc * 16;
  };
  const int r0 = tid / CH;
  const unsigned char* pa0 = a_row(r0);
  const unsigned char* pa1 = a_row(r0 + 32);
  const unsigned char* pa2 = a_row(r0 + 64);
  const unsigned char* pa3 = a_row(r0 + 96);
  const unsigned char* pb0 = b_row(r0);
  const unsigned char* pb1 = b_row(r0 + 32);
  const unsigned char* pb2 = b_row(r0 + 64);
  const unsigned char* pb3 = b_row(r0 + 96);
  const int so0 = swz(r0, lc), so1 = swz(r0 + 32, lc), so2 = swz(r0 + 64, lc), so3 = swz(r0 + 96, lc);

  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  // Rows of the LDS tiles this lane reads for its MFMA operands (byte offsets of
  // the row starts; the chunk swizzle is applied per read).
  const int l32 = lane & 31, half = lane >> 5;
  const int arow0 = wm * 64 + l32, arow1 = wm * 64 + 32 + l32;
  const int brow0 = (EPI == EPI_SWIGLU) ? (wn * 32 + l32) : (wn * 64 + l32);
  const int brow1 = (EPI == EPI_SWIGLU) ? (BN / 2 + wn * 32 + l32) : (wn * 64 + 32 + l32);

  const int nk = p.K * (int)sizeof(T) / ROWB;
  uint4 xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3;
#define LMOE_GLOAD(off)                                              \
  xa0 = *reinterpret_cast<const uint4*>(pa0 + (off));                \
  xa1 = *reinterpret_cast<const uint4*>(pa1 + (off));                \
  xa2 = *reinterpret_cast<const uint4*>(pa2 + (off));                \
  xa3 = *reinterpret_cast<const uint4*>(pa3 + (off));                \
  xb0 = *reinterpret_cast<const uint4*>(pb0 + (off));                \
  xb1 = *reinterpret_cast<const uint4*>(pb1 + (off));                \
  xb2 = *reinterpret_cast<const uint4*>(pb2 + (off));                \
  xb3 = *reinterpret_cast<const uint4*>(pb3 + (off));
#define LMOE_SSTORE(ab, bb)                                          \
  *reinterpret_cast<uint4*>((ab) + so0) = xa0;                       \
  *reinterpret_cast<uint4*>((ab) + so1) = xa1;                       \
  *reinterpret_cast<uint4*>((ab) + so2) = xa2;                       \
  *reinterpret_cast<uint4*>((ab) + so3) = xa3;                       \
  *reinterpret_cast<uint4*>((bb) + so0) = xb0;                       \
  *reinterpret_cast<uint4*>((bb) + so1) = xb1;                       \
  *reinterpret_cast<uint4*>((bb) + so2) = xb2;                       \
  *reinterpret_cast<uint4*>((bb) + so3) = xb3;
  LMOE_GLOAD(0)
  LMOE_SSTORE(As, Bs)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t off = (int64_t)(kt + 1) * ROWB;
      LMOE_GLOAD(off)
    }
    const unsigned char* as = As + st * BM * ROWB;
    const unsigned char* bs = Bs + st * BN * ROWB;
#pragma unroll
    for (int s = 0; s < CH / 2; ++s) {
      const int c = 2 * s + half;
      const uint4 a0 = *reinterpret_cast<const uint4*>(as + swz(arow0, c));
      const uint4 a1 = *reinterpret_cast<const uint4*>(as + swz(arow1, c));
      const uint4 b0 = *reinterpret_cast<const uint4*>(bs + swz(brow0, c));
      const uint4 b1 = *reinterpret_cast<const uint4*>(bs + swz(brow1, c));
      Mfma<T>::step(a0, b0, acc[0][0]);
      Mfma<T>::step(a0, b1, acc[0][1]);
      Mfma<T>::step(a1, b0, acc[1][0]);
      Mfma<T>::step(a1, b1, acc[1][1]);
    }
    if (more) {
      unsigned char* an = As + (st ^ 1) * BM * ROWB;
      unsigned char* bn = Bs + (st ^ 1) * BN * ROWB;
      LMOE_SSTORE(an, bn)
    }
    __syncthreads();
  }
#undef LMOE_GLOAD
#undef LMOE_SSTORE

  // ---- epilogue ----------------------------------------------------------
  // The output tile is staged in LDS (free after the last K-step) as row-major
  // [BM][OBN] of the output type, then written with 16-byte stores per lane, so
  // every store instruction covers whole contiguous row segments.
  // Register v of tile (mi, ni) holds row wm*64 + mi*32 + 8*(v/4) + 4*half + v%4.
  using OT = typename std::conditional<EPI == EPI_F32, float, T>::type;
  constexpr int OBN = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  OT* stile = reinterpret_cast<OT*>(lds);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      if (EPI == EPI_SWIGLU) {
        const float g = acc[mi][0][v], u = acc[mi][1][v];
        stile[r * OBN + wn * 32 + l32] = Elem<T>::from_f32(g / (1.0f + __expf(-g)) * u);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int c = wn * 64 + ni * 32 + l32;
          float val = acc[mi][ni][v];
          if (EPI == EPI_F32) {
            const int n = n0 + c;
            if (p.bias1 && n >= p.n_split && n < p.N) val += p.bias1[n - p.n_split];
            stile[r * OBN + c] = val;
          } else {
            stile[r * OBN + c] = Elem<T>::from_f32(val);   // EPI_DOWN: y rounded once, here
          }
        }
      }
    }
  __syncthreads();

  constexpr int EPC = 16 / (int)sizeof(OT);   // elements per 16-byte chunk
  constexpr int CPR = OBN / EPC;              // chunks per tile row
  for (int i = tid; i < BM * CPR; i += NT) {
    const int r = i / CPR, c = (i % CPR) * EPC;
    const int m = m0 + r;
    const int n = n0 + c;
    if (m >= m_end) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(stile + r * OBN + c);
    if (EPI == EPI_F32) {
      if (n < p.n_split) {
        *reinterpret_cast<uint4*>(static_cast<float*>(p.out0) + (int64_t)m * p.ldo0 + n) = val;
      } else {
        // second output (router logits): any width, so element stores
        const float* f = reinterpret_cast<const float*>(stile + r * OBN + c);
#pragma unroll
        for (int q = 0; q < EPC; ++q)
          if (n + q < p.N) static_cast<float*>(p.out1)[(int64_t)m * p.ldo1 + n + q - p.n_split] = f[q];
      }
    } else if (n < p.N || EPI == EPI_SWIGLU) {
      *reinterpret_cast<uint4*>(static_cast<T*>(p.out0) + (int64_t)m * p.ldo0 + n) = val;
    }
  }
  if (EPI == EPI_DOWN) {
    // Sum of squares of the stored (rounded) values per row and 64-column group.
    const int r = tid >> 1, grp = tid & 1;
    const int m = m0 + r, nb = n0 + grp * 64;
    if (m < m_end && nb < p.N) {
      const OT* row = stile + r * OBN + grp * 64;
      float ssq = 0.f;
      for (int j = 0; j < 64; ++j) {
        const float y = Elem<T>::to_f32(row[j]);
        ssq += y * y;
      }
      p.ss_out[(int64_t)m * p.ss_ld + nb / 64] = ssq;
    }
  }
}

template <typename T, int EPI>
hipError_t launch_t(const GemmParams& p, hipStream_t s) {
  dim3 grid;
  if (EPI == EPI_SWIGLU || EPI == EPI_DOWN) {
    grid.x = p.max_slots;
    grid.y = (EPI == EPI_SWIGLU) ? p.F / (BN / 2) : (p.N + BN - 1) / BN;
  } else {
    grid.x = (p.M + BM - 1) / BM;
    grid.y = (p.N + BN - 1) / BN;
  }
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_nt_kernel<T, EPI>), grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, EpiKind epi, bool bf16, hipStream_t s) {
  if (bf16) {
    switch (epi) {
      case EPI_F32: return launch_t<bf16_t, EPI_F32>(p, s);
      case EPI_ACT: return launch_t<bf16_t, EPI_ACT>(p, s);
      case EPI_SWIGLU: return launch_t<bf16_t, EPI_SWIGLU>(p, s);
      case EPI_DOWN: return launch_t<bf16_t, EPI_DOWN>(p, s);
    }
  } else {
    switch (epi) {
      case EPI_F32: return launch_t<float, EPI_F32>(p, s);
      case EPI_ACT: return launch_t<float, EPI_ACT>(p, s);
      case EPI_SWIGLU: return launch_t<float, EPI_SWIGLU>(p, s);
      case EPI_DOWN: return launch_t<float, EPI_DOWN>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lmoe
