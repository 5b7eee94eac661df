// Weight-streaming grouped GEMM for experts that received few rows (decode).
//
// With a handful of tokens per expert the expert GEMMs are bound by reading
// the weights from HBM, so the kernel is shaped for bytes in flight rather than
// for MFMA reuse: one wave64 per (expert, group of 64 weight rows) streams those
// rows over the whole K with 16-byte loads straight into registers (no LDS in
// the main loop, no block barrier), and multiplies them with the expert's
// token rows (up to 4 tiles of 16) on MFMA 16x16x32. Every weight byte is read
// exactly once; the token rows come from L2.
//
// MFMA 16x16x32 layout (CDNA4): lane l supplies row l % 16 and the 8-element
// K-chunk l / 16 of the 32-wide K-slice, for both operands; the 16x16 result
// leaves register v of lane l at row 4*(l/16) + v, column l % 16. Tokens are the
// result rows, weight rows the columns.
//
// EPI_SWIGLU: the wave's 64 weight rows are 32 gate rows and the matching 32 up
// rows, so each lane holds gate and up of the same (token, f) and applies
// silu(gate) * up in registers.
// EPI_DOWN: 64 output columns; the wave also reduces each token's sum of
// squares over those columns (of the bf16-rounded values it stores).
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

constexpr int MT = 4;   // token tiles of 16 per wave: experts with up to 64 rows
constexpr int U = 4;    // K-slices of 32 per loop iteration (256 bytes of each weight row)

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ void mfma16(const uint4& a, const uint4& b, f32x4& acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <int EPI>
__global__ __launch_bounds__(64) void stream_kernel(StreamParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t stile[MT * 16 * 64];
  const int e = blockIdx.x / p.groups, grp = blockIdx.x % p.groups;
  const int lo = p.offsets[e];
  const int m_e = p.offsets[e + 1] - lo;
  if (m_e == 0 || m_e > p.max_rows) return;
  const int lane = threadIdx.x, r16 = lane & 15, kq = lane >> 4;
  const int n_mt = (m_e + 15) >> 4;        // token tiles in use (wave-uniform)

  const bf16_t* Be = static_cast<const bf16_t*>(p.B) + (int64_t)e * p.b_expert_stride;
  const bf16_t* brow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int row;
    if (EPI == EPI_SWIGLU) row = (t < 2 ? 0 : p.F) + grp * 32 + (t & 1) * 16 + r16;
    else row = grp * 64 + t * 16 + r16;
    brow[t] = Be + (int64_t)row * p.ldb + kq * 8;
  }
  const bf16_t* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int i = mt * 16 + r16;
    if (i >= m_e) i = m_e - 1;               // rows past the end load a valid row; never stored
    const int64_t src = (EPI == EPI_SWIGLU) ? (int64_t)p.a_gather[lo + i] : (int64_t)(lo + i);
    arow[mt] = static_cast<const bf16_t*>(p.A) + src * p.lda + kq * 8;
  }

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k = 0; k < p.K; k += 32 * U) {
    uint4 b[U][4], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) b[u][t] = *reinterpret_cast<const uint4*>(brow[t] + k + 32 * u);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < n_mt) a[u][mt] = *reinterpret_cast<const uint4*>(arow[mt] + k + 32 * u);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < n_mt)
#pragma unroll
          for (int t = 0; t < 4; ++t) mfma16(a[u][mt], b[u][t], acc[mt][t]);
  }

  // ---- epilogue: stage the [rows][cols] tile in LDS, store 16-byte chunks ----
  constexpr int OC = (EPI == EPI_SWIGLU) ? 32 : 64;   // output columns of the wave
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= n_mt) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = mt * 16 + 4 * kq + v;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float g = acc[mt][h][v], u = acc[mt][2 + h][v];
          stile[i * OC + h * 16 + r16] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
        }
      } else {
        float ssq = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16_t y = f32_to_bf16(acc[mt][t][v]);
          stile[i * OC + t * 16 + r16] = y;
          const float yf = bf16_to_f32(y);
          ssq += yf * yf;
        }
        // sum over the 16 lanes holding this token's 64 columns
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ssq += __shfl_xor(ssq, o, kWave);
        if (r16 == 0 && i < m_e) p.ss_out[(int64_t)(lo + i) * p.ss_ld + grp] = ssq;
      }
    }
  }
  __syncthreads();
  constexpr int CPR = OC / 8;                // 16-byte chunks per output row
  const int col0 = grp * OC;
  for (int c = lane; c < m_e * CPR; c += 64) {
    const int i = c / CPR, q = c % CPR;
    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)(lo + i) * p.ldo + col0 + q * 8) =
        *reinterpret_cast<const uint4*>(stile + i * OC + q * 8);
  }
}

// Dense projections of a small batch (router + pooler, unpooler at decode
// sizes): one wave per (group of 64 weight rows, K-slice), all T <= 128 tokens
// held as up to 8 MFMA row tiles, weights streamed once. Each wave writes its
// fp32 partial sums to part[slice][t][n]; splitk_reduce adds the slices in
// slice order (deterministic), then applies the bias and the output type.
constexpr int MTD = 8;
constexpr int UD = 2;

__global__ __launch_bounds__(64) void dense_stream_kernel(DenseStreamParams p) {
  const int grp = blockIdx.x / p.slices, sl = blockIdx.x % p.slices;
  const int lane = threadIdx.x, r16 = lane & 15, kq = lane >> 4;
  const int n_mt = (p.T + 15) >> 4;
  const int kspan = p.K / p.slices, k0 = sl * kspan;
  const bf16_t* brow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = grp * 64 + t * 16 + r16;
    const bf16_t* b;
    if (n < p.n_split) b = static_cast<const bf16_t*>(p.B0) + (int64_t)n * p.ldb;
    else if (n < p.N) b = static_cast<const bf16_t*>(p.B1) + (int64_t)(n - p.n_split) * p.ldb;
    else b = static_cast<const bf16_t*>(p.B0);            // past N: a valid row, never stored
    brow[t] = b + k0 + kq * 8;
  }
  const bf16_t* arow[MTD];
#pragma unroll
  for (int mt = 0; mt < MTD; ++mt) {
    int i = mt * 16 + r16;
    if (i >= p.T) i = p.T - 1;
    arow[mt] = static_cast<const bf16_t*>(p.A) + (int64_t)i * p.lda + k0 + kq * 8;
  }
  f32x4 acc[MTD][4];
#pragma unroll
  for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kspan; k += 32 * UD) {
    uint4 b[UD][4], a[UD][MTD];
#pragma unroll
    for (int u = 0; u < UD; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) b[u][t] = *reinterpret_cast<const uint4*>(brow[t] + k + 32 * u);
#pragma unroll
    for (int u = 0; u < UD; ++u)
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt)
        if (mt < n_mt) a[u][mt] = *reinterpret_cast<const uint4*>(arow[mt] + k + 32 * u);
#pragma unroll
    for (int u = 0; u < UD; ++u)
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt)
        if (mt < n_mt)
#pragma unroll
          for (int t = 0; t < 4; ++t) mfma16(a[u][mt], b[u][t], acc[mt][t]);
  }
  float* part = p.part + (int64_t)sl * p.T * p.N;
#pragma unroll
  for (int mt = 0; mt < MTD; ++mt) {
    if (mt >= n_mt) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = mt * 16 + 4 * kq + v;
      if (i >= p.T) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = grp * 64 + t * 16 + r16;
        if (n < p.N) part[(int64_t)i * p.N + n] = acc[mt][t][v];
      }
    }
  }
}

// out = sum over slices of part[slice][t][n] (slice order), split like EPI_F32:
// columns [0, n_split) -> out0 (fp32, or bf16 if out0_bf16), [n_split, N) -> out1 + bias1.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(DenseStreamParams p) {
  const int64_t total = (int64_t)p.T * p.N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int sl = 0; sl < p.slices; ++sl) s += p.part[sl * total + i];
    const int t = (int)(i / p.N), n = (int)(i % p.N);
    if (n < p.n_split) {
      if (p.out0_bf16) static_cast<bf16_t*>(p.out0)[(int64_t)t * p.ldo0 + n] = f32_to_bf16(s);
      else static_cast<float*>(p.out0)[(int64_t)t * p.ldo0 + n] = s;
    } else {
      const int c = n - p.n_split;
      static_cast<float*>(p.out1)[(int64_t)t * p.ldo1 + c] = s + (p.bias1 ? p.bias1[c] : 0.f);
    }
  }
}

}  // namespace

int stream_max_rows() { return MT * 16; }
int dense_stream_max_tokens() { return MTD * 16; }

int dense_stream_slices(int K) {
  int s = K / 512;
  if (s < 1) s = 1;
  while (s > 1 && K % (s * 32 * UD) != 0) --s;
  return K % (s * 32 * UD) == 0 ? s : 0;
}

hipError_t launch_dense_stream(const DenseStreamParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int groups = (p.N + 63) / 64;
  hipLaunchKernelGGL(dense_stream_kernel, dim3(groups * p.slices), dim3(64), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t total = (int64_t)p.T * p.N;
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_stream(const StreamParams& p, EpiKind epi, hipStream_t s) {
  const int blocks = p.n_experts * p.groups;
  if (blocks == 0) return hipSuccess;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(stream_kernel<EPI_SWIGLU>, dim3(blocks), dim3(64), 0, s, p);
  else if (epi == EPI_DOWN)
    hipLaunchKernelGGL(stream_kernel<EPI_DOWN>, dim3(blocks), dim3(64), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lmoe
