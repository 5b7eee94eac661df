// Weight-streaming grouped GEMM of the MXFP4-expert path, for experts that
// received few rows (decode): MXFP8 E4M3 token rows times MXFP4 (E2M1) expert
// weights, one E8M0 scale per 32 values along K on both sides, on gfx950's
// block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), fp32 accumulation.
// MXFP4 as the expert weight format: LMSYS Muse Spark Open blog, "NVFP4 as a
// third MMA type"; encodings: OCP Microscaling v1.0.
//
// As in the bf16 weight-streaming kernel, a few tokens per expert leave the
// expert GEMMs bound by reading the weights, so one wave64 per (expert, group
// of 64 weight rows) streams those rows over the whole K once and multiplies
// them with the expert's token rows (up to 2 tiles of 16).
//
// Stage: 256 K-columns. Weights: 64 rows x 128 bytes (whole lines), moved by 8
// direct global-to-LDS loads of 8 rows x 128 bytes, non-temporal, with the
// 16-byte chunk c of row r at position c ^ f(r), f(r) = ((r >> 1) ^ (r << 2)) & 7
// (conflict-free fragment reads). Token rows (fp8, 256 bytes per stage) and
// the scales of both operands go straight to registers: the token rows are
// re-read by every wave of the expert and come from L2, and keeping them out
// of LDS leaves 16 KiB of LDS per wave. (Scale bytes read from LDS would also
// sit behind the weight loads: the compiler cannot tell them apart from the
// LDS being filled and waits for all loads first.) The scales come 32 bytes
// per row at a time, every 4 stages: loading 8 bytes per row every stage
// issued as many requests as the weights themselves and cost about a fifth of
// the rate. Two stages: the loads of the next stage are in flight while the
// current one is multiplied.
//
// Scaled-MFMA operand layout (gfx950, 16x16x128; lane l: row r = l % 16 of the
// operand, group q = l / 16):
//   fp8 operand (tokens), 32 bytes: K [16q, 16q + 16) then K [64 + 16q, +16);
//   fp4 operand (weights), 16 bytes: K [32q, 32q + 32), low nibble first;
//   scale: one E8M0 byte per lane, for K [32q, 32q + 32) of its row;
//   result: register v of lane l at row 4q + v, column l % 16.
// Tokens are the result rows, weight rows the columns.
//
// EPI_SWIGLU: the wave's 64 weight rows are 32 gate rows and the matching 32 up
// rows, so each lane holds gate and up of the same (token, f); the wave's 32
// columns of H are exactly one MX block, quantized to MXFP8 E4M3 (codes +
// E8M0 scale) as the down GEMM's input, with the same arithmetic as the tiled
// kernel. EPI_DOWN: 64 bf16 output columns plus each token's sum of squares
// over them (of the stored values).
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace lmoe {

namespace {

constexpr int XMT = 2;                 // token tiles of 16: experts with up to 32 rows
constexpr int XKC = 256;               // K-columns per stage
constexpr int kBufWord3 = 0x00020000;  // raw buffer descriptor, fourth word (CDNA)

#define LMOE_AS3 __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

// Two weight stages, separate objects so that the compiler can tell them apart.
__shared__ __attribute__((aligned(16))) unsigned char xw0[64 * 128], xw1[64 * 128];

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

// s_waitcnt immediate: at most n vector-memory operations outstanding (no
// condition on the other counters).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate: no LDS (or scalar memory) operation outstanding.
constexpr int kLdsIdle = 15 | (3 << 14) | (7 << 4);

// Token operand of one MFMA K-step: the two 16-byte halves of the lane.
struct TokStep {
  u32x4_t h[2];
};

template <int EPI, int NMT>
__device__ __forceinline__ void stream_mx_body(const StreamMxParams& p, int e, int grp, int lo, int m_e) {
  const int lane = threadIdx.x, r16 = lane & 15, q = lane >> 4;
  const int lrow = lane >> 3, lc = lane & 7;
  const int K = p.K;
  const int rs = K / 32;                      // scale bytes per row
  const int64_t wrow_bytes = K / 2;

  // global weight row of local row lr (0..63)
  auto wrow = [&](int lr) -> int {
    return (EPI == EPI_SWIGLU) ? ((lr < 32 ? 0 : p.F - 32) + grp * 32 + lr) : (grp * 64 + lr);
  };

  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.B + (int64_t)e * p.N * wrow_bytes), (short)0, (int)p.b_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsBs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.Bs + (int64_t)e * p.N * rs), (short)0, (int)p.bs_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A), (short)0, (int)p.a_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsAs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.As), (short)0, (int)p.as_bytes, kBufWord3);

  // Weights: load j moves local rows 8j .. 8j+7 (lane: row 8j + lrow).
  uint32_t wo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int lr = 8 * j + lrow;
    wo[j] = (uint32_t)wrow(lr) * (uint32_t)wrow_bytes + (uint32_t)((lc ^ swz8(lr)) << 4);
  }
  // Scales, per group of 4 stages (1024 K-columns: 32 bytes of each row): lane
  // (r16, q) loads bytes [8q, 8q + 8) of the group's 32 for row r16 of every
  // weight tile and token tile, so that one load covers 16 rows x 32 contiguous
  // bytes. The byte a lane needs for K-step ks of stage c (K-block
  // 8c + 4 ks + q) then sits in lane r16 + 16 (c % 4), word ks, byte q, and a
  // lane shuffle fetches it.
  uint32_t wso[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) wso[t] = (uint32_t)wrow(t * 16 + r16) * (uint32_t)rs + 8 * q;
  // Tokens: tile mt, row r16 (rows past the expert's end read its last row;
  // never stored), the lane's 16-byte column q.
  uint32_t ao[NMT], aso[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int tr = mt * 16 + r16;
    int pos = lo + (tr < m_e ? tr : m_e - 1);
    if (p.a_rows) pos = p.a_rows[pos];       // gathered rows (gate/up: the assignment's token)
    ao[mt] = (uint32_t)pos * (uint32_t)K + 16 * q;
    aso[mt] = (uint32_t)pos * (uint32_t)rs + 8 * q;
  }

  // Loads of stage c: weights through LDS, tokens to registers; with SC, also
  // the scales of group g.
#define LMOE_ISSUE(c, SW, TA, SC, g, WS, TS)                                                      \
  {                                                                                               \
    const int c_ = (c);                                                                           \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                                 \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (LMOE_AS3 void*)((SW) + 1024 * j), 16,        \
                                               (int)wo[j], c_ * 128, 0, 2);                       \
    _Pragma("unroll") for (int mt = 0; mt < NMT; ++mt)                                            \
      _Pragma("unroll") for (int ks = 0; ks < 2; ++ks)                                            \
        _Pragma("unroll") for (int h = 0; h < 2; ++h)                                             \
          TA[mt][ks].h[h] = __builtin_amdgcn_raw_buffer_load_b128(rsA, (int)ao[mt] + 128 * ks + 64 * h, \
                                                                  c_ * XKC, 0);                  \
    if (SC) {                                                                                     \
      const int g_ = (g);                                                                         \
      _Pragma("unroll") for (int t = 0; t < 4; ++t)                                               \
        WS[t] = __builtin_amdgcn_raw_buffer_load_b64(rsBs, (int)wso[t], g_ * 32, 0);              \
      _Pragma("unroll") for (int mt = 0; mt < NMT; ++mt)                                          \
        TS[mt] = __builtin_amdgcn_raw_buffer_load_b64(rsAs, (int)aso[mt], g_ * 32, 0);            \
    }                                                                                             \
  }

  f32x4_t acc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LDS byte offsets of this lane's weight fragments: row t*16 + r16, chunk
  // 4 ks + q of the stage (the swizzle depends on the row's low 4 bits only).
  int fo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) fo[ks] = r16 * 128 + (((4 * ks + q) ^ swz8(r16)) << 4);

  // Stage c = 4 g + i of its group (i static).
#define LMOE_COMPUTE(i, SW, TA, WS, TS)                                                           \
  {                                                                                               \
    const int src_ = 4 * (r16 + 16 * (i));                                                        \
    _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                            \
      uint4 b[4];                                                                                 \
      int sb[4];                                                                                  \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                             \
        b[t] = *reinterpret_cast<const uint4*>((SW) + t * 2048 + fo[ks]);                         \
        sb[t] = __builtin_amdgcn_ds_bpermute(src_, (int)WS[t][ks]) >> (8 * q);                    \
      }                                                                                           \
      _Pragma("unroll") for (int mt = 0; mt < NMT; ++mt) {                                        \
        const i32x8_t av = {(int)TA[mt][ks].h[0].x, (int)TA[mt][ks].h[0].y, (int)TA[mt][ks].h[0].z,  \
                            (int)TA[mt][ks].h[0].w, (int)TA[mt][ks].h[1].x, (int)TA[mt][ks].h[1].y,  \
                            (int)TA[mt][ks].h[1].z, (int)TA[mt][ks].h[1].w};                      \
        const int sa = __builtin_amdgcn_ds_bpermute(src_, (int)TS[mt][ks]) >> (8 * q);            \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                           \
          const i32x8_t bv = {(int)b[t].x, (int)b[t].y, (int)b[t].z, (int)b[t].w, 0, 0, 0, 0};    \
          acc[mt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mt][t], 0, 4, 0, sa, \
                                                                        0, sb[t]);               \
        }                                                                                         \
      }                                                                                           \
    }                                                                                             \
  }
  // One stage (c = 4 g + i): the previous reads of the weight buffer about to
  // be refilled are done (all LDS reads complete), start the next stage's loads
  // (with the next group's scales after the group's last stage; at the end a
  // harmless repeat of the last stage and group into buffers no later stage
  // reads), wait until only those are outstanding, then an LDS acquire fence
  // keeps the stage's reads below the wait, and multiply. The scheduling
  // barrier keeps every load of the next stage ahead of the current stage's
  // work (which otherwise gets hoisted between them, with waits for its
  // operands).
#define LMOE_STAGE(c, i, SW, TA, WS, TS, NW, NTA, NWS, NTS)                                       \
  {                                                                                               \
    __builtin_amdgcn_s_waitcnt(kLdsIdle);                                                         \
    LMOE_ISSUE(((c) + 1 < nc ? (c) + 1 : nc - 1), NW, NTA, (i) == 3,                              \
               ((c) + 1 < nc ? ((c) + 1) / 4 : nc / 4 - 1), NWS, NTS)                             \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    __builtin_amdgcn_s_waitcnt(vm_wait(8 + 4 * NMT + ((i) == 3 ? 4 + NMT : 0)));                  \
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");                              \
    LMOE_COMPUTE(i, SW, TA, WS, TS)                                                               \
  }
  const int nc = K / XKC;                     // a multiple of 4 (K % 1024 == 0)
  TokStep ta0[NMT][2], ta1[NMT][2];
  u32x2_t ws0[4], ws1[4], ts0[NMT], ts1[NMT];
  // the buffers' previous reads (an earlier pass's epilogue) are done
  __builtin_amdgcn_s_waitcnt(kLdsIdle);
  LMOE_ISSUE(0, xw0, ta0, true, 0, ws0, ts0)
  for (int c = 0; c < nc; c += 8) {
    // group c / 4 (scales in ws0, ts0), then group c / 4 + 1 (ws1, ts1) if any
    LMOE_STAGE(c, 0, xw0, ta0, ws0, ts0, xw1, ta1, ws1, ts1)
    LMOE_STAGE(c + 1, 1, xw1, ta1, ws0, ts0, xw0, ta0, ws1, ts1)
    LMOE_STAGE(c + 2, 2, xw0, ta0, ws0, ts0, xw1, ta1, ws1, ts1)
    LMOE_STAGE(c + 3, 3, xw1, ta1, ws0, ts0, xw0, ta0, ws1, ts1)
    if (c + 4 < nc) {
      LMOE_STAGE(c + 4, 0, xw0, ta0, ws1, ts1, xw1, ta1, ws0, ts0)
      LMOE_STAGE(c + 5, 1, xw1, ta1, ws1, ts1, xw0, ta0, ws0, ts0)
      LMOE_STAGE(c + 6, 2, xw0, ta0, ws1, ts1, xw1, ta1, ws0, ts0)
      LMOE_STAGE(c + 7, 3, xw1, ta1, ws1, ts1, xw0, ta0, ws0, ts0)
    }
  }
#undef LMOE_STAGE
#undef LMOE_COMPUTE
#undef LMOE_ISSUE
  __builtin_amdgcn_s_waitcnt(0);             // the last (repeated) loads have landed; reads done

  // ---- epilogue: stage the output rows in LDS, store 16-byte chunks ----
  unsigned char* stile = xw0;
  if (EPI == EPI_SWIGLU) {
    // row i of the tile: the 32 E4M3 codes of H for columns grp*32 .. +32
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = mt * 16 + 4 * q + v;
        float hv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float g = acc[mt][h][v], u = acc[mt][2 + h][v];
          hv[h] = g / (1.0f + __expf(-g)) * u;
        }
        // block maximum over the 16 lanes holding this token's 32 values
        float amax = fmaxf(fabsf(hv[0]), fabsf(hv[1]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
        const int X = mx_e4m3_exponent(amax);
        const uint32_t c2 = mx_e4m3_code4(hv[0], hv[1], 0.f, 0.f, X);
        stile[i * 32 + r16] = (uint8_t)c2;
        stile[i * 32 + 16 + r16] = (uint8_t)(c2 >> 8);
        if (r16 == 0 && i < m_e) p.out_scales[(int64_t)(lo + i) * p.ldos + grp] = mx_scale_code(X);
      }
    }
    __syncthreads();
    for (int c = lane; c < m_e * 2; c += 64) {
      const int i = c >> 1, hf = c & 1;
      *reinterpret_cast<uint4*>(static_cast<uint8_t*>(p.out) + (int64_t)(lo + i) * p.ldo + grp * 32 + hf * 16) =
          *reinterpret_cast<const uint4*>(stile + i * 32 + hf * 16);
    }
  } else {
    bf16_t* sy = reinterpret_cast<bf16_t*>(stile);   // up to 32 x 64 bf16 = 4 KiB
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = mt * 16 + 4 * q + v;
        float ssq = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16_t y = f32_to_bf16(acc[mt][t][v]);
          sy[i * 64 + t * 16 + r16] = y;
          const float yf = bf16_to_f32(y);
          ssq += yf * yf;
        }
        // sum over the 16 lanes holding this token's 64 columns
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ssq += __shfl_xor(ssq, o, kWave);
        if (r16 == 0 && i < m_e) p.ss_out[(int64_t)(lo + i) * p.ss_ld + grp] = ssq;
      }
    }
    __syncthreads();
    for (int c = lane; c < m_e * 8; c += 64) {
      const int i = c >> 3, qc = c & 7;
      *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)(lo + i) * p.ldo + grp * 64 + qc * 8) =
          *reinterpret_cast<const uint4*>(sy + i * 64 + qc * 8);
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(64) void stream_mx_kernel(StreamMxParams p) {
  const int e = blockIdx.x / p.groups, grp = blockIdx.x % p.groups;
  const int lo = p.offsets[e];
  const int m_e = p.offsets[e + 1] - lo;
  if (m_e == 0 || m_e > p.max_rows) return;
  // Passes of up to 32 rows, each streaming the group's weights again (more
  // than one only when the host let experts above 32 rows come here: batches
  // too small for the tiled kernel to be worth a launch).
  for (int r0 = 0; r0 < m_e; r0 += XMT * 16) {
    const int m = m_e - r0 < XMT * 16 ? m_e - r0 : XMT * 16;
    if (m <= 16)
      stream_mx_body<EPI, 1>(p, e, grp, lo + r0, m);
    else
      stream_mx_body<EPI, 2>(p, e, grp, lo + r0, m);
  }
}

}  // namespace

int stream_mx_max_rows() { return XMT * 16; }

hipError_t launch_stream_mx(const StreamMxParams& p, EpiKind epi, hipStream_t s) {
  const int blocks = p.n_experts * p.groups;
  if (blocks == 0) return hipSuccess;
  if (p.K % 1024 != 0) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(stream_mx_kernel<EPI_SWIGLU>, dim3(blocks), dim3(64), 0, s, p);
  else if (epi == EPI_DOWN)
    hipLaunchKernelGGL(stream_mx_kernel<EPI_DOWN>, dim3(blocks), dim3(64), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lmoe
