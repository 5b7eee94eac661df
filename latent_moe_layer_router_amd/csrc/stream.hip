// Weight-streaming grouped GEMM for experts that received few rows (decode).
//
// With a handful of tokens per expert the expert GEMMs are bound by reading
// the weights from HBM, so the kernel is shaped for the memory system rather
// than for MFMA reuse: one wave64 per (expert, group of 64 weight rows) streams
// those rows over the whole K, and multiplies them with the expert's token rows
// (up to 4 tiles of 16) on MFMA 16x16x32. Every weight byte is read once.
//
// The weights go through LDS so that each load instruction covers whole
// 128-byte lines: a direct global-to-LDS load moves 8 rows x 128 bytes (lane i:
// row i / 8, 16-byte chunk i % 8), marked non-temporal. In the MFMA layout a
// lane needs 16 different rows, which would make every load cover half lines;
// on MI355X half-line loads stream at about 5.8 TB/s, whole-line non-temporal
// ones at about 6.8 TB/s. The token rows take the same path (from L2), so one
// wait count covers a whole stage. Two stages of 64 K-columns: the loads of
// the next stage are in flight while the current one is multiplied.
//
// LDS layout of a stage: rows of 128 bytes (64 bf16), the 16-byte chunk c of
// row r stored at position c ^ f(r), f(r) = ((r >> 1) ^ (r << 2)) & 7, which
// makes the 16-row fragment reads conflict-free for 8- and 16-lane phases.
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

constexpr int MT = 4;            // token tiles of 16 per wave: experts with up to 64 rows
constexpr int KC = 64;           // K-columns per stage (128 bytes of each row)
constexpr int kBufWord3 = 0x00020000;   // raw buffer descriptor, fourth word (CDNA)

#define LMOE_AS3 __attribute__((address_space(3)))

// Two stages of 64 weight rows and up to 64 token rows, 128 bytes each; separate
// objects so that the compiler can tell the stages apart.
__shared__ __attribute__((aligned(16))) unsigned char sw0[64 * 128], sw1[64 * 128];
__shared__ __attribute__((aligned(16))) unsigned char sa0[64 * 128], sa1[64 * 128];

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ void mfma16(const uint4& a, const uint4& b, f32x4& acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

// s_waitcnt immediate: at most n vector-memory operations outstanding (no
// condition on the other counters).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate: no LDS (or scalar memory) operation outstanding.
constexpr int kLdsIdle = 15 | (3 << 14) | (7 << 4);

// One wave streams one (expert, group of 64 weight rows) through its own four
// 8 KiB LDS buffers (weight and token stages 0 and 1; the epilogue stages the
// output tile in sw0). Only this wave touches them.
template <int EPI, int NMT>
__device__ __forceinline__ void stream_body(const StreamParams& p, int e, int grp, int lo, int m_e,
                                            unsigned char* sw0, unsigned char* sw1, unsigned char* sa0,
                                            unsigned char* sa1) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, kq = lane >> 4;
  const int lrow = lane >> 3, lc = lane & 7;

  // Weights: load j moves local rows 8j .. 8j+7 (lane: row 8j + lrow). In the
  // packed layout a stage's 64 columns of a row group are one 8 KiB block, so
  // each load moves 1 KiB of consecutive bytes; the stages are kw bytes apart.
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(static_cast<const bf16_t*>(p.B) + (int64_t)e * p.b_expert_stride), (short)0,
      (int)p.b_bytes, kBufWord3);
  uint32_t wo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int lr = 8 * j + lrow;
    const int row = (EPI == EPI_SWIGLU) ? ((lr < 32 ? 0 : p.F - 32) + grp * 32 + lr) : (grp * 64 + lr);
    wo[j] = (p.b_packed ? (uint32_t)(row >> 6) * (uint32_t)(p.K >> 6) * 8192u + (uint32_t)(row & 63) * 128u
                        : (uint32_t)row * (uint32_t)(p.ldb * 2)) +
            (uint32_t)((lc ^ swz8(lr)) << 4);
  }
  const int kw = p.b_packed ? 8192 : KC * 2;
  // Tokens: load i moves token rows 8i .. 8i+7 of the expert (rows past its end
  // load its last row; never stored).
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), (short)0, (int)p.a_bytes, kBufWord3);
  uint32_t ao[2 * NMT];
#pragma unroll
  for (int i = 0; i < 2 * NMT; ++i) {
    const int tr = 8 * i + lrow;
    int pos = lo + (tr < m_e ? tr : m_e - 1);
    if (p.a_rows) pos = p.a_rows[pos];       // gathered rows (gate/up: the assignment's token)
    ao[i] = (uint32_t)pos * (uint32_t)(p.lda * 2) + (uint32_t)((lc ^ swz8(tr)) << 4);
  }
#define LMOE_ISSUE(c, SW, SA)                                                                   \
  {                                                                                            \
    const int ko_ = (c) * KC * 2, kow_ = (c) * kw;                                             \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                              \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (LMOE_AS3 void*)((SW) + 1024 * j), 16,     \
                                               (int)wo[j], kow_, 0, 2);                        \
    _Pragma("unroll") for (int i = 0; i < 2 * NMT; ++i)                                        \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (LMOE_AS3 void*)((SA) + 1024 * i), 16,     \
                                               (int)ao[i], ko_, 0, 0);                         \
  }

  f32x4 acc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS byte offsets of this lane's fragments: row t*16 + r16 (weights) or
  // mt*16 + r16 (tokens), logical chunk 4u + kq of the stage.
  int fo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) fo[u] = r16 * 128 + (((4 * u + kq) ^ swz8(r16)) << 4);
  // (swz8 depends on the row's low 4 bits only, so rows 16 t + r16 share fo[u].)

#define LMOE_COMPUTE(SW, SA)                                                                    \
  _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                              \
    uint4 b[4], a[NMT];                                                                        \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                              \
      b[t] = *reinterpret_cast<const uint4*>((SW) + t * 2048 + fo[u]);                         \
    _Pragma("unroll") for (int mt = 0; mt < NMT; ++mt)                                         \
      a[mt] = *reinterpret_cast<const uint4*>((SA) + mt * 2048 + fo[u]);                       \
    _Pragma("unroll") for (int mt = 0; mt < NMT; ++mt)                                         \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) mfma16(a[mt], b[t], acc[mt][t]);           \
  }
  // One stage: the previous reads of the buffer about to be refilled are done
  // (all LDS reads complete), start the next stage's loads (at the end a
  // harmless repeat of the last stage into the buffer no later stage reads),
  // wait until only those are outstanding, then an LDS acquire fence keeps the
  // stage's reads below the wait, and multiply.
#define LMOE_STAGE(c, SW, SA, NW, NA)                                                           \
  {                                                                                            \
    __builtin_amdgcn_s_waitcnt(kLdsIdle);                                                      \
    LMOE_ISSUE(((c) + 1 < nc ? (c) + 1 : nc - 1), NW, NA)                                       \
    __builtin_amdgcn_s_waitcnt(vm_wait(8 + 2 * NMT));                                          \
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");                           \
    LMOE_COMPUTE(SW, SA)                                                                       \
  }
  const int nc = p.K / KC;                   // even (K % 128 == 0)
  // the buffers' previous reads (an earlier group's epilogue) are done
  __builtin_amdgcn_s_waitcnt(kLdsIdle);
  LMOE_ISSUE(0, sw0, sa0)
  for (int c = 0; c < nc; c += 2) {
    LMOE_STAGE(c, sw0, sa0, sw1, sa1)
    LMOE_STAGE(c + 1, sw1, sa1, sw0, sa0)
  }
#undef LMOE_STAGE
#undef LMOE_COMPUTE
#undef LMOE_ISSUE
  __builtin_amdgcn_s_waitcnt(0);             // the last (repeated) loads have landed; reads done

  // ---- epilogue: stage the [rows][cols] tile in LDS, store 16-byte chunks ----
  constexpr int OC = (EPI == EPI_SWIGLU) ? 32 : 64;   // output columns of the wave
  bf16_t* stile = reinterpret_cast<bf16_t*>(sw0);    // up to 64 x 64 bf16 = 8 KiB
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
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
  // the tile is staged (this wave's LDS writes complete) before it is read back
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");
  constexpr int CPR = OC / 8;                // 16-byte chunks per output row
  const int col0 = grp * OC;
  for (int c = lane; c < m_e * CPR; c += 64) {
    const int i = c / CPR, q = c % CPR;
    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)(lo + i) * p.ldo + col0 + q * 8) =
        *reinterpret_cast<const uint4*>(stile + i * OC + q * 8);
  }
}

template <int EPI>
__global__ __launch_bounds__(64) void stream_kernel(StreamParams p) {
  if (p.fused_n && *p.fused_n >= p.whole_min) return;   // the fused kernel ran these experts whole
  // Two consecutive row groups of one expert per workgroup (groups is even):
  // half the workgroups, so a launch with nothing to do costs half as much.
  const int pairs = p.groups >> 1;
  const int e = blockIdx.x / pairs, grp0 = 2 * (blockIdx.x % pairs);
  const int lo = p.offsets[e];
  const int m_e = p.offsets[e + 1] - lo;
  if (m_e == 0 || m_e > p.max_rows) return;
  for (int grp = grp0; grp < grp0 + 2; ++grp) {
    // Passes of up to 64 rows, each streaming the group's weights again (more
    // than one only when the host let experts above 64 rows come here:
    // batches too small for the tiled kernel to be worth a launch).
    for (int r0 = 0; r0 < m_e; r0 += MT * 16) {
      const int m = m_e - r0 < MT * 16 ? m_e - r0 : MT * 16;
      switch ((m + 15) >> 4) {               // token tiles in use (uniform)
        case 1: stream_body<EPI, 1>(p, e, grp, lo + r0, m, sw0, sw1, sa0, sa1); break;
        case 2: stream_body<EPI, 2>(p, e, grp, lo + r0, m, sw0, sw1, sa0, sa1); break;
        case 3: stream_body<EPI, 3>(p, e, grp, lo + r0, m, sw0, sw1, sa0, sa1); break;
        default: stream_body<EPI, 4>(p, e, grp, lo + r0, m, sw0, sw1, sa0, sa1); break;
      }
    }
  }
}

// Fused expert kernel for decode-sized batches: both expert GEMMs of every
// streamed expert (1..max_rows rows) in one launch, when there are at least
// whole_min of them (about as many as CUs, e.g. a decode batch; counted on the
// device). A persistent grid of one workgroup of FW waves per CU takes whole
// experts from a device-side queue (a ticket counter that the sort zeroes; the
// sort also lists the streamed experts). For each, the workgroup runs the
// weight-streaming gate/up GEMM with the SwiGLU epilogue over all of the
// expert's 2F weight rows (wave w takes the 64-row groups w, w + FW, ...),
// writes h to the expert's H rows, meets its other waves at a barrier (h
// complete and visible to them), then streams the down GEMM over all Dp output
// columns with the bf16 and sum-of-squares epilogue. With fewer streamed
// experts (giving each a single CU would leave most of the GPU idle) the
// kernel returns at once and the two single-wave launches that follow it do
// the work; they return at once when it ran.
// No workgroup ever waits for another: a workgroup only takes tickets and
// leaves once they run past the list, an expert's whole chain stays inside one
// workgroup, and every wave of a workgroup reaches its barriers equally often.
// One launch instead of two removes the second kernel's ramp and tail.
constexpr int FW = 4;                  // waves per workgroup (4 x 32 KiB of LDS)

// Each wave's own buffers, separate objects (as in the single-wave kernel) so
// that the compiler can tell them apart around the loads into LDS.
__shared__ __attribute__((aligned(16))) unsigned char fw00[8192], fw01[8192], fa00[8192], fa01[8192];
__shared__ __attribute__((aligned(16))) unsigned char fw10[8192], fw11[8192], fa10[8192], fa11[8192];
__shared__ __attribute__((aligned(16))) unsigned char fw20[8192], fw21[8192], fa20[8192], fa21[8192];
__shared__ __attribute__((aligned(16))) unsigned char fw30[8192], fw31[8192], fa30[8192], fa31[8192];

template <int EPI>
__device__ __forceinline__ void stream_groups(const StreamParams& p, int e, int lo, int m_e, int first,
                                              unsigned char* w0, unsigned char* w1, unsigned char* a0,
                                              unsigned char* a1) {
  for (int grp = first; grp < p.groups; grp += FW) {
    for (int r0 = 0; r0 < m_e; r0 += MT * 16) {     // passes of up to 64 rows, as above
      const int m = m_e - r0 < MT * 16 ? m_e - r0 : MT * 16;
      switch ((m + 15) >> 4) {               // token tiles in use (uniform)
        case 1: stream_body<EPI, 1>(p, e, grp, lo + r0, m, w0, w1, a0, a1); break;
        case 2: stream_body<EPI, 2>(p, e, grp, lo + r0, m, w0, w1, a0, a1); break;
        case 3: stream_body<EPI, 3>(p, e, grp, lo + r0, m, w0, w1, a0, a1); break;
        default: stream_body<EPI, 4>(p, e, grp, lo + r0, m, w0, w1, a0, a1); break;
      }
    }
  }
}

template <int EPI>
__device__ __forceinline__ void stream_groups_of_wave(const StreamParams& p, int e, int lo, int m_e, int wave) {
  switch (wave) {
    case 0: stream_groups<EPI>(p, e, lo, m_e, 0, fw00, fw01, fa00, fa01); break;
    case 1: stream_groups<EPI>(p, e, lo, m_e, 1, fw10, fw11, fa10, fa11); break;
    case 2: stream_groups<EPI>(p, e, lo, m_e, 2, fw20, fw21, fa20, fa21); break;
    default: stream_groups<EPI>(p, e, lo, m_e, 3, fw30, fw31, fa30, fa31); break;
  }
}

__global__ __launch_bounds__(FW * 64) void fused_stream_kernel(FusedStreamParams f) {
  __shared__ int ticket;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_items = *f.n_items;
  if (n_items < f.whole_min) return;         // the single-wave launches take these experts
  for (;;) {
    if (threadIdx.x == 0) ticket = atomicAdd(f.queue, 1);
    __syncthreads();
    const int item = ticket;
    __syncthreads();                         // every wave has read it before the next one is taken
    if (item >= n_items) break;              // uniform over the workgroup
    const int e = f.items[item];
    const int lo = f.gu.offsets[e], m_e = f.gu.offsets[e + 1] - lo;
    stream_groups_of_wave<EPI_SWIGLU>(f.gu, e, lo, m_e, wave);
    __syncthreads();                         // the expert's h rows are written and visible here
    stream_groups_of_wave<EPI_DOWN>(f.dn, e, lo, m_e, wave);
  }
}

// Dense projections of a small batch (router + pooler, unpooler at decode
// sizes). A workgroup of 4 waves takes 128 weight rows (32 per wave) over one
// K-slice and all T <= 128 tokens: both operands reach LDS through direct
// global-to-LDS loads in a four-stage pipeline of 64-wide K-steps; the token
// slice is loaded once per workgroup and shared by its waves, each weight byte
// is read once. Each workgroup writes its fp32 partial sums to
// part[slice][t][n] (n padded to whole groups); the reduction adds the slices
// in slice order (deterministic), then applies the bias and the output type:
// splitk_reduce here, or, for the router + pooler, the pooled-norm kernel that
// also normalizes each P row (launch_splitk_pool_norm).
constexpr int DW = 4;                  // waves per workgroup
constexpr int DR = 32;                 // weight rows per wave
constexpr int DS = 4;                  // pipeline stages
constexpr int DN = DW * DR;            // weight rows per workgroup
constexpr int MTD = 8;                 // token tiles of 16 (T <= 128)
constexpr int DSW = DW * DR * 128;     // weight bytes per stage
constexpr int DST = 128 * 128;         // token bytes per stage
constexpr int WJ = DR / 8, LPS = WJ + 4;
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past every extent

// One object per stage (weights, then tokens at DSW): the compiler tells the
// stages apart around the loads into LDS only while it tracks few enough
// objects; with a weight and a token object per stage it waited for the later
// stages' loads before reading the current one.
__shared__ __attribute__((aligned(16))) unsigned char ds0[DSW + DST], ds1[DSW + DST], ds2[DSW + DST],
    ds3[DSW + DST];

__global__ __launch_bounds__(DW * 64) void dense_stream_kernel(DenseStreamParams p) {
  const int grp = blockIdx.x / p.slices, sl = blockIdx.x % p.slices;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kq = lane >> 4, lrow = lane >> 3, lc = lane & 7;
  const int n_mt = (p.T + 15) >> 4;
  // stages of 64 K-columns: slice sl takes [c0, c1) of nct
  const int nct = p.K / KC;
  const int c0 = (int)((int64_t)nct * sl / p.slices), c1 = (int)((int64_t)nct * (sl + 1) / p.slices);
  const int nc = c1 - c0;

  // This wave's 32 weight rows lie in B0 or in B1 (n_split is a multiple of 64).
  const int nw = grp * DN + wave * DR;
  const bool in1 = nw >= p.n_split;
  const bf16_t* Bw = in1 ? static_cast<const bf16_t*>(p.B1) + (int64_t)(nw - p.n_split) * p.ldb
                         : static_cast<const bf16_t*>(p.B0) + (int64_t)nw * p.ldb;
  int valid = (in1 ? p.N : p.n_split) - nw;  // rows of this wave that exist
  valid = valid < 0 ? 0 : (valid > DR ? DR : valid);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(Bw), (short)0, valid * (int)p.ldb * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.A), (short)0, p.T * (int)p.lda * 2, kBufWord3);
  // Load j of a stage moves LDS rows 32*wave + 8j .. +7 of both operands
  // (lane: row + lrow, stored chunk position lc = logical chunk ^ swz8(row)).
  uint32_t wo[WJ], to[4];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int lr = 8 * j + lrow;
    const uint32_t ch = (uint32_t)((lc ^ swz8(lr)) << 4);
    wo[j] = lr < valid ? (uint32_t)lr * (uint32_t)(p.ldb * 2) + ch : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + 8 * j + lrow;
    const uint32_t ch = (uint32_t)((lc ^ swz8(r)) << 4);
    to[j] = r < p.T ? (uint32_t)r * (uint32_t)(p.lda * 2) + ch : kOutOfRange;
  }
  const int dbase = wave * DR * 128, tbase = wave * 32 * 128;
#define LMOE_DISSUE(c, SW, ST)                                                                   \
  {                                                                                             \
    const int ko_ = (c0 + (c)) * KC * 2;                                                        \
    _Pragma("unroll") for (int j = 0; j < WJ; ++j)                                              \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (LMOE_AS3 void*)((SW) + dbase + 1024 * j), 16, \
                                               (int)wo[j], ko_, 0, 2);                          \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                               \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (LMOE_AS3 void*)((ST) + tbase + 1024 * j), 16, \
                                               (int)to[j], ko_, 0, 0);                          \
  }
  constexpr int NTW = DR / 16;
  f32x4 acc[MTD][NTW];
#pragma unroll
  for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  int fo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) fo[u] = r16 * 128 + (((4 * u + kq) ^ swz8(r16)) << 4);
  const int wrow = wave * DR * 128;              // this wave's weight tiles in a stage
// All fragments of a K-half are read before its MFMAs (every token tile is in
// the stage, zero past T), so the reads are in flight together instead of
// one read, one wait, two MFMAs at a time.
#define LMOE_DCOMPUTE(SW, ST)                                                                    \
  _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                               \
    uint4 b[NTW], a[MTD];                                                                       \
    _Pragma("unroll") for (int t = 0; t < NTW; ++t)                                             \
      b[t] = *reinterpret_cast<const uint4*>((SW) + wrow + t * 2048 + fo[u]);                   \
    _Pragma("unroll") for (int mt = 0; mt < MTD; ++mt)                                          \
      a[mt] = *reinterpret_cast<const uint4*>((ST) + mt * 2048 + fo[u]);                        \
    _Pragma("unroll") for (int mt = 0; mt < MTD; ++mt)                                          \
      if (mt < n_mt) {                                                                          \
        _Pragma("unroll") for (int t = 0; t < NTW; ++t) mfma16(a[mt], b[t], acc[mt][t]);        \
      }                                                                                         \
  }
  // Stage c: this wave's loads of stage c have landed (at most the two later
  // stages' 16 loads outstanding) and its reads of stage c - 1 are done; after
  // the barrier every wave's part of stage c is in LDS and nobody reads the
  // buffer of stage c - 1 any more, which then takes stage c + 3.
#define LMOE_DSTAGE(c, SW, ST, NW, NT)                                                           \
  if ((c) < nc) {                                                                               \
    __builtin_amdgcn_s_waitcnt(vm_wait((DS - 2) * LPS) & ~(15 << 8));                            \
    __builtin_amdgcn_s_barrier();                                                               \
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");                            \
    LMOE_DISSUE(((c) + DS - 1 < nc ? (c) + DS - 1 : nc - 1), NW, NT)                             \
    LMOE_DCOMPUTE(SW, ST)                                                                       \
  }
  LMOE_DISSUE(0, ds0, ds0 + DSW)
  LMOE_DISSUE((1 < nc ? 1 : nc - 1), ds1, ds1 + DSW)
  LMOE_DISSUE((2 < nc ? 2 : nc - 1), ds2, ds2 + DSW)
  for (int c = 0; c < nc; c += 4) {
    LMOE_DSTAGE(c, ds0, ds0 + DSW, ds3, ds3 + DSW)
    LMOE_DSTAGE(c + 1, ds1, ds1 + DSW, ds0, ds0 + DSW)
    LMOE_DSTAGE(c + 2, ds2, ds2 + DSW, ds1, ds1 + DSW)
    LMOE_DSTAGE(c + 3, ds3, ds3 + DSW, ds2, ds2 + DSW)
  }
#undef LMOE_DSTAGE
#undef LMOE_DCOMPUTE
#undef LMOE_DISSUE
  __builtin_amdgcn_s_waitcnt(0);             // the last (repeated) loads have landed

  // partials: acc[mt][t][v] is token 16 mt + 4 kq + v, column nw + 16 t + r16
  const int np = p.slices > 0 ? ((p.N + DN - 1) / DN) * DN : 0;
  float* part = p.part + (int64_t)sl * p.T * np;
#pragma unroll
  for (int mt = 0; mt < MTD; ++mt) {
    if (mt >= n_mt) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = mt * 16 + 4 * kq + v;
      if (i < p.T) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) part[(int64_t)i * np + nw + t * 16 + r16] = acc[mt][t][v];
      }
    }
  }
}

// out = sum over slices of part[slice][t][n] (slice order), split like EPI_F32:
// columns [0, n_split) -> out0 (fp32, or bf16 if out0_bf16), [n_split, N) -> out1 + bias1.
// One thread per 4 consecutive columns of a token.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(DenseStreamParams p) {
  const int np = ((p.N + DN - 1) / DN) * DN;
  const int64_t total = (int64_t)p.T * np, q = total / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < q; i += (int64_t)gridDim.x * blockDim.x) {
    float4 s = *reinterpret_cast<const float4*>(p.part + 4 * i);
    for (int sl = 1; sl < p.slices; ++sl) {
      const float4 v = *reinterpret_cast<const float4*>(p.part + sl * total + 4 * i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const int t = (int)(4 * i / np), n0 = (int)(4 * i % np);
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = n0 + e;
      if (n >= p.N) break;
      if (n < p.n_split) {
        if (p.out0_bf16) static_cast<bf16_t*>(p.out0)[(int64_t)t * p.ldo0 + n] = f32_to_bf16(sv[e]);
        else static_cast<float*>(p.out0)[(int64_t)t * p.ldo0 + n] = sv[e];
      } else {
        const int c = n - p.n_split;
        static_cast<float*>(p.out1)[(int64_t)t * p.ldo1 + c] = sv[e] + (p.bias1 ? p.bias1[c] : 0.f);
      }
    }
  }
}

}  // namespace

int stream_max_rows() { return MT * 16; }
int dense_stream_max_tokens() { return MTD * 16; }

// Slices for an N x K projection: about one workgroup per CU (256), at least one
// 64-wide K-step per slice.
int dense_stream_slices(int N, int K) {
  const int groups = (N + DN - 1) / DN;
  int s = 256 / groups;
  if (s < 1) s = 1;
  if (s > K / KC) s = K / KC;
  return s;
}
int dense_stream_part_ld(int N) { return ((N + DN - 1) / DN) * DN; }
int64_t dense_stream_part_floats(int T, int N, int K) {
  return (int64_t)dense_stream_slices(N, K) * T * dense_stream_part_ld(N);
}

hipError_t launch_dense_stream_partials(const DenseStreamParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int groups = (p.N + DN - 1) / DN;
  hipLaunchKernelGGL(dense_stream_kernel, dim3(groups * p.slices), dim3(DW * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dense_stream(const DenseStreamParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  hipError_t err = launch_dense_stream_partials(p, s);
  if (err != hipSuccess) return err;
  const int64_t q = (int64_t)p.T * (((p.N + DN - 1) / DN) * DN) / 4;
  const int blocks = (int)((q + 255) / 256 < 2048 ? (q + 255) / 256 : 2048);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fused_stream(const FusedStreamParams& f, int n_cu, hipStream_t s) {
  if (f.gu.n_experts == 0 || n_cu <= 0) return hipSuccess;
  if (f.gu.groups % FW || f.dn.groups % FW) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fused_stream_kernel, dim3(n_cu), dim3(FW * 64), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_stream(const StreamParams& p, EpiKind epi, hipStream_t s) {
  const int blocks = p.n_experts * (p.groups >> 1);
  if (blocks == 0) return hipSuccess;
  if (p.groups & 1) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(stream_kernel<EPI_SWIGLU>, dim3(blocks), dim3(64), 0, s, p);
  else if (epi == EPI_DOWN)
    hipLaunchKernelGGL(stream_kernel<EPI_DOWN>, dim3(blocks), dim3(64), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lmoe
