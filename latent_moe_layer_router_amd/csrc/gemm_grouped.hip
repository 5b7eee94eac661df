// Tiled bf16 GEMMs of the prefill path. Grouped (M == 0): the expert GEMMs for
// experts with many rows, gate/up with the SwiGLU epilogue, down with the bf16
// output and per-64-column sums of squares. Dense (M > 0): the router + pooler
// (fp32 out, the router's columns from a second matrix plus a bias) and the
// unpooler (fp32 or bf16 out), M split evenly over ntiles_m row tiles of at
// most 320 rows (the caller picks the count that fills whole rounds of tiles).
//
// Row tiles of up to 320 rows x 256 weight rows, 512 threads = 8 wave64 in a
// 2 x 4 grid, each wave up to 160 x 64 = 5 x 2 MFMA 32x32x16 bf16 (160
// accumulator registers of the 256 each of two waves per SIMD gets). An expert's rows
// are split evenly over ceil(rows / 320) tiles and each tile's rows evenly
// between its two wave rows (in multiples of 32), so a 512-row expert runs two
// tiles of 256 (four 32-row groups per wave) and one of 513..640 rows still
// two tiles (of up to five groups). With 256-row tiles, near-uniform routing
// (512 +- 23 rows per expert) gave half the experts a third tile that loads
// the expert's whole weight slice once more; the loads bound this kernel.
// (A 4-wave layout of the same tile needs 320 accumulator registers per lane,
// more than the AGPR file, and the copies between AGPRs and VGPRs that follow
// made it 2.2x slower.)
//
// Operands reach LDS through direct global-to-LDS buffer loads in a four-stage
// pipeline of 32-wide K-steps (A 20 KiB + B 16 KiB per stage, 144 KiB): the
// loads for step k + 3 are in flight while step k computes. A stage is 20 A
// loads and 16 B loads of 16 rows x 64 bytes; wave w issues loads w, w + 8,
// ... (waves 0-3 five per stage, waves 4-7 four; A loads wholly past the
// tile's last row are skipped). The 16-byte chunks of a row are XOR-swizzled
// so that fragment reads are conflict-free.
//
// Tile order over the 8 XCDs: one index space (expert, n-tile, m-tile) cut
// into 8 contiguous chunks, one per XCD, so that the CUs of an XCD share the
// expert's weight slices and token rows in their L2.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

constexpr int GW = 8;                  // waves
constexpr int GNT = GW * 64;
constexpr int GBM = 320, GBN = 256;    // A rows (max), B rows per tile
constexpr int GMI = 5, GNI = 2;        // 32-row groups, 32-column groups per wave
constexpr int RB = 64;                 // bytes of each tile row per stage (32 bf16)
constexpr int GSA = GBM * RB, GSB = GBN * RB;
constexpr int LA = GBM / 16;            // A loads of 16 rows per stage
constexpr int kBufWord3 = 0x00020000;  // raw buffer descriptor, fourth word (CDNA)
constexpr uint32_t kOutOfRange = 0x80000000u;   // past every extent used here

#define LMOE_AS3 __attribute__((address_space(3)))

// Four pipeline stages, separate LDS objects so that the compiler can tell
// them apart when it orders reads against the loads still in flight.
__shared__ __attribute__((aligned(16))) unsigned char gA0[GSA], gB0[GSB], gA1[GSA], gB1[GSB],
    gA2[GSA], gB2[GSB], gA3[GSA], gB3[GSB];

// Byte offset of logical 16-byte chunk c (0..3) of tile row r (64-byte rows),
// stored at position c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3: 32 lanes on 32
// consecutive rows at one logical chunk hit distinct 16-byte bank slots.
__device__ __forceinline__ int swz(int r, int c) {
  return r * RB + ((c ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4);
}

__device__ __forceinline__ void mfma32(const uint4& a, const uint4& b, f32x16_t& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// At most N global loads of this wave in flight (its two later stages) and no
// LDS read outstanding: the scheduler may move the previous step's MFMAs (not
// their reads) past the barrier that follows.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Stage hand-off barrier (after the explicit wait; an LDS acquire fence keeps
// the stage's reads below it).
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int EPI>
__global__ __launch_bounds__(GNT, 1) void gemm_grouped_kernel(GroupedParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // ---- tile of this workgroup (XCD-chunked order) --------------------------
  // Grouped: tiles (expert, n-tile, m-tile) of the experts' sorted rows. Dense:
  // tiles (m-tile, n-tile) of an M x N product, M split evenly over ntiles_m.
  constexpr bool dense = (EPI == EPI_F32 || EPI == EPI_ACT);
  const int total = dense ? p.ntiles_m * p.ntiles_n : p.ntiles_n * p.mt_off[p.E];
  const int chunk = (total + 7) / 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int t = xcd * chunk + local;
  if (local >= chunk || t >= total) return;
  int e = 0, ntile, m0, m_end;
  if (dense) {
    ntile = t % p.ntiles_n;
    const int mi_t = t / p.ntiles_n;
    m0 = (int)((int64_t)p.M * mi_t / p.ntiles_m);
    m_end = (int)((int64_t)p.M * (mi_t + 1) / p.ntiles_m);
  } else {
    int lo = 0, hi = p.E;                    // expert e: ntiles_n*mt_off[e] <= t < ntiles_n*mt_off[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.ntiles_n * p.mt_off[mid] <= t) lo = mid; else hi = mid;
    }
    e = lo;
    // the expert's rows split evenly over its row tiles (each at most 320 rows)
    const int mt_e = p.mt_off[e + 1] - p.mt_off[e];
    const int tl = t - p.ntiles_n * p.mt_off[e];
    const int mi_t = tl % mt_e, cnt = p.offsets[e + 1] - p.offsets[e];
    ntile = tl / mt_e;
    m0 = p.offsets[e] + (int)((int64_t)cnt * mi_t / mt_e);
    m_end = p.offsets[e] + (int)((int64_t)cnt * (mi_t + 1) / mt_e);
  }
  const int n0 = ntile * (EPI == EPI_SWIGLU ? GBN / 2 : GBN);   // output column start
  // the tile's rows split between the wave rows: wm = 0 takes the first r_half
  // (a multiple of 32, at least half), wm = 1 the rest; at most 160 each
  const int tile_rows = m_end - m0;
  const int r_half = 32 * ((((tile_rows + 1) >> 1) + 31) >> 5);
  const int wrow0 = wm * r_half;
  const int mrows = wm == 0 ? min(r_half, tile_rows) : tile_rows - r_half;
  const int nmi = __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : (mrows >= 32 * GMI ? GMI : (mrows + 31) / 32));

  // ---- global-to-LDS loads --------------------------------------------------
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), (short)0, (int)p.a_bytes, kBufWord3);
  // B rows of the tile: grouped, the expert's matrix (rows n0 + r, or the
  // gate/up pairs); dense, the tile's own 256 rows from B (columns below
  // n_split) or B1, the extent ending at row N (rows past it read as zero).
  const bf16_t* Bt;
  int b_ext;
  if (dense) {
    Bt = (n0 < p.n_split) ? static_cast<const bf16_t*>(p.B) + (int64_t)n0 * p.ldb
                          : static_cast<const bf16_t*>(p.B1) + (int64_t)(n0 - p.n_split) * p.ldb;
    b_ext = min(GBN, p.N - n0) * (int)p.ldb * 2;
  } else {
    Bt = static_cast<const bf16_t*>(p.B) + (int64_t)e * p.b_expert_stride;
    b_ext = (int)p.b_bytes;
  }
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Bt), (short)0, b_ext, kBufWord3);
  const int pos = lane & 3;
  // Rows past the tile's end get an offset beyond every extent: the load reads
  // nothing from memory. Those rows are never stored.
  auto a_off = [&](int r) -> uint32_t {
    const int m = m0 + r;
    if (m >= m_end) return kOutOfRange;
    const uint32_t c = pos ^ (((r >> 1) ^ (r >> 3)) & 3);
    const int src = p.a_rows ? p.a_rows[m] : m;   // gathered rows (gate/up: the assignment's token)
    return (uint32_t)src * (uint32_t)(p.lda * 2) + c * 16;
  };
  auto b_off = [&](int r) -> uint32_t {
    const int n = dense ? r : (EPI == EPI_SWIGLU) ? ((r < GBN / 2) ? (n0 + r) : (p.F + n0 + r - GBN / 2)) : (n0 + r);
    const uint32_t c = pos ^ (((r >> 1) ^ (r >> 3)) & 3);
    return (uint32_t)n * (uint32_t)(p.ldb * 2) + c * 16;
  };
  // load j (of a stage) moves rows 16 j .. 16 j + 15, lane i row 16 j + i / 4
  // at chunk position i % 4; wave w issues j = w, w + 8, w + 16 (A, while j <
  // 20) and j = w, w + 8 (B)
  uint32_t ga[3], gb[2];
#pragma unroll
  for (int i = 0; i < 3; ++i) ga[i] = (wave + 8 * i < LA) ? a_off(16 * (wave + 8 * i) + (lane >> 2)) : kOutOfRange;
#pragma unroll
  for (int i = 0; i < 2; ++i) gb[i] = b_off(16 * (wave + 8 * i) + (lane >> 2));
  // Waves 0-3 issue a third A load (rows 256 + 16 wave ..) only if some of its
  // rows are in the tile: a 256-row tile then moves 32 rows per K-step instead
  // of 36 x 16. The LDS rows a skipped load would have filled are read only
  // for output rows past the tile's end, which are never stored.
  const bool three_a = wave + 16 < LA && 16 * (wave + 16) < tile_rows;

#define LMOE_LD(RS, OFF, DST, KO) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds((RS), (LMOE_AS3 void*)(DST), 16, (int)(OFF), (KO), 0, 0);
#define LMOE_ISSUE(kt, SA, SBB)                                                                         \
  {                                                                                                    \
    const int kr_ = (kt) + krot;                                                                       \
    const int ko = (kr_ >= nk ? kr_ - nk : kr_) * RB;                                                  \
    LMOE_LD(rsA, ga[0], (SA) + wave * 16 * RB, ko)                                                     \
    LMOE_LD(rsA, ga[1], (SA) + (wave + 8) * 16 * RB, ko)                                               \
    if (three_a) LMOE_LD(rsA, ga[2], (SA) + (wave + 16) * 16 * RB, ko)                                 \
    LMOE_LD(rsB, gb[0], (SBB) + wave * 16 * RB, ko)                                                    \
    LMOE_LD(rsB, gb[1], (SBB) + (wave + 8) * 16 * RB, ko)                                              \
  }
  // two later stages of 5 (waves 0-3) or 4 loads
#define LMOE_WAIT()                    \
  if (three_a) wait_vm<10>();          \
  else wait_vm<8>();

  f32x16_t acc[GMI][GNI];
#pragma unroll
  for (int mi = 0; mi < GMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < GNI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  // LDS rows of this lane's MFMA operands: A rows wrow0 + 32 mi + l32 (the
  // swizzle depends on a row's low 5 bits only); B rows: SwiGLU the gate (ni =
  // 0) and up (ni = 1) rows of the same 32 output columns, down 64 columns.
  const int l32 = lane & 31, half = lane >> 5;
  const int aoff0 = swz(wrow0 + l32, half), aoff1 = swz(wrow0 + l32, 2 + half);
  auto brow_of = [&](int ni) {
    return (EPI == EPI_SWIGLU) ? (ni * (GBN / 2) + wn * 32 + l32) : (wn * 64 + ni * 32 + l32);
  };
  const int b00 = swz(brow_of(0), half), b01 = swz(brow_of(0), 2 + half);
  const int b10 = swz(brow_of(1), half), b11 = swz(brow_of(1), 2 + half);

  // Operand fragments: two register sets, so that the LDS reads of the next
  // 16-wide K-slice are in flight while the MFMAs of the current one run.
  uint4 xa0, xa1, xa2, xa3, xa4, xb0, xb1;
  uint4 ya0, ya1, ya2, ya3, ya4, yb0, yb1;

#define LMOE_READ(NMI, SA, SBB, AO, B0, B1, PA, PB)                                               \
  if ((NMI) > 0) {                                                                              \
    PB##0 = *reinterpret_cast<const uint4*>((SBB) + (B0));                                      \
    PB##1 = *reinterpret_cast<const uint4*>((SBB) + (B1));                                      \
    PA##0 = *reinterpret_cast<const uint4*>((SA) + (AO));                                       \
  }                                                                                             \
  if ((NMI) > 1) PA##1 = *reinterpret_cast<const uint4*>((SA) + (AO) + 32 * RB);                \
  if ((NMI) > 2) PA##2 = *reinterpret_cast<const uint4*>((SA) + (AO) + 64 * RB);                \
  if ((NMI) > 3) PA##3 = *reinterpret_cast<const uint4*>((SA) + (AO) + 96 * RB);                \
  if ((NMI) > 4) PA##4 = *reinterpret_cast<const uint4*>((SA) + (AO) + 128 * RB);
#define LMOE_MFMA(NMI, PA, PB)                                                                   \
  if ((NMI) > 0) { mfma32(PA##0, PB##0, acc[0][0]); mfma32(PA##0, PB##1, acc[0][1]); }          \
  if ((NMI) > 1) { mfma32(PA##1, PB##0, acc[1][0]); mfma32(PA##1, PB##1, acc[1][1]); }          \
  if ((NMI) > 2) { mfma32(PA##2, PB##0, acc[2][0]); mfma32(PA##2, PB##1, acc[2][1]); }          \
  if ((NMI) > 3) { mfma32(PA##3, PB##0, acc[3][0]); mfma32(PA##3, PB##1, acc[3][1]); }          \
  if ((NMI) > 4) { mfma32(PA##4, PB##0, acc[4][0]); mfma32(PA##4, PB##1, acc[4][1]); }
  // K-step k (stage k in SA/SBB, stage k + 1 in NA/NB). On entry stage k is
  // visible to all waves, the loads of stages k + 1 .. k + 3 are in flight and
  // the x registers hold the step's first K-slice. The step reads the second
  // slice (y) and runs the first slice's MFMAs (x); waits for stage k + 1 and
  // its own LDS reads, then the barrier: no wave reads stage k any more, so the
  // loads of stage k + 4 go into its buffer (clamped to the last stage: a
  // harmless re-read into a buffer no later step reads); reads the next step's
  // first slice (x) and runs the second slice's MFMAs (y).
#define LMOE_STEP(NMI, k, SA, SBB, NA, NB)                                                       \
  {                                                                                             \
    LMOE_READ(NMI, SA, SBB, aoff1, b01, b11, ya, yb)                                            \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, xa, xb)                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_WAIT()                                                                                 \
    bar();                                                                                      \
    LMOE_ISSUE(((k) + 4 < nk ? (k) + 4 : nk - 1), SA, SBB)                                      \
    LMOE_READ(NMI, NA, NB, aoff0, b00, b10, xa, xb)                                             \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, ya, yb)                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
#define LMOE_KLOOP(NMI)                                                                          \
  {                                                                                             \
    LMOE_READ(NMI, gA0, gB0, aoff0, b00, b10, xa, xb)                                           \
    for (int k = 0; k < nk; k += 4) {                                                           \
      LMOE_STEP(NMI, k, gA0, gB0, gA1, gB1)                                                     \
      LMOE_STEP(NMI, k + 1, gA1, gB1, gA2, gB2)                                                 \
      LMOE_STEP(NMI, k + 2, gA2, gB2, gA3, gB3)                                                 \
      LMOE_STEP(NMI, k + 3, gA3, gB3, gA0, gB0)                                                 \
    }                                                                                           \
  }

  const int nk = p.K / 32;                   // a multiple of 4 (K % 128 == 0)
  // Each column tile walks K from its own starting step (4 steps further per
  // column tile), so that the tiles sharing a row tile's token slice request it
  // a few steps apart. The order depends on the column tile only, so every
  // output element is summed in one fixed order, whatever the batch.
  const int krot = (ntile * 4) % nk;
  LMOE_ISSUE(0, gA0, gB0)
  LMOE_ISSUE(1, gA1, gB1)
  LMOE_ISSUE(2, gA2, gB2)
  LMOE_WAIT()
  bar();
  LMOE_ISSUE(3, gA3, gB3)
  // One K loop per number of live 32-row groups (uniform per wave; all waves
  // run the same barriers): 5, 4 (3 groups run it too), 2 (1-2 groups), none.
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
#undef LMOE_STEP
#undef LMOE_MFMA
#undef LMOE_READ
#undef LMOE_WAIT
#undef LMOE_ISSUE
#undef LMOE_LD
  __syncthreads();   // every load has landed and every wave has finished reading

  if (EPI == EPI_F32) {
    // fp32 out, straight from the accumulators: the 32 lanes of a half-wave
    // store 32 consecutive columns of a row (128 bytes). Columns below n_split
    // go to out, the rest to out1 plus bias1 (router logits).
#pragma unroll
    for (int mi = 0; mi < GMI; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = mi * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (r >= mrows) continue;
        const int m = m0 + wrow0 + r;
#pragma unroll
        for (int ni = 0; ni < GNI; ++ni) {
          const int n = n0 + wn * 64 + ni * 32 + l32;
          if (n >= p.N) continue;
          if (n < p.n_split)
            static_cast<float*>(p.out)[(int64_t)m * p.ldo + n] = acc[mi][ni][v];
          else
            p.out1[(int64_t)m * p.ldo1 + (n - p.n_split)] =
                acc[mi][ni][v] + (p.bias1 ? p.bias1[n - p.n_split] : 0.f);
        }
      }
    return;
  }

  // ---- epilogue, by wave row: stage [160][OBN] bf16 in LDS, 16-byte stores ---
  // Rows [32 q, 32 q + 32) of the staged half live in buffer q (gA0, gB0, gA1,
  // gB1, gA2: at least 16 KiB each, 32 rows of up to 512 bytes).
  constexpr int OBN = (EPI == EPI_SWIGLU) ? GBN / 2 : GBN;
  auto srow = [&](int r) -> bf16_t* {
    unsigned char* b;
    switch (r >> 5) {
      case 0: b = gA0; break;
      case 1: b = gB0; break;
      case 2: b = gA1; break;
      case 3: b = gB1; break;
      default: b = gA2; break;
    }
    return reinterpret_cast<bf16_t*>(b) + (r & 31) * OBN;
  };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int mi = 0; mi < GMI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = mi * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          bf16_t* row = srow(r);
          if (EPI == EPI_SWIGLU) {
            const float g = acc[mi][0][v], u = acc[mi][1][v];
            row[wn * 32 + l32] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
          } else {
#pragma unroll
            for (int ni = 0; ni < GNI; ++ni) row[wn * 64 + ni * 32 + l32] = f32_to_bf16(acc[mi][ni][v]);
          }
        }
    }
    __syncthreads();
    // rows of this half: tile rows [h r_half, h r_half + hrows)
    const int hrows = h == 0 ? min(r_half, tile_rows) : tile_rows - r_half;
    const int mh = m0 + h * r_half;
    constexpr int CPR = OBN / 8;
    for (int i = tid; i < hrows * CPR; i += GNT) {
      const int r = i / CPR, c = (i % CPR) * 8;
      if (dense && n0 + c >= p.N) continue;
      *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)(mh + r) * p.ldo + n0 + c) =
          *reinterpret_cast<const uint4*>(srow(r) + c);
    }
    if (EPI == EPI_DOWN) {
      // sums of squares of the stored bf16 values, per row and 64-column group
      for (int i = tid; i < hrows * (GBN / 64); i += GNT) {
        const int r = i / (GBN / 64), grp = i % (GBN / 64);
        const bf16_t* row = srow(r) + grp * 64;
        float ssq = 0.f;
        for (int j = 0; j < 64; ++j) {
          const float y = bf16_to_f32(row[j]);
          ssq += y * y;
        }
        p.ss_out[(int64_t)(mh + r) * p.ss_ld + (n0 + grp * 64) / 64] = ssq;
      }
    }
    __syncthreads();   // the half is read out before the next one is staged
  }
}

}  // namespace

int gemm_grouped_tile_m() { return GBM; }

// One tile per CU at a time (144 KiB of LDS). Measured at 16K rows, a tile's
// time goes as (g + 1.5), g the 32-row groups of its larger wave row (4 for
// 256 rows, 5 for 257..320): so choose the row-tile count (tiles of 128 to 320
// rows) that minimizes ceil(tiles / n_cu) * (2 g + 3), and among equal costs
// the smallest tiles. At M = 16384 and 17 column tiles (router + pooler) that
// is 60 row tiles of about 273 rows, 4 full rounds (1.145 ms against 1.21 ms
// for 64 tiles of 256 rows, 5 rounds); at 32 column tiles (unpooler) 64 tiles
// of 256 rows stay best (56 tiles of 293 rows measured 2% slower).
int gemm_grouped_dense_row_tiles(int M, int ntiles_n, int n_cu) {
  if (M <= 0 || ntiles_n <= 0 || n_cu <= 0) return 1;
  const int lo = (M + GBM - 1) / GBM;
  const int hi = lo > (M + 127) / 128 ? lo : (M + 127) / 128;
  int best = lo;
  int64_t best_cost = -1, best_rows = 0;
  for (int ntm = lo; ntm <= hi; ++ntm) {
    const int64_t rows = (M + ntm - 1) / ntm;
    const int64_t g = ((rows + 1) / 2 + 31) / 32;
    const int64_t rounds = ((int64_t)ntm * ntiles_n + n_cu - 1) / n_cu;
    const int64_t cost = rounds * (2 * g + 3);
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && rows < best_rows)) {
      best = ntm;
      best_cost = cost;
      best_rows = rows;
    }
  }
  return best;
}

hipError_t launch_gemm_grouped(const GroupedParams& p, EpiKind epi, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (p.K % 128 != 0) return hipErrorInvalidValue;
  const bool dense = epi == EPI_F32 || epi == EPI_ACT;
  if (dense != (p.M > 0) || (dense && p.n_split < p.N && p.n_split % GBN != 0)) return hipErrorInvalidValue;
  if (dense && (p.ntiles_m < 1 || (int64_t)p.ntiles_m * GBM < p.M || p.ntiles_m * p.ntiles_n > p.max_tiles))
    return hipErrorInvalidValue;
  const int grid = ((p.max_tiles + 7) / 8) * 8;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm_grouped_kernel<EPI_SWIGLU>, dim3(grid), dim3(GNT), 0, s, p);
  else if (epi == EPI_DOWN)
    hipLaunchKernelGGL(gemm_grouped_kernel<EPI_DOWN>, dim3(grid), dim3(GNT), 0, s, p);
  else if (epi == EPI_F32)
    hipLaunchKernelGGL(gemm_grouped_kernel<EPI_F32>, dim3(grid), dim3(GNT), 0, s, p);
  else
    hipLaunchKernelGGL(gemm_grouped_kernel<EPI_ACT>, dim3(grid), dim3(GNT), 0, s, p);
  return hipGetLastError();
}

}  // namespace lmoe
