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
// are split over ceil(rows / 320) tiles in whole units of 64 rows and each
// tile's rows evenly between its two wave rows (in multiples of 32), so a
// 512-row expert runs two tiles of 256 (four 32-row groups per wave) and one of
// 513..640 rows two tiles of 320 and the rest (five and at most four groups). With 256-row tiles, near-uniform routing
// (512 +- 23 rows per expert) gave half the experts a third tile that loads
// the expert's whole weight slice once more; the loads bound this kernel.
// (A 4-wave layout of the same tile needs 320 accumulator registers per lane,
// more than the AGPR file, and the copies between AGPRs and VGPRs that follow
// made it 2.2x slower.)
//
// Operands reach LDS through direct global-to-LDS buffer loads. The token
// rows (A) move in 32-wide K-steps, 64 bytes of each row, through three
// buffers (20 KiB each): the loads for step k + 3 are issued at step k. The
// weights (B) move in stages of two K-steps, whole 128-byte row segments, 8
// rows per load, through three buffers (32 KiB each): the loads for steps
// 2s + 6 and 2s + 7 are issued at step 2s + 1, once both halves of a buffer
// are read (156 KiB in all). The weights come from HBM on their first touch,
// the token rows mostly from L2: the weights run further ahead, and whole-line
// loads halve their requests for the same bytes. A stage of A is 20 loads of
// 16 rows x 64 bytes (wave w issues loads w, w + 8, w + 16; waves 4-7's third
// has no rows, and rows past the tile's last row read nothing); a stage of B is
// 32 loads of 8 rows x 128 bytes, four per wave. The 16-byte chunks of each
// row are XOR-swizzled so that fragment reads are conflict-free. Between two
// barriers each wave's loads and LDS reads are interleaved one by one with its
// MFMAs.
//
// Tile order over the 8 XCDs: one index space (expert, n-tile, m-tile) cut
// into 8 contiguous chunks, one per XCD, so that the CUs of an XCD share the
// expert's weight slices and token rows in their L2. The workgroups are
// persistent (one per CU, each walking its XCD's chunk at a stride of the
// XCD's workgroup count), and a tile's first loads are issued before the
// previous tile's epilogue.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

constexpr int GW = 8;                  // waves
constexpr int GNT = GW * 64;
constexpr int GBM = 320, GBN = 256;    // A rows (max), B rows per tile
constexpr int GMI = 5, GNI = 2;        // 32-row groups, 32-column groups per wave
constexpr int RB = 64;                 // bytes of each A row per stage (32 bf16)
constexpr int RBB = 128;               // bytes of each B row per stage (two K-steps)
constexpr int GSA = GBM * RB, GSB = GBN * RBB;
constexpr int LA = GBM / 16;            // A loads of 16 rows per stage
constexpr int kBufWord3 = 0x00020000;  // raw buffer descriptor, fourth word (CDNA)
constexpr uint32_t kOutOfRange = 0x80000000u;   // past every extent used here

#define LMOE_AS3 __attribute__((address_space(3)))

// Three A buffers and three B buffers, separate LDS objects so that the
// compiler can tell them apart when it orders reads against the loads still in
// flight.
__shared__ __attribute__((aligned(16))) unsigned char gA0[GSA], gB0[GSB], gA1[GSA], gB1[GSB],
    gA2[GSA], gB2[GSB];
// Target of the third A load of waves 4-7, which has no rows to move (1 KiB
// per wave; the 160 KiB of LDS in all): every wave then issues the same loads,
// and the K loop has no branch to split its instruction scheduling.
__shared__ __attribute__((aligned(16))) unsigned char gAx[4 * 1024];

// Byte offset of logical 16-byte chunk c (0..3) of tile row r (64-byte rows),
// stored at position c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3: 32 lanes on 32
// consecutive rows at one logical chunk hit distinct 16-byte bank slots.
__device__ __forceinline__ int swz(int r, int c) {
  return r * RB + ((c ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4);
}

// Byte offset of logical 16-byte chunk c (0..7) of B row r (128-byte rows),
// stored at position c ^ g(r), g(r) = ((r >> 1) ^ (r << 2)) & 7: the chunk
// positions of any 8 consecutive rows are a permutation of 0..7, so 32 lanes
// reading 32 consecutive rows at one logical chunk are conflict-free.
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ (r << 2)) & 7; }
__device__ __forceinline__ int swzb(int r, int c) { return r * RBB + ((c ^ swz8(r)) << 4); }

__device__ __forceinline__ void mfma32(const uint4& a, const uint4& b, f32x16_t& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// Two fp32 values rounded to bf16 by the packed hardware conversion (to
// nearest, ties to even, as f32_to_bf16 rounds every finite value; a NaN stays
// a NaN), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, b16x2_t));
}

// silu(g) * u with the hardware exponential and reciprocal (a few ulp of fp32,
// far below the bf16 rounding that follows).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// At most N global loads of this wave in flight (those issued after the last
// one the next step needs) and no LDS read outstanding: the scheduler may move
// the previous step's MFMAs (not their reads) past the barrier that follows.
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

// Stage hand-off barrier of the epilogue's LDS staging: the LDS writes (or
// reads) before it are complete. The release fence also covers this wave's
// global-to-LDS loads (their LDS writes count), so the next tile's first loads
// have landed by the first staging barrier; they land during the staging
// anyway (a barrier without that wait measured the same).
__device__ __forceinline__ void lds_bar() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Tile t: its expert (grouped), column tile and rows [m0, m_end).
struct TileGeo {
  int e, ntile, m0, m_end;
};

template <bool kDense>
__device__ __forceinline__ TileGeo tile_geo(const GroupedParams& p, int t) {
  TileGeo g;
  g.e = 0;
  if (kDense) {
    // tiles (m-tile, n-tile) of an M x N product, M split evenly over ntiles_m
    g.ntile = t % p.ntiles_n;
    const int mi_t = t / p.ntiles_n;
    g.m0 = (int)((int64_t)p.M * mi_t / p.ntiles_m);
    g.m_end = (int)((int64_t)p.M * (mi_t + 1) / p.ntiles_m);
  } else {
    // tiles (expert, n-tile, m-tile) of the experts' sorted rows: expert e has
    // ntiles_n * mt_off[e] <= t < ntiles_n * mt_off[e + 1]
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.ntiles_n * p.mt_off[mid] <= t) lo = mid; else hi = mid;
    }
    g.e = lo;
    // the expert's rows split over its row tiles in whole units of 64 rows
    // (each tile at most 320 rows): a tile's time goes with the 32-row groups
    // of its larger wave row, ceil(rows / 64), so 530 rows run as 320 + 210
    // (5 + 4 groups) rather than 265 + 265 (5 + 5)
    const int mt_e = p.mt_off[lo + 1] - p.mt_off[lo];
    const int tl = t - p.ntiles_n * p.mt_off[lo];
    const int mi_t = tl % mt_e, cnt = p.offsets[lo + 1] - p.offsets[lo];
    const int G = (cnt + 63) >> 6;
    const int g0 = (int)((int64_t)G * mi_t / mt_e), g1 = (int)((int64_t)G * (mi_t + 1) / mt_e);
    g.ntile = tl / mt_e;
    g.m0 = p.offsets[lo] + min(cnt, 64 * g0);
    g.m_end = p.offsets[lo] + min(cnt, 64 * g1);
  }
  return g;
}

// Persistent: each workgroup (one per CU) walks tiles of its XCD's chunk of
// the tile order, a fixed stride apart. A tile's first B stage and A step are
// issued before the previous tile's epilogue, which stages its output through
// the other buffers, so their latency hides behind it.
template <int EPI>
__global__ __launch_bounds__(GNT, 1) void gemm_grouped_kernel(GroupedParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // ---- tiles of this workgroup (XCD-chunked order) -------------------------
  constexpr bool dense = (EPI == EPI_F32 || EPI == EPI_ACT);
  const int total = dense ? p.ntiles_m * p.ntiles_n : p.ntiles_n * p.mt_off[p.E];
  const int chunk = (total + 7) / 8;
  const int xcd = blockIdx.x % 8, stride = gridDim.x / 8;
  int local = blockIdx.x / 8;
  if (local >= chunk || xcd * chunk + local >= total) return;
  TileGeo geo = tile_geo<dense>(p, xcd * chunk + local);

  const int nk = p.K / 32;                   // a multiple of 4 (K % 128 == 0)
  const int rowb = (int)p.ldb * 2;
  // The wave's four B loads (rows r, r + 64, r + 128, r + 192; the swizzle
  // depends on the row's low 4 bits only) differ by whole rows: one offset
  // register plus uniform row deltas in the scalar offset. SwiGLU rows 128..255
  // are the up rows, F - 128 further on.
  // In the packed expert layout (grouped mode only) rows come in groups of 64
  // whose stage of two K-steps is one 8 KiB block: the row deltas are whole
  // groups of K / 64 blocks, and a stage is 8 KiB further.
  const bool bpk = !dense && p.b_packed;
  const int rowu = bpk ? (p.K >> 6) * 8192 / 64 : rowb;   // bytes per row in whole-group deltas
  const int up = (EPI == EPI_SWIGLU && !dense) ? (p.F - GBN / 2) * rowu : 0;
  const int gbd1 = 64 * rowu, gbd2 = 128 * rowu + up, gbd3 = 192 * rowu + up;
  const int kstep_b = bpk ? 4096 : RB;       // bytes per K-step of B (a stage is two)

  // ---- global-to-LDS loads of a tile ----------------------------------------
  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t ga[3], gb0;
  int krot;
  auto setup_loads = [&](const TileGeo& g) {
    // the lane index, opaque: the offsets below are computed here for each
    // tile, not hoisted out of the tile loop and kept live across it
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int n0 = g.ntile * (EPI == EPI_SWIGLU ? GBN / 2 : GBN);
    rsA = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), (short)0, (int)p.a_bytes, kBufWord3);
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
      Bt = static_cast<const bf16_t*>(p.B) + (int64_t)g.e * p.b_expert_stride;
      b_ext = (int)p.b_bytes;
    }
    rsB = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Bt), (short)0, b_ext, kBufWord3);
    // A load j (of a stage) moves rows 16 j .. 16 j + 15, lane i row 16 j + i / 4
    // at chunk position i % 4; wave w issues j = w, w + 8, w + 16 (j < 20; the
    // third load of waves 4-7 has no rows and goes to gAx). Rows past the
    // tile's end get an offset beyond every extent: the load reads nothing from
    // memory. Those rows are never stored.
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int r = 16 * (wave + 8 * i) + (ln >> 2);
      const int m = g.m0 + r;
      uint32_t o = kOutOfRange;
      if (wave + 8 * i < LA && m < g.m_end) {
        const uint32_t c = (ln & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
        const int src = p.a_rows ? p.a_rows[m] : m;   // gathered rows (gate/up: the assignment's token)
        o = (uint32_t)src * (uint32_t)(p.lda * 2) + c * 16;
      }
      ga[i] = o;
    }
    // B load j (of a stage) moves rows 8 j .. 8 j + 7, lane i row 8 j + i / 8 at
    // chunk position i % 8 (which holds logical chunk (i % 8) ^ g(row)); wave w
    // issues j = w, w + 8, w + 16, w + 24.
    {
      const int r = 8 * wave + (ln >> 3);
      const int n = dense ? r : n0 + r;
      gb0 = (bpk ? (uint32_t)(n >> 6) * (uint32_t)(p.K >> 6) * 8192u + (uint32_t)(n & 63) * 128u
                 : (uint32_t)n * (uint32_t)rowb) +
            (uint32_t)(((ln & 7) ^ swz8(r)) << 4);
    }
    // Dense products: each column tile walks K from its own starting step (4
    // steps further per column tile), so that the tiles sharing a row tile's
    // rows request them a few steps apart (the unpooler ran 2% faster so).
    // Expert tiles start at step 0: the concurrent tiles of an expert then
    // request its token rows in step, which L2 serves once (with the
    // rotation they read 24.1 GB per gate/up launch at the prefill shape,
    // without it 19.3 GB, and ran 1.5% slower). The order depends on the
    // column tile only, so every output element is summed in one fixed
    // order, whatever the batch.
    krot = dense ? (g.ntile * 4) % nk : 0;
  };

#define LMOE_LD(RS, OFF, DST, KO) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds((RS), (LMOE_AS3 void*)(DST), 16, (int)(OFF), (KO), 0, 0);
  // A for K-step kt (rotated), into buffer SA
#define LMOE_ISSUE_A(kt, SA)                                                                            \
  {                                                                                                    \
    const int kr_ = (kt) + krot;                                                                       \
    const int ko = (kr_ >= nk ? kr_ - nk : kr_) * RB;                                                  \
    LMOE_LD(rsA, ga[0], (SA) + wave * 16 * RB, ko)                                                     \
    LMOE_LD(rsA, ga[1], (SA) + (wave + 8) * 16 * RB, ko)                                               \
    LMOE_LD(rsA, ga[2], (wave < 4) ? (SA) + (wave + 16) * 16 * RB : gAx + (wave - 4) * 1024, ko)      \
  }
  // B for K-steps 2 st and 2 st + 1 (rotated; krot is even, so the pair never
  // wraps), into buffer SBB
#define LMOE_ISSUE_B(st, SBB)                                                                           \
  {                                                                                                    \
    const int kr_ = 2 * (st) + krot;                                                                   \
    const int ko = (kr_ >= nk ? kr_ - nk : kr_) * kstep_b;                                             \
    LMOE_LD(rsB, gb0, (SBB) + wave * 8 * RBB, ko)                                                      \
    LMOE_LD(rsB, gb0, (SBB) + (wave + 8) * 8 * RBB, ko + gbd1)                                         \
    LMOE_LD(rsB, gb0, (SBB) + (wave + 16) * 8 * RBB, ko + gbd2)                                        \
    LMOE_LD(rsB, gb0, (SBB) + (wave + 24) * 8 * RBB, ko + gbd3)                                        \
  }
  // Waits for the next step's operands. Loads are issued in blocks, one per
  // step k: the B stage (odd k only) and then A for step k + 3. Counters drain
  // in issue order, so a wait lets through the blocks issued after the last
  // load it needs, which is always A for step k + 1 (block k - 2; the B stage
  // holding step k + 1 came earlier): block k - 1, that is one A block, plus
  // one B stage when k - 1 is odd. A blocks are 3 loads, B stages 4.
#define LMOE_WAIT_EVEN() wait_vm<7>();
#define LMOE_WAIT_ODD() wait_vm<3>();

  // LDS rows of this lane's MFMA operands: A rows wrow0 + 32 mi + l32 (the
  // swizzle depends on a row's low 5 bits only); B rows: SwiGLU the gate (ni =
  // 0) and up (ni = 1) rows of the same 32 output columns, down 64 columns.
  // The second B fragment's row is the first's plus 128 (SwiGLU) or 32 (down)
  // rows, a multiple of 8 that leaves the swizzle alone: a constant byte
  // offset. One offset register per operand (ao for A, bo0 for B) walks the
  // logical chunks in place: the second 16-wide K-slice
  // of a step is the first's chunk with bit 1 set (byte offset XOR 32), a B
  // row's odd K-step its even one's with bit 2 set (XOR 64). The XORs are
  // opaque to the compiler, which otherwise keeps every variant (and their
  // sums with the buffers' LDS addresses) in registers and spills inside the
  // K loop.
  constexpr int kB1Off = ((EPI == EPI_SWIGLU) ? GBN / 2 : 32) * RBB;
#define LMOE_XOR(X, IMM) __asm__ volatile("v_xor_b32 %0, " #IMM ", %0" : "+v"(X))

  // Operand fragments: two register sets, so that the LDS reads of the next
  // 16-wide K-slice are in flight while the MFMAs of the current one run.
  uint4 xa0, xa1, xa2, xa3, xa4, xb0, xb1;
  uint4 ya0, ya1, ya2, ya3, ya4, yb0, yb1;
  f32x16_t acc[GMI][GNI];

#define LMOE_READ(NMI, SA, SBB, AO, B0, PA, PB)                                                   \
  if ((NMI) > 0) {                                                                              \
    PB##0 = *reinterpret_cast<const uint4*>((SBB) + (B0));                                      \
    PB##1 = *reinterpret_cast<const uint4*>((SBB) + (B0) + kB1Off);                             \
    PA##0 = *reinterpret_cast<const uint4*>((SA) + (AO));                                       \
  }                                                                                             \
  if ((NMI) > 1) PA##1 = *reinterpret_cast<const uint4*>((SA) + (AO) + 32 * RB);                \
  if ((NMI) > 2) PA##2 = *reinterpret_cast<const uint4*>((SA) + (AO) + 64 * RB);                \
  if ((NMI) > 3) PA##3 = *reinterpret_cast<const uint4*>((SA) + (AO) + 96 * RB);                \
  if ((NMI) > 4) PA##4 = *reinterpret_cast<const uint4*>((SA) + (AO) + 128 * RB);
  // MFMAs of 32-row groups LO..HI-1 (of the NMI live ones)
#define LMOE_MFMA(NMI, PA, PB, LO, HI)                                                                            \
  if ((NMI) > 0 && 0 >= (LO) && 0 < (HI)) { mfma32(PA##0, PB##0, acc[0][0]); mfma32(PA##0, PB##1, acc[0][1]); } \
  if ((NMI) > 1 && 1 >= (LO) && 1 < (HI)) { mfma32(PA##1, PB##0, acc[1][0]); mfma32(PA##1, PB##1, acc[1][1]); } \
  if ((NMI) > 2 && 2 >= (LO) && 2 < (HI)) { mfma32(PA##2, PB##0, acc[2][0]); mfma32(PA##2, PB##1, acc[2][1]); } \
  if ((NMI) > 3 && 3 >= (LO) && 3 < (HI)) { mfma32(PA##3, PB##0, acc[3][0]); mfma32(PA##3, PB##1, acc[3][1]); } \
  if ((NMI) > 4 && 4 >= (LO) && 4 < (HI)) { mfma32(PA##4, PB##0, acc[4][0]); mfma32(PA##4, PB##1, acc[4][1]); }
  // Scheduling of a stretch between two barriers: NM MFMAs, each followed by
  // up to one global-to-LDS load (the first NV) and one LDS read (the first
  // ND), so that a wave issues its loads and reads while its matrix core works
  // instead of in a burst that leaves it idle (both waves of a SIMD reach the
  // same barrier, so the other wave cannot fill the gap).
#define LMOE_INTERLEAVE(NM, NV, ND)                                                              \
  {                                                                                             \
    _Pragma("unroll") for (int q_ = 0; q_ < (NM); ++q_) {                                        \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
      if (q_ < (NV)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                          \
      if (q_ < (ND)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          \
    }                                                                                           \
  }
  // K-step k: A of step k in SA, of step k + 1 in NA; B of step k in SBB at
  // parity PK (0: first K-step of the B stage, 1: second), of step k + 1 in
  // NBB. On entry A and B of step k are visible to all waves and the x
  // registers hold the step's first K-slice. The step reads the second slice
  // (y) while the first slice's MFMAs run (x); waits for step k + 1's operands
  // and its own LDS reads, then the barrier: no wave reads step k's A buffer
  // any more (nor, at an odd step, its B buffer), so those take the loads
  // issued now (clamped to the last step or stage: a harmless re-read into a
  // buffer no later step reads), which go out with the next step's first-slice
  // reads (x) between the second slice's MFMAs (y).
#define LMOE_STEP(NMI, k, PK, SA, SBB, NA, NBB)                                                  \
  {                                                                                             \
    LMOE_XOR(ao, 32);                                                                           \
    LMOE_XOR(bo0, 32);                                                                          \
    LMOE_READ(NMI, SA, SBB, ao, bo0, ya, yb)                                                    \
    LMOE_MFMA(NMI, xa, xb, 0, GMI)                                                              \
    LMOE_INTERLEAVE(2 * (NMI), 0, (NMI) > 0 ? 2 + (NMI) : 0)                                    \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_XOR(ao, 32);                                                                           \
    LMOE_XOR(bo0, 96);                                                                          \
    if (PK) { LMOE_WAIT_ODD() } else { LMOE_WAIT_EVEN() }                                      \
    bar();                                                                                      \
    if (PK) LMOE_ISSUE_B(((k) + 5) / 2 < nk / 2 ? ((k) + 5) / 2 : nk / 2 - 1, SBB)            \
    LMOE_ISSUE_A(((k) + 3 < nk ? (k) + 3 : nk - 1), SA)                                         \
    LMOE_READ(NMI, NA, NBB, ao, bo0, xa, xb)                                                    \
    LMOE_MFMA(NMI, ya, yb, 0, GMI)                                                              \
    LMOE_INTERLEAVE(2 * (NMI), (PK) ? 7 : 3, (NMI) > 0 ? 2 + (NMI) : 0)                         \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
  // Six steps per iteration (the A buffers repeat every 3 steps, the B
  // buffers every 6), then up to four more (K-steps are a multiple of 4).
#define LMOE_KLOOP(NMI)                                                                          \
  {                                                                                             \
    LMOE_READ(NMI, gA0, gB0, ao, bo0, xa, xb)                                              \
    int k = 0;                                                                                  \
    for (; k + 6 <= nk; k += 6) {                                                               \
      LMOE_STEP(NMI, k, 0, gA0, gB0, gA1, gB0)                                                  \
      LMOE_STEP(NMI, k + 1, 1, gA1, gB0, gA2, gB1)                                              \
      LMOE_STEP(NMI, k + 2, 0, gA2, gB1, gA0, gB1)                                              \
      LMOE_STEP(NMI, k + 3, 1, gA0, gB1, gA1, gB2)                                              \
      LMOE_STEP(NMI, k + 4, 0, gA1, gB2, gA2, gB2)                                              \
      LMOE_STEP(NMI, k + 5, 1, gA2, gB2, gA0, gB0)                                              \
    }                                                                                           \
    if (k < nk) {                                                                               \
      LMOE_STEP(NMI, k, 0, gA0, gB0, gA1, gB0)                                                  \
      LMOE_STEP(NMI, k + 1, 1, gA1, gB0, gA2, gB1)                                              \
    }                                                                                           \
    if (k + 2 < nk) {                                                                           \
      LMOE_STEP(NMI, k + 2, 0, gA2, gB1, gA0, gB1)                                              \
      LMOE_STEP(NMI, k + 3, 1, gA0, gB1, gA1, gB2)                                              \
    }                                                                                           \
  }

  // The first tile's B stage 0 and A step 0 (later tiles get theirs during the
  // previous tile's epilogue).
  setup_loads(geo);
  LMOE_ISSUE_B(0, gB0)
  LMOE_ISSUE_A(0, gA0)
  for (;;) {
    const int m0 = geo.m0, m_end = geo.m_end;
    const int n0 = geo.ntile * (EPI == EPI_SWIGLU ? GBN / 2 : GBN);   // output column start
    // the tile's rows split between the wave rows: wm = 0 takes the first r_half
    // (a multiple of 32, at least half), wm = 1 the rest; at most 160 each
    const int tile_rows = m_end - m0;
    const int r_half = 32 * ((((tile_rows + 1) >> 1) + 31) >> 5);
    const int wrow0 = wm * r_half;
    const int mrows = wm == 0 ? min(r_half, tile_rows) : tile_rows - r_half;
    const int nmi = __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : (mrows >= 32 * GMI ? GMI : (mrows + 31) / 32));
    // The lane index, opaque per tile: what derives from it (fragment and
    // staging offsets) is computed where it is used, not hoisted out of the
    // tile loop and kept live across the K loop.
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int l32 = ln & 31, half = ln >> 5;
    auto brow_of = [&](int ni) {
      return (EPI == EPI_SWIGLU) ? (ni * (GBN / 2) + wn * 32 + l32) : (wn * 64 + ni * 32 + l32);
    };

    // Prologue, continued: B stages 1 and 2 and A for steps 1 and 2 (the
    // steady state's block order), then wait for step 0's operands: B stage 0,
    // A step 0 and whatever was issued between them and these (the previous
    // tile's output stores).
    LMOE_ISSUE_B((1 < nk / 2 ? 1 : nk / 2 - 1), gB1)
    LMOE_ISSUE_A(1, gA1)
    LMOE_ISSUE_B((2 < nk / 2 ? 2 : nk / 2 - 1), gB2)
    LMOE_ISSUE_A(2, gA2)
    wait_vm<14>();
    bar();

#pragma unroll
    for (int mi = 0; mi < GMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < GNI; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
    int ao = swz(wrow0 + l32, half);           // A, first slice
    int bo0 = swzb(brow_of(0), half);          // B, first slice, even step

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
    // every load has landed (including the clamped re-reads of the last
    // steps) and every wave has finished reading the buffers
    __builtin_amdgcn_s_waitcnt(0);
    bar();

    // The next tile's first B stage and A step, into buffers the epilogue
    // does not use.
    local += stride;
    const bool more = local < chunk && xcd * chunk + local < total;
    if (more) {
      geo = tile_geo<dense>(p, xcd * chunk + local);
      setup_loads(geo);
      LMOE_ISSUE_B(0, gB0)
      LMOE_ISSUE_A(0, gA0)
    }

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
    } else {
      // ---- epilogue, by wave row: stage [160][OBN] bf16 in LDS, 16-byte stores
      // Rows [0, 64) of the staged half live in gB1, [64, 128) in gB2, [128,
      // 160) in gA1 (rows of up to 512 bytes: 32 KiB, 32 KiB, 16 KiB); gA0 and
      // gB0 take the next tile's first loads meanwhile.
      constexpr int OBN = (EPI == EPI_SWIGLU) ? GBN / 2 : GBN;
      constexpr int RBO = OBN * 2;            // bytes per staged row
      constexpr int CPR = OBN / 8;            // 16-byte chunks per staged row
      // Byte b of staged row r sits at b ^ ((r & 4) << 4): the two half-waves
      // write rows four apart, which then land 64 bytes apart (different banks).
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (wm == h) {
#pragma unroll
          for (int mi = 0; mi < GMI; ++mi) {
            // rows 32 mi .. 32 mi + 31 of the half: a buffer known at compile time
            unsigned char* buf = mi < 2 ? gB1 : (mi < 4 ? gB2 : gA1);
            // rows r and r + 1 (v, v + 1) in one packed conversion; both have
            // the same bit 2, so the same swizzle
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
              const int r = (mi & 1) * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
              unsigned char* row = buf + r * RBO;
              const int sw = (r & 4) << 4;
              if (EPI == EPI_SWIGLU) {
                const uint32_t pk = pack_bf16x2(swiglu(acc[mi][0][v], acc[mi][1][v]),
                                                swiglu(acc[mi][0][v + 1], acc[mi][1][v + 1]));
                const int b = ((wn * 32 + l32) * 2) ^ sw;
                *reinterpret_cast<bf16_t*>(row + b) = static_cast<bf16_t>(pk);
                *reinterpret_cast<bf16_t*>(row + RBO + b) = static_cast<bf16_t>(pk >> 16);
              } else {
#pragma unroll
                for (int ni = 0; ni < GNI; ++ni) {
                  const uint32_t pk = pack_bf16x2(acc[mi][ni][v], acc[mi][ni][v + 1]);
                  const int b = ((wn * 64 + ni * 32 + l32) * 2) ^ sw;
                  *reinterpret_cast<bf16_t*>(row + b) = static_cast<bf16_t>(pk);
                  *reinterpret_cast<bf16_t*>(row + RBO + b) = static_cast<bf16_t>(pk >> 16);
                }
              }
            }
          }
        }
        lds_bar();
        // rows of this half: tile rows [h r_half, h r_half + hrows); staged
        // rows [0, 64) in gB1, [64, 128) in gB2, [128, 160) in gA1
        const int hrows = h == 0 ? min(r_half, tile_rows) : tile_rows - r_half;
        const int mh = m0 + h * r_half;
        // the thread index, opaque (as the lane index above)
        int td = tid;
        __asm__ volatile("" : "+v"(td));
        auto store_rows = [&](const unsigned char* buf, int r_lo, int r_hi) {
          for (int i = td; i < (r_hi - r_lo) * CPR; i += GNT) {
            const int r = i / CPR, c = i % CPR;
            if (dense && n0 + 8 * c >= p.N) continue;
            *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)(mh + r_lo + r) * p.ldo + n0 + 8 * c) =
                *reinterpret_cast<const uint4*>(buf + r * RBO + ((c * 16) ^ ((r & 4) << 4)));
          }
          if (EPI == EPI_DOWN) {
            // sums of squares of the stored bf16 values, per row and 64-column
            // group: 8 lanes per (row, group), 16 bytes each (the groups of a
            // row on consecutive lanes), then a sum over the 8 lanes. Whole
            // 8-lane sets are active together (the bound is a multiple of 32).
            for (int i = td; i < (r_hi - r_lo) * 32; i += GNT) {
              const int r = i >> 5, grp = (i >> 3) & 3, sub = i & 7;
              const uint4 q = *reinterpret_cast<const uint4*>(buf + r * RBO + ((grp * 128 + sub * 16) ^ ((r & 4) << 4)));
              float ssq = 0.f;
              for (uint32_t w : {q.x, q.y, q.z, q.w}) {
                const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
                ssq += lo * lo;
                ssq += hi * hi;
              }
              ssq += __shfl_xor(ssq, 1);
              ssq += __shfl_xor(ssq, 2);
              ssq += __shfl_xor(ssq, 4);
              if (sub == 0) p.ss_out[(int64_t)(mh + r_lo + r) * p.ss_ld + n0 / 64 + grp] = ssq;
            }
          }
        };
        store_rows(gB1, 0, min(hrows, 64));
        store_rows(gB2, 64, max(64, min(hrows, 128)));
        store_rows(gA1, 128, max(128, hrows));
        lds_bar();   // the half is read out before the next one (or the next tile's loads) overwrite it
      }
    }
    if (!more) break;
  }
#undef LMOE_KLOOP
#undef LMOE_STEP
#undef LMOE_INTERLEAVE
#undef LMOE_MFMA
#undef LMOE_READ
#undef LMOE_XOR
#undef LMOE_WAIT_EVEN
#undef LMOE_WAIT_ODD
#undef LMOE_ISSUE_A
#undef LMOE_ISSUE_B
#undef LMOE_LD
}

}  // namespace

int gemm_grouped_tile_m() { return GBM; }

// One tile per CU at a time (160 KiB of LDS). Measured at 16K rows, a tile's
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

hipError_t launch_gemm_grouped(const GroupedParams& p, EpiKind epi, int n_cu, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (p.K % 128 != 0) return hipErrorInvalidValue;
  const bool dense = epi == EPI_F32 || epi == EPI_ACT;
  if (dense != (p.M > 0) || (dense && p.n_split < p.N && p.n_split % GBN != 0)) return hipErrorInvalidValue;
  if (dense && (p.ntiles_m < 1 || (int64_t)p.ntiles_m * GBM < p.M || p.ntiles_m * p.ntiles_n > p.max_tiles))
    return hipErrorInvalidValue;
  // persistent: at most one workgroup per compute unit (a multiple of 8, one
  // per XCD in turn), never more than the tile bound
  const int cap = n_cu >= 8 ? (n_cu / 8) * 8 : 8;
  const int grid = min(((p.max_tiles + 7) / 8) * 8, cap);
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
