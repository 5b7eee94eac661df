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
// Operands reach LDS through direct global-to-LDS buffer loads. The token
// rows (A) move in 32-wide K-steps, 64 bytes of each row, through three
// buffers (20 KiB each): the loads for step k + 3 are issued at step k. The
// weights (B) move in stages of two K-steps, whole 128-byte row segments, 8
// rows per load, through three buffers (32 KiB each): the loads for steps
// 2s + 6 and 2s + 7 are issued at step 2s + 1, once both halves of a buffer
// are read (156 KiB in all). The weights come from HBM on their first touch,
// the token rows mostly from L2: the weights run further ahead, and whole-line
// loads halve their requests for the same bytes. A stage of A is 20 loads of
// 16 rows x 64 bytes (wave w issues loads w, w + 8, w + 16: waves 0-3 three,
// waves 4-7 two; A loads wholly past the tile's last row are skipped); a
// stage of B is 32 loads of 8 rows x 128 bytes, four per wave. The 16-byte
// chunks of each row are XOR-swizzled so that fragment reads are
// conflict-free.
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
  // B load j (of a stage) moves rows 8 j .. 8 j + 7, lane i row 8 j + i / 8 at
  // chunk position i % 8 (which holds logical chunk (i % 8) ^ g(row)); wave w
  // issues j = w, w + 8, w + 16, w + 24.
  auto b_off = [&](int r) -> uint32_t {
    const int n = dense ? r : (EPI == EPI_SWIGLU) ? ((r < GBN / 2) ? (n0 + r) : (p.F + n0 + r - GBN / 2)) : (n0 + r);
    const uint32_t c = (lane & 7) ^ swz8(r);
    return (uint32_t)n * (uint32_t)(p.ldb * 2) + c * 16;
  };
  // A load j (of a stage) moves rows 16 j .. 16 j + 15, lane i row 16 j + i / 4
  // at chunk position i % 4; wave w issues j = w, w + 8, w + 16 (while j < 20)
  uint32_t ga[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) ga[i] = (wave + 8 * i < LA) ? a_off(16 * (wave + 8 * i) + (lane >> 2)) : kOutOfRange;
  // The wave's four B loads (rows r, r + 64, r + 128, r + 192; the swizzle
  // depends on the row's low 4 bits only) differ by whole rows: one offset
  // register plus uniform row deltas in the scalar offset. SwiGLU rows 128..255
  // are the up rows, F - 128 further on.
  const uint32_t gb0 = b_off(8 * wave + (lane >> 3));
  const int rowb = (int)p.ldb * 2;
  const int up = (EPI == EPI_SWIGLU && !dense) ? (p.F - GBN / 2) * rowb : 0;
  const int gbd1 = 64 * rowb, gbd2 = 128 * rowb + up, gbd3 = 192 * rowb + up;
  // Waves 0-3 issue a third A load (rows 256 + 16 wave ..) only if some of its
  // rows are in the tile: a 256-row tile then moves 32 rows per K-step instead
  // of 36 x 16. The LDS rows a skipped load would have filled are read only
  // for output rows past the tile's end, which are never stored.
  const bool three_a = wave + 16 < LA && 16 * (wave + 16) < tile_rows;

#define LMOE_LD(RS, OFF, DST, KO) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds((RS), (LMOE_AS3 void*)(DST), 16, (int)(OFF), (KO), 0, 0);
  // A for K-step kt (rotated), into buffer SA
#define LMOE_ISSUE_A(kt, SA)                                                                            \
  {                                                                                                    \
    const int kr_ = (kt) + krot;                                                                       \
    const int ko = (kr_ >= nk ? kr_ - nk : kr_) * RB;                                                  \
    LMOE_LD(rsA, ga[0], (SA) + wave * 16 * RB, ko)                                                     \
    LMOE_LD(rsA, ga[1], (SA) + (wave + 8) * 16 * RB, ko)                                               \
    if (three_a) LMOE_LD(rsA, ga[2], (SA) + (wave + 16) * 16 * RB, ko)                                 \
  }
  // B for K-steps 2 st and 2 st + 1 (rotated; krot is even, so the pair never
  // wraps), into buffer SBB
#define LMOE_ISSUE_B(st, SBB)                                                                           \
  {                                                                                                    \
    const int kr_ = 2 * (st) + krot;                                                                   \
    const int ko = (kr_ >= nk ? kr_ - nk : kr_) * RB;                                                  \
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
  // one B stage when k - 1 is odd. A blocks are 3 loads (waves with three_a)
  // or 2, B stages 4.
#define LMOE_WAIT_EVEN()               \
  if (three_a) wait_vm<7>();           \
  else wait_vm<6>();
#define LMOE_WAIT_ODD()                \
  if (three_a) wait_vm<3>();           \
  else wait_vm<2>();

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
  // One offset register per operand (ao for A, bo0 and bo1 for the two B
  // fragments) walks the logical chunks in place: the second 16-wide K-slice
  // of a step is the first's chunk with bit 1 set (byte offset XOR 32), a B
  // row's odd K-step its even one's with bit 2 set (XOR 64). The XORs are
  // opaque to the compiler, which otherwise keeps every variant (and their
  // sums with the buffers' LDS addresses) in registers and spills inside the
  // K loop.
  const int l32 = lane & 31, half = lane >> 5;
  auto brow_of = [&](int ni) {
    return (EPI == EPI_SWIGLU) ? (ni * (GBN / 2) + wn * 32 + l32) : (wn * 64 + ni * 32 + l32);
  };
  int ao = swz(wrow0 + l32, half);           // A, first slice
  int bo0 = swzb(brow_of(0), half), bo1 = swzb(brow_of(1), half);   // B, first slice, even step
#define LMOE_XOR(X, IMM) __asm__ volatile("v_xor_b32 %0, " #IMM ", %0" : "+v"(X))

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
  // K-step k: A of step k in SA, of step k + 1 in NA; B of step k in SBB at
  // parity PK (0: first K-step of the B stage, 1: second), of step k + 1 in
  // NBB. On entry A and B of step k are visible to all waves and the x
  // registers hold the step's first K-slice. The step reads the second slice
  // (y) and runs the first slice's MFMAs (x); waits for step k + 1's operands
  // and its own LDS reads, then the barrier: no wave reads step k's A buffer
  // any more (nor, at an odd step, its B buffer), so those take the loads
  // issued now (clamped to the last step or stage: a harmless re-read into a
  // buffer no later step reads); reads the next step's first slice (x) and
  // runs the second slice's MFMAs (y).
#define LMOE_STEP(NMI, k, PK, SA, SBB, NA, NBB)                                                  \
  {                                                                                             \
    LMOE_XOR(ao, 32);                                                                           \
    LMOE_XOR(bo0, 32);                                                                          \
    LMOE_XOR(bo1, 32);                                                                          \
    LMOE_READ(NMI, SA, SBB, ao, bo0, bo1, ya, yb)                                               \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, xa, xb)                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    if (PK) { LMOE_WAIT_ODD() } else { LMOE_WAIT_EVEN() }                                      \
    bar();                                                                                      \
    if (PK) LMOE_ISSUE_B(((k) + 5) / 2 < nk / 2 ? ((k) + 5) / 2 : nk / 2 - 1, SBB)            \
    LMOE_ISSUE_A(((k) + 3 < nk ? (k) + 3 : nk - 1), SA)                                         \
    LMOE_XOR(ao, 32);                                                                           \
    LMOE_XOR(bo0, 96);                                                                          \
    LMOE_XOR(bo1, 96);                                                                          \
    LMOE_READ(NMI, NA, NBB, ao, bo0, bo1, xa, xb)                                               \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, ya, yb)                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
  // Six steps per iteration (the A buffers repeat every 3 steps, the B
  // buffers every 6), then up to four more (K-steps are a multiple of 4).
#define LMOE_KLOOP(NMI)                                                                          \
  {                                                                                             \
    LMOE_READ(NMI, gA0, gB0, ao, bo0, bo1, xa, xb)                                              \
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

  const int nk = p.K / 32;                   // a multiple of 4 (K % 128 == 0)
  // Each column tile walks K from its own starting step (4 steps further per
  // column tile), so that the tiles sharing a row tile's token slice request it
  // a few steps apart. The order depends on the column tile only, so every
  // output element is summed in one fixed order, whatever the batch.
  const int krot = (ntile * 4) % nk;
  // Prologue: B stages 0..2 and A for steps 0..2 in the steady state's order
  // (block k holds the B stage first), then wait for step 0's operands: A for
  // step 0 and everything before it.
  LMOE_ISSUE_B(0, gB0)
  LMOE_ISSUE_B((1 < nk / 2 ? 1 : nk / 2 - 1), gB1)
  LMOE_ISSUE_A(0, gA0)
  LMOE_ISSUE_A(1, gA1)
  LMOE_ISSUE_B((2 < nk / 2 ? 2 : nk / 2 - 1), gB2)
  LMOE_ISSUE_A(2, gA2)
  if (three_a) wait_vm<10>();
  else wait_vm<8>();
  bar();
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
#undef LMOE_XOR
#undef LMOE_WAIT_EVEN
#undef LMOE_WAIT_ODD
#undef LMOE_ISSUE_A
#undef LMOE_ISSUE_B
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
