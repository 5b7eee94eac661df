// Large-tile dense GEMM (bf16): the router + pooler and the unpooler at
// prefill sizes, out = A . B^T with fp32 out (and the router's columns, from a
// second weight matrix plus a bias) or bf16 out.
//
// Tile 256 x 256 (A rows x B rows), 256 threads = 4 wave64 in a 2 x 2 grid,
// each wave a 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 bf16 (accumulators in
// AGPRs). Per 16-wide K-slice a wave reads 8 operand chunks from LDS for 16
// MFMAs, which keeps LDS traffic well under its bandwidth.
//
// Operands reach LDS through gfx950's direct global-to-LDS loads (no register
// staging) in a four-stage pipeline of 32-wide K-steps (4 x 32 KiB): the loads
// for step k + 3 are issued while step k computes, so three steps of latency
// (about 3000 cycles at full MFMA rate) are covered.
//
// Scheduling for the 8 XCDs: the tiles form one index space ordered (m-tile,
// n-tile); it is cut into 8 contiguous chunks and workgroup b (dispatched to
// XCD b % 8) takes tile (b % 8) * chunk + b / 8. So the CUs of one XCD share
// row tiles of A in their L2.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

constexpr int BM = 256, BNB = 256;   // A rows, B rows per tile
constexpr int NT = 256;
constexpr int RB = 64;                // bytes of each tile row per pipeline stage (32 bf16)
constexpr int SB = BM * RB;           // bytes per operand per stage (16 KiB)

#define LMOE_AS3 __attribute__((address_space(3)))

// Fourth word of a raw buffer descriptor on CDNA (no swizzle, no stride,
// 32-bit data format field set so that offsets are bytes).
constexpr int kBufWord3 = 0x00020000;
// A buffer offset past every extent used here (all below 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;

// Four pipeline stages for A and B, each a separate LDS object so that the
// compiler can tell the stages apart when it orders reads against the
// asynchronous global-to-LDS loads still in flight for other stages.
__shared__ __attribute__((aligned(16))) unsigned char sA0[SB], sB0[SB], sA1[SB], sB1[SB],
    sA2[SB], sB2[SB], sA3[SB], sB3[SB];

// Byte offset of logical 16-byte chunk c (0..3) of tile row r (64-byte rows).
// The chunk is stored at position c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3.
// A 128-bit fragment read has 32 lanes on 32 consecutive rows at one logical
// chunk; with this f any 8 consecutive rows (from a multiple of 8) land on 8
// distinct 16-byte slots of a 128-byte bank line, and any 16 (from a multiple
// of 16) on 16 distinct slots of 256 bytes, so the read is conflict-free
// whether the LDS serves 8 or 16 lanes of a 128-bit read per clock.
__device__ __forceinline__ int swz(int r, int c) {
  return r * RB + ((c ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4);
}

__device__ __forceinline__ void mfma32(const uint4& a, const uint4& b, f32x16_t& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// Before the stage barrier: wait until this wave has at most 16 global loads
// in flight (its two later stages of 8) and none of its LDS reads outstanding.
// The second part matters because the scheduler may move the previous step's
// MFMAs (not their LDS reads) past the barrier, after which another wave's
// load may overwrite the buffer those reads come from.
__device__ __forceinline__ void wait_vm(int) { __builtin_amdgcn_s_waitcnt(0x4070); }

// Stage hand-off barrier. __syncthreads would fence global memory and so wait
// for every load in flight (the later pipeline stages), and even an LDS-scoped
// release fence waits for them, since direct-to-LDS loads count as LDS writes.
// So: each wave first waits explicitly for its own loads of the stage and its
// own LDS reads (wait_vm), then the barrier, then an LDS-scoped acquire fence
// that keeps the compiler from hoisting the stage's LDS reads above it.
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm256_kernel(Gemm256Params p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets in SGPRs
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile of this workgroup (XCD-chunked order): (m-tile, n-tile) -------
  const int ntm = (p.M + BM - 1) / BM;
  const int total = ntm * p.ntiles_n;
  const int chunk = (total + 7) / 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int t = xcd * chunk + local;
  if (local >= chunk || t >= total) return;
  const int ntile = t % p.ntiles_n;
  const int m0 = (t / p.ntiles_n) * BM;
  const int m_end = p.M;
  const int n0 = ntile * BNB;                // output column start

  // ---- global-to-LDS loads ------------------------------------------------
  // Per stage each wave moves 4 x 16 rows of A and of B, one 1 KiB load each:
  // lane i carries row (4 w + j) * 16 + i / 4 and lands at LDS chunk position
  // i % 4 of that row, so it fetches the logical chunk stored there.
  // The loads are buffer loads: the base addresses and extents sit in two
  // buffer descriptors (SGPRs), each lane keeps a 32-bit byte offset per row,
  // and the K-step's offset is a scalar. Reads past an extent return zero.
  // (Buffer loads, unlike global ones, are known to the compiler to touch only
  // global memory and LDS through the DMA path, so it keeps exact LDS-read
  // wait counts around them.)
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), (short)0, (int)p.a_bytes, kBufWord3);
  // B rows of the tile: its own 256 rows from B (columns below n_split) or B1,
  // the extent ending at row N (rows past it read as zero).
  const bf16_t* Bt = (n0 < p.n_split) ? static_cast<const bf16_t*>(p.B) + (int64_t)n0 * p.ldb
                                      : static_cast<const bf16_t*>(p.B1) + (int64_t)(n0 - p.n_split) * p.ldb;
  const int b_ext = min(BNB, p.N - n0) * (int)p.ldb * 2;
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Bt), (short)0, b_ext, kBufWord3);
  const int pos = lane & 3;
  // Rows past the end (tail tiles) get an offset beyond every extent: the
  // buffer load then reads nothing from memory (its lanes return zero), so a
  // tile with few rows costs little more than its B slice. Those rows are
  // never stored.
  auto a_off = [&](int r) -> uint32_t {
    const int m = m0 + r;
    if (m >= m_end) return kOutOfRange;
    const uint32_t c = pos ^ (((r >> 1) ^ (r >> 3)) & 3);
    return (uint32_t)m * (uint32_t)(p.lda * 2) + c * 16;
  };
  auto b_off = [&](int r) -> uint32_t {
    const uint32_t c = pos ^ (((r >> 1) ^ (r >> 3)) & 3);
    return (uint32_t)r * (uint32_t)(p.ldb * 2) + c * 16;
  };
  const int rr = wave * 64 + (lane >> 2);    // row of load j is rr + 16 j
  const uint32_t ga0 = a_off(rr), ga1 = a_off(rr + 16), ga2 = a_off(rr + 32), ga3 = a_off(rr + 48);
  const uint32_t gb0 = b_off(rr), gb1 = b_off(rr + 16), gb2 = b_off(rr + 32), gb3 = b_off(rr + 48);
  const int dbase = wave * 64 * RB;          // this wave's 4 KiB region of each operand stage

#define LMOE_LD(RS, OFF, DST, KO) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds((RS), (LMOE_AS3 void*)(DST), 16, (int)(OFF), (KO), 0, 0);
#define LMOE_ISSUE(kt, SA, SBB)                                                                         \
  {                                                                                                    \
    const int kr_ = (kt) + krot;                                                                       \
    const int ko = (kr_ >= nk ? kr_ - nk : kr_) * RB;                                                  \
    LMOE_LD(rsA, ga0, (SA) + dbase, ko)                                                                \
    LMOE_LD(rsA, ga1, (SA) + dbase + 16 * RB, ko)                                                      \
    LMOE_LD(rsA, ga2, (SA) + dbase + 32 * RB, ko)                                                      \
    LMOE_LD(rsA, ga3, (SA) + dbase + 48 * RB, ko)                                                      \
    LMOE_LD(rsB, gb0, (SBB) + dbase, ko)                                                               \
    LMOE_LD(rsB, gb1, (SBB) + dbase + 16 * RB, ko)                                                     \
    LMOE_LD(rsB, gb2, (SBB) + dbase + 32 * RB, ko)                                                     \
    LMOE_LD(rsB, gb3, (SBB) + dbase + 48 * RB, ko)                                                     \
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  // LDS rows of this lane's MFMA operands: A rows wm*128 + 32 mi + l32, B rows
  // wn*128 + 32 ni + l32.
  const int l32 = lane & 31, half = lane >> 5;
  const int aoff0 = swz(wm * 128 + l32, half), aoff1 = swz(wm * 128 + l32, 2 + half);
  auto brow_of = [&](int ni) { return wn * 128 + ni * 32 + l32; };
  const int b00 = swz(brow_of(0), half), b01 = swz(brow_of(0), 2 + half);
  const int b10 = swz(brow_of(1), half), b11 = swz(brow_of(1), 2 + half);
  const int b20 = swz(brow_of(2), half), b21 = swz(brow_of(2), 2 + half);
  const int b30 = swz(brow_of(3), half), b31 = swz(brow_of(3), 2 + half);
  // rows of this wave that hold real tokens (tail tiles skip empty 32-row groups)
  const int mrows = m_end - (m0 + wm * 128);
  const int nmi = __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : (mrows >= 128 ? 4 : (mrows + 31) / 32));

  // Operand fragments: two register sets, so that the LDS reads of the next
  // 16-wide K-slice are in flight while the MFMAs of the current one run.
  uint4 xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3;
  uint4 ya0, ya1, ya2, ya3, yb0, yb1, yb2, yb3;

  // Reads of one K-slice's fragments (only the A rows of the NMI live 32-row
  // groups; none at all if NMI == 0).
#define LMOE_READ(NMI, SA, SBB, AO, B0, B1, B2, B3, PA, PB)                                      \
  if ((NMI) > 0) {                                                                              \
    PB##0 = *reinterpret_cast<const uint4*>((SBB) + (B0));                                      \
    PB##1 = *reinterpret_cast<const uint4*>((SBB) + (B1));                                      \
    PB##2 = *reinterpret_cast<const uint4*>((SBB) + (B2));                                      \
    PB##3 = *reinterpret_cast<const uint4*>((SBB) + (B3));                                      \
    PA##0 = *reinterpret_cast<const uint4*>((SA) + (AO));                                       \
  }                                                                                             \
  if ((NMI) > 1) PA##1 = *reinterpret_cast<const uint4*>((SA) + (AO) + 32 * RB);                \
  if ((NMI) > 2) PA##2 = *reinterpret_cast<const uint4*>((SA) + (AO) + 64 * RB);                \
  if ((NMI) > 3) PA##3 = *reinterpret_cast<const uint4*>((SA) + (AO) + 96 * RB);
#define LMOE_MFMA(NMI, PA, PB)                                                                   \
  if ((NMI) > 0) {                                                                              \
    mfma32(PA##0, PB##0, acc[0][0]); mfma32(PA##0, PB##1, acc[0][1]);                           \
    mfma32(PA##0, PB##2, acc[0][2]); mfma32(PA##0, PB##3, acc[0][3]);                           \
  }                                                                                             \
  if ((NMI) > 1) {                                                                              \
    mfma32(PA##1, PB##0, acc[1][0]); mfma32(PA##1, PB##1, acc[1][1]);                           \
    mfma32(PA##1, PB##2, acc[1][2]); mfma32(PA##1, PB##3, acc[1][3]);                           \
  }                                                                                             \
  if ((NMI) > 2) {                                                                              \
    mfma32(PA##2, PB##0, acc[2][0]); mfma32(PA##2, PB##1, acc[2][1]);                           \
    mfma32(PA##2, PB##2, acc[2][2]); mfma32(PA##2, PB##3, acc[2][3]);                           \
  }                                                                                             \
  if ((NMI) > 3) {                                                                              \
    mfma32(PA##3, PB##0, acc[3][0]); mfma32(PA##3, PB##1, acc[3][1]);                           \
    mfma32(PA##3, PB##2, acc[3][2]); mfma32(PA##3, PB##3, acc[3][3]);                           \
  }
  // K-step k (stage k in buffers SA/SBB, stage k + 1 in NA/NB). On entry stage k
  // is visible to all waves, the loads of stages k + 1 .. k + 3 are in flight and
  // the x registers hold the fragments of the step's first K-slice. The step
  //   reads the second slice (y) and runs the first slice's MFMAs (x);
  //   waits for stage k + 1 and for its own LDS reads, then the barrier: after
  //   it no wave reads stage k any more, so the loads of stage k + 4 go into
  //   its buffer (clamped to the last stage: a harmless re-read into a buffer
  //   no later step reads, so every step has the same loads in flight);
  //   reads the next step's first slice (x) and runs the second slice's MFMAs (y).
  // The scheduling barriers keep each group of LDS reads ahead of the MFMAs
  // that follow it, so their latency hides behind those MFMAs.
#define LMOE_STEP(NMI, k, SA, SBB, NA, NB)                                                       \
  {                                                                                             \
    LMOE_READ(NMI, SA, SBB, aoff1, b01, b11, b21, b31, ya, yb)                                  \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, xa, xb)                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    wait_vm(16);                                                                                \
    bar();                                                                                      \
    LMOE_ISSUE(((k) + 4 < nk ? (k) + 4 : nk - 1), SA, SBB)                                      \
    LMOE_READ(NMI, NA, NB, aoff0, b00, b10, b20, b30, xa, xb)                                   \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    LMOE_MFMA(NMI, ya, yb)                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
#define LMOE_KLOOP(NMI)                                                                          \
  {                                                                                             \
    LMOE_READ(NMI, sA0, sB0, aoff0, b00, b10, b20, b30, xa, xb)                                 \
    for (int k = 0; k < nk; k += 4) {                                                           \
      LMOE_STEP(NMI, k, sA0, sB0, sA1, sB1)                                                     \
      LMOE_STEP(NMI, k + 1, sA1, sB1, sA2, sB2)                                                 \
      LMOE_STEP(NMI, k + 2, sA2, sB2, sA3, sB3)                                                 \
      LMOE_STEP(NMI, k + 3, sA3, sB3, sA0, sB0)                                                 \
    }                                                                                           \
  }

  // Prologue: stages 0..2 in flight; wait for stage 0, then start stage 3.
  const int nk = p.K / 32;                   // a multiple of 4 (K % 128 == 0)
  // Each column tile walks K from its own starting step (4 steps further per
  // column tile), so that the tiles sharing a row tile's token slice request
  // it a few steps apart rather than at once (measured: about 2% faster at
  // the prefill shape). The order depends on the column tile only, so every
  // output element is summed in one fixed order, whatever the batch.
  const int krot = (ntile * 4) % nk;
  LMOE_ISSUE(0, sA0, sB0)
  LMOE_ISSUE(1, sA1, sB1)
  LMOE_ISSUE(2, sA2, sB2)
  wait_vm(16);
  bar();
  LMOE_ISSUE(3, sA3, sB3)
  // One K loop per number of live 32-row groups (uniform per wave; waves of a
  // tile may differ, and all run the same barriers): full, half (1-2 groups,
  // computing 2) and none (3 groups run the full loop).
  if (nmi > 2) {
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
#undef LMOE_ISSUE
#undef LMOE_LD
  __syncthreads();   // every load has landed and every wave has finished reading

  if (EPI == EPI_F32) {
    // fp32 out, straight from the accumulators: the 32 lanes of a half-wave
    // store 32 consecutive columns of a row (128 bytes). Columns below n_split
    // go to out, the rest to out1 plus bias1 (router logits).
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 128 + mi * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (m >= m_end) continue;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int n = n0 + wn * 128 + ni * 32 + l32;
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

  // ---- bf16 out: stage [256][256] in LDS, 16-byte stores -------------------
  // The staging tile spans the stage buffers: rows [32 q, 32 q + 32) live in
  // buffer q (A0, B0, A1, ..., B3 in declaration order), 16 KiB each.
  auto srow = [&](int r) -> bf16_t* {
    unsigned char* b;
    switch (r >> 5) {
      case 0: b = sA0; break;
      case 1: b = sB0; break;
      case 2: b = sA1; break;
      case 3: b = sB1; break;
      case 4: b = sA2; break;
      case 5: b = sB2; break;
      case 6: b = sA3; break;
      default: b = sB3; break;
    }
    return reinterpret_cast<bf16_t*>(b) + (r & 31) * BNB;
  };
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 128 + mi * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      bf16_t* row = srow(r);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) row[wn * 128 + ni * 32 + l32] = f32_to_bf16(acc[mi][ni][v]);
    }
  __syncthreads();
  constexpr int CPR = BNB / 8;
  for (int i = tid; i < BM * CPR; i += NT) {
    const int r = i / CPR, c = (i % CPR) * 8;
    const int m = m0 + r;
    if (m >= m_end || n0 + c >= p.N) continue;
    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + (int64_t)m * p.ldo + n0 + c) =
        *reinterpret_cast<const uint4*>(srow(r) + c);
  }
}

}  // namespace

hipError_t launch_gemm256(const Gemm256Params& p, EpiKind epi, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (p.M <= 0) return hipErrorInvalidValue;
  const int grid = ((p.max_tiles + 7) / 8) * 8;
  if (epi == EPI_F32 && p.M > 0)
    hipLaunchKernelGGL(gemm256_kernel<EPI_F32>, dim3(grid), dim3(NT), 0, s, p);
  else if (epi == EPI_ACT && p.M > 0)
    hipLaunchKernelGGL(gemm256_kernel<EPI_ACT>, dim3(grid), dim3(NT), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lmoe
