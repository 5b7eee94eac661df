// Internal launch interface between the runtime (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

// Output handling of one GEMM launch (C = A . B^T, fp32 accumulation).
enum EpiKind {
  EPI_F32 = 0,     // cols [0, n_split) -> out0 fp32; cols [n_split, N) -> out1 fp32 (+ bias1)
  EPI_ACT = 1,     // out0 in the element type
  EPI_SWIGLU = 2,  // grouped: out0[p][f] = silu(gate) * up, gate/up rows of the expert's B
  EPI_DOWN = 3     // grouped: out0[p][n] = y (element type), ss_out[p][n/64] = sum of y^2
};

struct GemmParams {
  int M, N, K;                 // dense: M rows; N output columns; K inner
  const void* A;
  int64_t lda;                 // elements
  const int32_t* a_rows;       // if set, product row m reads A row a_rows[m] (gate/up: its token)
  const void* B0;
  const void* B1;              // EPI_F32: rows [n_split, N) come from B1
  int n_split;
  int64_t ldb;                 // elements
  int64_t b_expert_stride;     // grouped: elements between consecutive experts' matrices
  const int32_t* tiles;        // grouped: [slot] -> (expert, first row) pairs
  const int32_t* n_tiles;      // grouped: number of valid slots (device)
  const int32_t* offsets;      // grouped: [E+1] row offsets per expert
  int max_slots;               // grouped: grid size in slots
  void* out0;
  int64_t ldo0;
  void* out1;
  int64_t ldo1;
  const float* bias1;
  float* ss_out;
  int ss_ld;
  int F;                       // EPI_SWIGLU: up rows start at F inside the expert's B
};

// GEMM tile geometry shared with the runtime's tile list.
constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;

hipError_t launch_gemm(const GemmParams& p, EpiKind epi, bool bf16, hipStream_t s);

// Weight-streaming grouped GEMM (bf16) for experts with 1..max_rows rows; one
// wave per (expert, group of 64 weight rows). EPI_SWIGLU or EPI_DOWN.
struct StreamParams {
  const void* A;
  int64_t lda;
  const int32_t* a_rows;       // if set, product row m reads A row a_rows[m] (gate/up: its token)
  const void* B;
  int64_t ldb;
  int64_t b_expert_stride;
  const int32_t* offsets;      // [E+1]
  int n_experts;
  int groups;                  // weight-row groups per expert (F/32 for SwiGLU, Dp/64 for down)
  int max_rows;                // experts with more rows are left to the tiled GEMM
  int K;                       // multiple of 128
  int F;
  uint32_t a_bytes;            // extent of A in bytes (below 2^31)
  uint32_t b_bytes;            // extent of one expert's B in bytes (below 2^31)
  void* out;
  int64_t ldo;
  float* ss_out;
  int ss_ld;
  const int32_t* fused_n;      // if set: nothing to do when *fused_n >= whole_min (the fused
  int whole_min;               // kernel ran the streamed experts whole)
  int b_packed;                // B in the packed expert layout (pack_experts; K a multiple of 64)
};
int stream_max_rows();
hipError_t launch_stream(const StreamParams& p, EpiKind epi, hipStream_t s);

// The packed expert layout of a bf16 [rows][cols] matrix (rows and cols
// multiples of 64): blocks of 64 rows x 64 columns, 8 KiB each, block (g, s) at
// byte (g * cols / 64 + s) * 8192, its row r at r * 128 and column c at c * 2;
// element (i, j) at ((i / 64) * (cols / 64) + j / 64) * 8192 + (i % 64) * 128 +
// (j % 64) * 2. A weight-streaming stage (64 rows x 64 columns) is then one
// contiguous block. pack_experts copies n_mats such matrices from the row-major
// src to dst (no overlap).
hipError_t launch_pack_experts(const uint16_t* src, uint16_t* dst, int64_t n_mats, int rows, int cols,
                               hipStream_t s);

// The streamed experts' GEMMs in one persistent launch (n_cu workgroups): gu
// as for launch_stream(EPI_SWIGLU), dn as for launch_stream(EPI_DOWN), each
// with groups a multiple of 4. items lists the experts to run (n_items of
// them, both on the device); queue is a counter that must be zero at launch
// (the sort zeroes it). With n_items >= whole_min both GEMMs run here, whole
// experts per workgroup; otherwise nothing, and launch_stream (both EPIs) with
// fused_n = n_items and the same whole_min does the work.
struct FusedStreamParams {
  StreamParams gu, dn;
  const int32_t* items;
  const int32_t* n_items;
  int32_t* queue;
  int whole_min;
};
hipError_t launch_fused_stream(const FusedStreamParams& f, int n_cu, hipStream_t s);

// Dense C = A . B^T for T <= dense_stream_max_tokens() rows (bf16), split over
// K-slices into fp32 partials, then reduced in slice order. n_split must be a
// multiple of 64.
struct DenseStreamParams {
  const void* A;
  int64_t lda;
  const void* B0;
  const void* B1;              // rows [n_split, N) come from B1
  int n_split;
  int64_t ldb;
  int T, N, K;
  int slices;                  // from dense_stream_slices(N, K)
  float* part;                 // dense_stream_part_floats(T, N, K) floats of scratch
  void* out0;                  // [T][ldo0] fp32, or bf16 if out0_bf16
  int64_t ldo0;
  int out0_bf16;
  float* out1;                 // [T][ldo1] fp32
  int64_t ldo1;
  const float* bias1;
};
int dense_stream_max_tokens();
int dense_stream_slices(int N, int K);               // K a multiple of 64
int64_t dense_stream_part_floats(int T, int N, int K);
int dense_stream_part_ld(int N);                     // floats per token row of part
hipError_t launch_dense_stream(const DenseStreamParams& p, hipStream_t s);
// The split-K partials only (part, [slices][T][dense_stream_part_ld(N)]); the
// reduction is left to the caller.
hipError_t launch_dense_stream_partials(const DenseStreamParams& p, hipStream_t s);

// Tiled bf16 GEMMs of the prefill path (launch_gemm_grouped), 8 waves per tile.
// Dense (M > 0; EPI_F32 or EPI_ACT): out = A . B^T over M rows (row tiles of
// 256) and N columns (ntiles_n tiles of 256, the last may be partial), rows
// [n_split, N) of B^T taken from B1 (n_split a multiple of 256, or N); EPI_F32
// writes fp32 out and out1 + bias1, EPI_ACT bf16 out. Grouped (M == 0;
// EPI_SWIGLU or EPI_DOWN): expert e has mt_off[e+1] - mt_off[e] row tiles of up
// to gemm_grouped_tile_m() rows (its rows in sorted order from offsets[e],
// split evenly), each times ntiles_n column tiles.
struct GroupedParams {
  const void* A;
  int64_t lda;
  const int32_t* a_rows;       // if set, product row m reads A row a_rows[m] (gate/up: its token)
  const void* B;
  int64_t ldb;
  int64_t b_expert_stride;
  const int32_t* offsets;      // [E+1] rows per expert (sorted order)
  const int32_t* mt_off;       // [E+1] exclusive prefix of row tiles per expert (grouped)
  int E;
  int ntiles_n;                // F/128 (SwiGLU: 128 gate + 128 up rows per tile) or Dp/256
  int max_tiles;               // grid size, a bound on the tile count
  uint32_t a_bytes;            // extent of A in bytes (below 2^31)
  uint32_t b_bytes;            // extent of one expert's B in bytes (below 2^31)
  int K;                       // multiple of 128
  int F;
  void* out;
  int64_t ldo;
  float* ss_out;
  int ss_ld;
  // dense mode
  int M;                       // rows (0: grouped)
  int ntiles_m;                // row tiles, M split evenly (at most gemm_grouped_tile_m() rows each)
  int N;                       // columns
  const void* B1;              // rows of B^T at n_split and above
  int n_split;                 // multiple of 256
  float* out1;
  int64_t ldo1;
  const float* bias1;
  int b_packed;                // grouped: B in the packed expert layout (pack_experts)
};
int gemm_grouped_tile_m();
// Dense mode: the row-tile count for an M-row product with ntiles_n column
// tiles on n_cu compute units (tiles of at most gemm_grouped_tile_m() rows).
int gemm_grouped_dense_row_tiles(int M, int ntiles_n, int n_cu);
// n_cu: compute units of the device (the persistent grid's size).
hipError_t launch_gemm_grouped(const GroupedParams& p, EpiKind epi, int n_cu, hipStream_t s);

// Grouped expert GEMMs of the MXFP4-expert path: MXFP8 E4M3 activations x
// MXFP4 weights on the block-scaled MFMA. EPI_SWIGLU writes H as MXFP8 (codes
// to out, scales to out_scales); EPI_DOWN writes y as bf16 and the sums of
// squares.
struct GroupedMxParams {
  const uint8_t* A;            // [rows][K] E4M3 codes (rows in sorted order, or gathered by a_rows)
  const uint8_t* As;           // [rows][K/32] E8M0 scales
  const int32_t* a_rows;       // if set, product row m reads A row a_rows[m] (gate/up: its token)
  const uint8_t* B;            // [E][N][K/2] E2M1 codes, two per byte (low nibble first)
  const uint8_t* Bs;           // [E][N][K/32] E8M0 scales
  int N;                       // B rows per expert (2F for gate/up, Dp for down)
  const int32_t* offsets;      // [E+1]
  const int32_t* mt_off;       // [E+1]
  int E;
  int ntiles_n;
  int max_tiles;
  uint32_t a_bytes;            // extents of A and As in bytes (below 2^31)
  uint32_t as_bytes;
  int K;                       // multiple of 512
  int F;
  void* out;                   // EPI_SWIGLU: [rows][F] E4M3 codes; EPI_DOWN: [rows][ldo] bf16
  int64_t ldo;
  uint8_t* out_scales;         // EPI_SWIGLU: [rows][ldos] E8M0
  int64_t ldos;
  float* ss_out;               // EPI_DOWN
  int ss_ld;
};
// Row tiles of up to gemm_grouped_mx_tile_m() rows (each expert's rows split
// evenly over ceil(rows / tile) tiles, mt_off counting them) x 256 weight
// rows; 8 waves per tile. K a multiple of 1024.
int gemm_grouped_mx_tile_m();
hipError_t launch_gemm_grouped_mx(const GroupedMxParams& p, EpiKind epi, hipStream_t s);

// Weight-streaming grouped GEMM of the MXFP4-expert path for experts with
// 1..max_rows rows (max_rows <= stream_mx_max_rows()); one wave per (expert,
// group of 64 weight rows). K a multiple of 1024.
// Same operand and output formats as GroupedMxParams.
struct StreamMxParams {
  const uint8_t* A;            // [rows][K] E4M3 codes (rows in sorted order, or gathered by a_rows)
  const uint8_t* As;           // [rows][K/32] E8M0 scales
  const int32_t* a_rows;       // if set, product row m reads A row a_rows[m] (gate/up: its token)
  const uint8_t* B;            // [E][N][K/2] E2M1 codes
  const uint8_t* Bs;           // [E][N][K/32] E8M0 scales
  int N;                       // B rows per expert (2F for gate/up, Dp for down)
  const int32_t* offsets;      // [E+1]
  int n_experts;
  int groups;                  // F/32 for SwiGLU, Dp/64 for down
  int max_rows;
  int K;
  int F;
  uint32_t a_bytes;            // extents of A and As in bytes (below 2^31)
  uint32_t as_bytes;
  uint32_t b_bytes;            // extents of one expert's B and Bs in bytes (below 2^31)
  uint32_t bs_bytes;
  void* out;                   // EPI_SWIGLU: [rows][ldo] E4M3 codes; EPI_DOWN: [rows][ldo] bf16
  int64_t ldo;
  uint8_t* out_scales;         // EPI_SWIGLU: [rows][ldos] E8M0
  int64_t ldos;
  float* ss_out;               // EPI_DOWN: [rows][ss_ld]
  int ss_ld;
};
int stream_mx_max_rows();
hipError_t launch_stream_mx(const StreamMxParams& p, EpiKind epi, hipStream_t s);

// Router top-k + softmax; also builds, per chunk of 64 tokens, a bitmask of
// the chunk's tokens that selected each expert (ORed into chunk_masks, which
// must be zero on entry; launch_sort leaves them zero again).
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       uint64_t* chunk_masks, hipStream_t s);

// p[0 .. n) = 0, as a kernel (no memset node when the forward is captured).
hipError_t launch_clear_u64(uint64_t* p, int64_t n, hipStream_t s);

// Counting sort of the T*k assignments by expert (stable), from the chunk masks.
struct SortParams {
  const int32_t* ids;
  const float* topk_w;
  uint64_t* chunk_masks;        // [n_chunks][E]; cleared again by the sort
  int32_t* chunk_base;          // [n_chunks][E] scratch
  int32_t* counts;              // [E]
  int32_t* offsets;             // [E+1]
  int32_t* sorted_assign;       // [T*k]
  int32_t* inv;                 // [T*k]
  int32_t* row_tok;             // [T*k] token of each sorted row
  int32_t* tiles;               // [max_slots][2]
  int32_t* n_tiles;             // [1]
  int T, E, k, tile_m;
  int small_max;                // experts with 1..small_max rows get no tiles (streamed instead)
  int32_t* mt_off;              // [E+1] row-tile prefix for the large-tile grouped GEMM
  int tile_m2;                  // its rows per tile
  int32_t* stream_items;        // if set: [E] the experts with 1..small_max rows, ascending
  int32_t* n_stream;            //   [1] their number
  int32_t* queue;               //   [1] set to zero (the fused kernel's ticket counter)
};
hipError_t launch_sort(const SortParams& p, hipStream_t s);

// xp[t] = bf16/f32( P[t] * rsqrt(mean(P[t]^2) + eps) * g ), one row per token;
// the expert GEMMs gather the rows of their sorted assignments.
hipError_t launch_pool_norm(const float* P, const float* g, int T, int Dp, float eps, void* xp, bool bf16,
                            hipStream_t s);

// Router + pooler at small batches: reduce the split-K partials of d (fp32
// out0 = P, out1 = logits + bias1) and normalize each P row into xp in one
// kernel. mode 0: bf16 xp, 2: MXFP8 (codes to xp, scales). With tk.ids set,
// each token's top-k (launch_topk's outputs) too, from the logits it reduced
// (then out1 must be the [T][E] logits, ldo1 = E).
struct TopkOut {
  int32_t* ids;            // [T][k], or null: no top-k here
  float* w;                // [T][k]
  uint64_t* chunk_masks;   // [T/64][E], zero before the call
  int k;
};
hipError_t launch_splitk_pool_norm(const DenseStreamParams& d, const float* g, float eps, void* xp, int mode,
                                   uint8_t* scales, const TopkOut& tk, hipStream_t s);

// MXFP4-expert path: xp quantized to MXFP8 E4M3 blocks of 32 (codes [T][Dp],
// scales [T][Dp/32]) instead of stored as bf16.
hipError_t launch_pool_norm_mx(const float* P, const float* g, int T, int Dp, float eps, uint8_t* codes,
                               uint8_t* scales, hipStream_t s);
// n fp32 values (n a multiple of 32) -> MXFP8 E4M3 codes [n] and scales [n/32].
hipError_t launch_mx_quant(const float* x, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t s);

// NVFP4 expert weights (E2M1 codes [M][rows][cols/2], UE4M3 scales per 16
// [M][rows][cols/16], FP32 scale per matrix [M]) re-encoded as MXFP4 (codes
// [M][rows][cols/2], E8M0 scales [M][rows][cols/32]); cols a multiple of 32.
// out_codes may be codes itself.
hipError_t launch_nvfp4_to_mxfp4(const uint8_t* codes, const uint8_t* scales16, const float* gscale,
                                 int64_t n_mats, int64_t rows, int64_t cols, uint8_t* out_codes,
                                 uint8_t* out_scales, hipStream_t s);

// u[t] = sum_j w[t][j] * rsqrt(sum(ss[inv[t,j]]) / Dp + eps) * g_e * y[inv[t,j]]
struct CombineParams {
  const void* y;           // [T*k][Dp] sorted rows
  const float* ss;         // [T*k][Dp/64]
  const int32_t* inv;      // [T*k]
  const int32_t* ids;      // [T][k]
  const float* w;          // [T][k]
  const float* g_expert;   // [E][Dp]
  void* u;                 // [T][Dp]
  int T, k, Dp;
  float eps;
};
hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s);

}  // namespace lmoe
