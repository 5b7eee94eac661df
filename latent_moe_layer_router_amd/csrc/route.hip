// Routing: top-k + softmax over the selected logits, and the token-to-expert
// permutation as a stable counting sort.
//
// Top-k (LMSYS blog, "Kernel optimizations": a top-k routing kernel emits the
// expert ids and weights in the layout the expert kernel reads): one wave64 per
// token, each lane holding E/64 logits; k rounds of a wave arg-max on
// (logit desc, index asc). Weights are the softmax of the k selected logits.
//
// Permutation (blog, "AMD support": the atomic-add expert sort became an LDS
// kernel on MI355X). Tokens are taken in chunks of 64, one bit per token:
//  1. while doing top-k, each token ORs bit (t % 64) into its chunk's mask of
//     every expert it selected (global atomic OR; the masks start at zero and
//     step 3 clears them again after use);
//  2. a single workgroup turns the masks into per-(chunk, expert) bases
//     (running sums of popcounts over chunks) and the per-expert offsets
//     (exclusive prefix sum over experts with wavefront prefix sums), and lays
//     out the grouped-GEMM tile list;
//  3. each chunk places its assignments: the rank of token t inside expert e
//     is the popcount of e's mask below t's bit, so equal keys keep token order.
// Every step is integer and order-independent, hence bit-exact and
// deterministic.
#include "common.h"
#include "kernels.h"
#include "route.h"

namespace lmoe {

namespace {

// One wave per token, 4 per workgroup, so that even a decode-sized batch
// spreads over the GPU.
constexpr int kTopkWaves = 4;

__global__ __launch_bounds__(kTopkWaves * 64) void topk_kernel(const float* __restrict__ logits, int T,
                                                               int E, int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ w,
                                                               uint64_t* __restrict__ chunk_masks) {
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t >= T) return;                        // whole waves
  topk_token(logits + (int64_t)t * E, t, E, k, ids, w, chunk_masks);
}

// Exclusive prefix sum over the block (blockDim.x a multiple of 64, <= 1024).
__device__ int block_exclusive_scan(int x, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int v = lane < nw ? wave_tot[lane] : 0;
    int vi = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(vi, o, kWave);
      if (lane >= o) vi += y;
    }
    if (lane < nw) wave_tot[lane] = vi - v;        // exclusive wave bases
    if (lane == nw - 1) *total = vi;
  }
  __syncthreads();
  const int r = incl - x + wave_tot[wave];
  __syncthreads();
  return r;
}

// One workgroup of 1024 threads: thread (part q, expert e) with e < E_pad (E
// rounded up to a wave) takes a contiguous share of the chunks, so that the
// per-expert walk over the chunks runs in 1024 / E_pad parallel pieces.
// Chunk `chunk`'s assignments, by one wave: token t = 64 chunk + lane places
// its k assignments, then the wave clears the chunk's masks for the next
// call's atomic ORs (every lane's mask loads have returned by then: their
// values fed the positions stored before).
__device__ __forceinline__ void scatter_chunk(const SortParams& p, int chunk, int lane) {
  const int t = chunk * kChunk + lane;
  if (t < p.T) {
    const uint64_t below = lanemask_lt(lane);
    for (int j = 0; j < p.k; ++j) {
      const int a = t * p.k + j;
      const int e = p.ids[a];
      const uint64_t m = p.chunk_masks[(int64_t)chunk * p.E + e];
      const int pos = p.offsets[e] + p.chunk_base[(int64_t)chunk * p.E + e] + __popcll(m & below);
      p.sorted_assign[pos] = a;
      p.inv[a] = pos;
      p.row_tok[pos] = t;
    }
  }
  __builtin_amdgcn_wave_barrier();
  for (int e = lane; e < p.E; e += kChunk) p.chunk_masks[(int64_t)chunk * p.E + e] = 0ull;
}

constexpr int kScanScatterChunks = 1024 / kWave;

__global__ __launch_bounds__(1024) void sort_scan_kernel(SortParams p) {
  __shared__ int wave_tot[16];
  __shared__ int total;
  __shared__ int part_tot[1024];
  const int e_pad = ((p.E + kWave - 1) / kWave) * kWave;
  const int parts = blockDim.x / e_pad;
  const int e = threadIdx.x % e_pad, q = threadIdx.x / e_pad;
  const bool live = e < p.E && q < parts;
  const int n_chunks = (p.T + kChunk - 1) / kChunk;
  const int per = (n_chunks + parts - 1) / parts;
  const int c0 = q * per, c1 = min(n_chunks, c0 + per);
  // 1. this piece's count (eight mask loads in flight at a time)
  int mine = 0;
  if (live) {
    for (int c = c0; c < c1; c += 8) {
      uint64_t m[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = (c + i < c1) ? p.chunk_masks[(int64_t)(c + i) * p.E + e] : 0ull;
#pragma unroll
      for (int i = 0; i < 8; ++i) mine += __popcll(m[i]);
    }
  }
  part_tot[threadIdx.x] = mine;
  __syncthreads();
  // 2. the piece's base within its expert, and the expert's count
  int base = 0, cnt = 0;
  for (int r = 0; r < parts; ++r) {
    const int v = part_tot[r * e_pad + e];
    base += r < q ? v : 0;
    cnt += v;
  }
  // 3. per-chunk bases of this piece
  if (live) {
    int run = base;
    for (int c = c0; c < c1; ++c) {
      p.chunk_base[(int64_t)c * p.E + e] = run;
      run += __popcll(p.chunk_masks[(int64_t)c * p.E + e]);
    }
  }
  // Expert offsets and tile lists from the first piece of each expert (threads
  // 0 .. E_pad-1, in expert order; the others add nothing to the scans).
  const bool head = e < p.E && q == 0;
  if (head) p.counts[e] = cnt;
  const int off = block_exclusive_scan(head ? cnt : 0, wave_tot, &total);
  if (head) p.offsets[e] = off;
  if (threadIdx.x == 0) p.offsets[p.E] = total;
  // Grouped-GEMM tiles: expert e gets ceil(count / tile_m) row tiles, unless its
  // rows are few enough for the weight-streaming kernel.
  // (no expert has more than T rows: with T <= small_max the tile lists are
  // empty, and their scans are skipped; the condition is uniform)
  const bool tiled = p.T > p.small_max;
  const int nt = (head && cnt > p.small_max) ? (cnt + p.tile_m - 1) / p.tile_m : 0;
  const int tbase = tiled ? block_exclusive_scan(nt, wave_tot, &total) : 0;
  for (int i = 0; i < nt; ++i) {
    p.tiles[2 * (tbase + i)] = e;
    p.tiles[2 * (tbase + i) + 1] = off + i * p.tile_m;
  }
  if (threadIdx.x == 0) *p.n_tiles = tiled ? total : 0;
  // the streamed experts (1..small_max rows), for the fused kernel's queue
  if (p.stream_items) {
    const int st = (head && cnt > 0 && cnt <= p.small_max) ? 1 : 0;
    const int sbase = block_exclusive_scan(st, wave_tot, &total);
    if (st) p.stream_items[sbase] = e;
    if (threadIdx.x == 0) {
      *p.n_stream = total;
      *p.queue = 0;
    }
  }
  // the large-tile GEMM: ceil(count / 256) row tiles
  const int nt2 = (head && cnt > p.small_max) ? (cnt + p.tile_m2 - 1) / p.tile_m2 : 0;
  const int mbase = tiled ? block_exclusive_scan(nt2, wave_tot, &total) : 0;
  if (head) p.mt_off[e] = mbase;
  if (threadIdx.x == 0) p.mt_off[p.E] = tiled ? total : 0;
  // Up to 16 chunks: the placement too, one wave per chunk, once the offsets
  // and chunk bases written above are visible to every wave and every wave's
  // reads of the masks are done.
  if (n_chunks <= kScanScatterChunks) {
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    if (wave < n_chunks) scatter_chunk(p, wave, threadIdx.x & 63);
  }
}

__global__ __launch_bounds__(64) void sort_scatter_kernel(SortParams p) {
  scatter_chunk(p, blockIdx.x, threadIdx.x);
}

// Zero n 64-bit words (the chunk masks after an interrupted call). A kernel
// rather than a memset, so that a forward captured into a HIP graph holds no
// memset node.
__global__ __launch_bounds__(256) void clear_u64_kernel(uint64_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

}  // namespace

hipError_t launch_clear_u64(uint64_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  hipLaunchKernelGGL(clear_u64_kernel, dim3((int)(want < 1024 ? want : 1024)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       uint64_t* chunk_masks, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((T + kTopkWaves - 1) / kTopkWaves), dim3(kTopkWaves * 64), 0, s,
                     logits, T, E, k, ids, w, chunk_masks);
  return hipGetLastError();
}

hipError_t launch_sort(const SortParams& p, hipStream_t s) {
  const int n_chunks = (p.T + kChunk - 1) / kChunk;
  if (n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(1024), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_chunks <= kScanScatterChunks) return err;
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(n_chunks), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace lmoe
