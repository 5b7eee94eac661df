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

namespace lmoe {

namespace {

constexpr int kChunk = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / kWave;  // 16

// Wave-wide maximum with DPP moves (no LDS round trip): butterflies inside
// quads, half-rows and rows of 16 lanes, then row broadcasts carry each row's
// maximum upward; lane 63 ends with the wave's maximum.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x140, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One wave per token (4 per workgroup), so that even a decode-sized batch
// spreads over the GPU: k rounds of a wave arg-max, each on the lanes' best
// untaken logits (lowest index on ties) with the wave maximum from wave_max and
// the winner the lowest index among the lanes holding it (usually one lane).
// The token's bit goes into its chunk's mask of each selected expert with a
// global atomic OR, which gives the same masks in any order.
//
// Non-finite logits: NaN scores as -inf, and a lane offers its first untaken
// slot even when every untaken score it holds is -inf. Since k <= E, some
// valid slot is untaken in each round, so some lane has an offer, the ballot
// is never empty and every round selects a valid, distinct expert (with ties,
// -inf ones included, going to the lower index). Weights: the softmax of the
// selected scores; when the largest one is infinite (all selected -inf, or some
// +inf), equal shares among the slots holding it, the softmax's limit.
constexpr int kTopkWaves = 4;

__global__ __launch_bounds__(kTopkWaves * 64) void topk_kernel(const float* __restrict__ logits, int T,
                                                               int E, int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ w,
                                                               uint64_t* __restrict__ chunk_masks) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t >= T) return;                        // whole waves
  const int per = (E + kWave - 1) / kWave;
  float v[kMaxPerLane];
  unsigned taken = 0;
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int e = q * kWave + lane;
    const bool ok = q < per && e < E;
    // unconditional load from a clamped (valid) address, masked afterwards
    const float x = logits[(int64_t)t * E + (e < E ? e : E - 1)];
    v[q] = (!ok || x != x) ? -INFINITY : x;
    if (!ok) taken |= 1u << q;               // slots past E are never offered
  }
  float sel_v = 0.f, top = 0.f, den = 0.f;
  int n_top = 0;                             // selected slots whose score equals the first
  int my_id = 0;                             // lane j < k keeps the j-th selected expert
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;                     // no offer yet
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q)
      // ascending q: the first untaken slot is always offered, later ones only
      // if strictly larger, so ties keep the lower index
      if (!(taken >> q & 1u) && (bi == 0x7FFFFFFF || v[q] > bv)) {
        bv = v[q];
        bi = q * kWave + lane;
      }
    const float vmax = wave_max(bv);
    const uint64_t tie = __ballot(bi != 0x7FFFFFFF && bv == vmax);   // never empty (see above)
    int win;
    if (__popcll(tie) == 1) {
      win = __builtin_amdgcn_readlane(bi, __ffsll((unsigned long long)tie) - 1);
    } else {                                   // several lanes hold the maximum
      win = 0x7FFFFFFF;
      for (uint64_t m = tie; m; m &= m - 1) {
        const int l = __ffsll((unsigned long long)m) - 1;
        const int c = __builtin_amdgcn_readlane(bi, l);
        win = c < win ? c : win;
      }
    }
    if ((win & 63) == lane) taken |= 1u << (win >> 6);
    if (j == 0) top = vmax;
    den += expf(vmax - top);
    n_top += vmax == top;
    if (lane == j) {
      my_id = win;
      sel_v = vmax;
    }
  }
  if (lane < k) {
    const float wj = isinf(top) ? (sel_v == top ? 1.f / (float)n_top : 0.f) : expf(sel_v - top) / den;
    ids[(int64_t)t * k + lane] = my_id;
    w[(int64_t)t * k + lane] = wj;
    atomicOr(reinterpret_cast<unsigned long long*>(chunk_masks) + (int64_t)(t / kChunk) * E + my_id,
             1ull << (t % kChunk));
  }
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
  const int nt = (head && cnt > p.small_max) ? (cnt + p.tile_m - 1) / p.tile_m : 0;
  const int tbase = block_exclusive_scan(nt, wave_tot, &total);
  for (int i = 0; i < nt; ++i) {
    p.tiles[2 * (tbase + i)] = e;
    p.tiles[2 * (tbase + i) + 1] = off + i * p.tile_m;
  }
  if (threadIdx.x == 0) *p.n_tiles = total;
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
  const int mbase = block_exclusive_scan(nt2, wave_tot, &total);
  if (head) p.mt_off[e] = mbase;
  if (threadIdx.x == 0) p.mt_off[p.E] = total;
}

__global__ __launch_bounds__(64) void sort_scatter_kernel(SortParams p) {
  const int chunk = blockIdx.x, lane = threadIdx.x;
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
  // The chunk's masks are read only here (after the scan): clear them for the
  // next call's atomic ORs, once every lane has read its own.
  __syncthreads();
  for (int e = lane; e < p.E; e += kChunk) p.chunk_masks[(int64_t)chunk * p.E + e] = 0ull;
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
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(n_chunks), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace lmoe
