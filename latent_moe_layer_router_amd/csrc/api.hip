// C ABI of the latent-MoE block (include/lmoe.h): argument checks, the
// workspace plan and the launch sequence of one forward pass on one stream.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/lmoe.h"
#include "kernels.h"

using namespace lmoe;

namespace {

thread_local std::string g_last_error;

lmoe_status fail(lmoe_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Byte layout of the workspace for a configuration (every region 256-byte aligned).
struct Plan {
  size_t P, logits, ids, w, masks, chunk_base, counts, offsets, sorted_assign, inv,
      row_tok, tiles, n_tiles, mt_off, stream_items, n_stream, queue, xp, H, xq, xs, hq, hs, Y, ss,
      u, part;
  size_t total;
  int max_slots;
};

size_t grow(size_t& cur, size_t bytes) {
  const size_t at = cur;
  cur += (bytes + 255) & ~size_t(255);
  return at;
}

int slots_for(int64_t T, int k, int E) {
  const int64_t A = T * k;
  return (int)((A + kGemmBM - 1) / kGemmBM + (A < E ? A : E));
}

Plan make_plan(const lmoe_config& c) {
  Plan p{};
  const int64_t Tm = c.max_tokens, k = c.top_k, E = c.n_experts, Dp = c.d_pooled, F = c.d_ff;
  const int64_t A = Tm * k;
  const int64_t es = c.act_dtype == LMOE_BF16 ? 2 : 4;
  const int64_t n_chunks = (Tm + 63) / 64;
  p.max_slots = slots_for(Tm, (int)k, (int)E);
  size_t cur = 0;
  p.P = grow(cur, Tm * Dp * 4);
  p.logits = grow(cur, Tm * E * 4);
  p.ids = grow(cur, A * 4);
  p.w = grow(cur, A * 4);
  p.masks = grow(cur, n_chunks * E * 8);
  p.chunk_base = grow(cur, n_chunks * E * 4);
  p.counts = grow(cur, E * 4);
  p.offsets = grow(cur, (E + 1) * 4);
  p.sorted_assign = grow(cur, A * 4);
  p.inv = grow(cur, A * 4);
  p.row_tok = grow(cur, A * 4);
  p.tiles = grow(cur, (size_t)p.max_slots * 8);
  p.n_tiles = grow(cur, 4);
  p.mt_off = grow(cur, (E + 1) * 4);
  p.stream_items = grow(cur, E * 4);
  p.n_stream = grow(cur, 4);
  p.queue = grow(cur, 4);
  // Expert inputs: xp one row per token (the gate/up GEMMs gather it through
  // row_tok), H one row per assignment in sorted (expert-major) order; bf16/fp32,
  // or (MXFP4 experts) MXFP8 codes and scales.
  const bool mx = c.expert_wdtype == LMOE_MXFP4;
  p.xp = grow(cur, mx ? 0 : Tm * Dp * es);
  p.H = grow(cur, mx ? 0 : A * F * es);
  p.xq = grow(cur, mx ? Tm * Dp : 0);
  p.xs = grow(cur, mx ? Tm * Dp / 32 : 0);
  p.hq = grow(cur, mx ? A * F : 0);
  p.hs = grow(cur, mx ? A * F / 32 : 0);
  p.Y = grow(cur, A * Dp * es);
  p.ss = grow(cur, A * (Dp / 64) * 4);
  p.u = grow(cur, Tm * Dp * es);
  // split-K partials of the small-batch dense projections (bf16, T <= 128)
  int64_t part = 0;
  if (c.act_dtype == LMOE_BF16) {
    const int64_t Ts = Tm < dense_stream_max_tokens() ? Tm : dense_stream_max_tokens();
    const int64_t a = dense_stream_part_floats((int)Ts, Dp + E, c.d_model);
    const int64_t b = dense_stream_part_floats((int)Ts, c.d_model, c.d_pooled);
    part = (a > b ? a : b) * 4;
  }
  p.part = grow(cur, part);
  p.total = cur;
  return p;
}

lmoe_status check_config(const lmoe_config* c) {
  if (!c) return fail(LMOE_E_INVAL, "config is NULL");
  if (c->abi_version != LMOE_ABI_VERSION)
    return fail(LMOE_E_INVAL, "abi_version " + std::to_string(c->abi_version) + " != " +
                                  std::to_string(LMOE_ABI_VERSION));
  if (c->d_model <= 0 || c->d_pooled <= 0 || c->d_ff <= 0 || c->d_model % 64 || c->d_pooled % 64 ||
      c->d_ff % 64)
    return fail(LMOE_E_UNSUPPORTED, "d_model, d_pooled and d_ff must be positive multiples of 64");
  if (c->n_experts < 1 || c->n_experts > 1024)
    return fail(LMOE_E_UNSUPPORTED, "n_experts must be in [1, 1024]");
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts)
    return fail(LMOE_E_UNSUPPORTED, "top_k must be in [1, min(n_experts, 16)]");
  if (!(c->eps_pool >= 0.f) || !(c->eps_expert >= 0.f) || c->eps_pool > 1e30f || c->eps_expert > 1e30f)
    return fail(LMOE_E_INVAL, "eps_pool and eps_expert must be finite and >= 0");
  if (c->act_dtype != LMOE_F32 && c->act_dtype != LMOE_BF16)
    return fail(LMOE_E_UNSUPPORTED, "act_dtype must be LMOE_F32 or LMOE_BF16");
  if (c->expert_wdtype == LMOE_MXFP4) {
    // MXFP4 experts: bf16 activations elsewhere, MXFP8 expert inputs, the
    // block-scaled tiled GEMM (K a multiple of 1024, 32-bit byte offsets).
    if (c->act_dtype != LMOE_BF16)
      return fail(LMOE_E_UNSUPPORTED, "MXFP4 experts need act_dtype LMOE_BF16");
    if (c->d_pooled % 1024 || c->d_ff % 1024)
      return fail(LMOE_E_UNSUPPORTED, "MXFP4 experts need d_pooled and d_ff multiples of 1024");
    const int64_t A = (int64_t)c->max_tokens * c->top_k;
    if (A * c->d_ff >= ((int64_t)1 << 31) || A * c->d_pooled >= ((int64_t)1 << 31) ||
        (int64_t)c->d_ff * c->d_pooled >= ((int64_t)1 << 31))
      return fail(LMOE_E_UNSUPPORTED, "MXFP4 experts: max_tokens too large for 32-bit offsets");
  } else if (c->expert_wdtype != c->act_dtype) {
    return fail(LMOE_E_UNSUPPORTED, "expert_wdtype must be act_dtype or LMOE_MXFP4");
  }
  if (c->out_dtype != LMOE_F32 && c->out_dtype != c->act_dtype)
    return fail(LMOE_E_UNSUPPORTED, "out_dtype must be LMOE_F32 or act_dtype");
  if (c->max_tokens < 1) return fail(LMOE_E_INVAL, "max_tokens must be >= 1");
  if ((int64_t)c->max_tokens * c->top_k > (int64_t)INT32_MAX / 2 ||
      (int64_t)c->max_tokens * c->top_k * c->d_ff > (int64_t)1 << 40)
    return fail(LMOE_E_UNSUPPORTED, "max_tokens too large");
  if (c->flags & ~(LMOE_FLAG_ROUTER_BIAS | LMOE_FLAG_PACKED_EXPERTS)) return fail(LMOE_E_INVAL, "unknown flag bits");
  if (c->flags & LMOE_FLAG_PACKED_EXPERTS) {
    // Every expert GEMM must then run on the kernels that read the packed
    // layout (the weight-streaming ones and the tiled grouped GEMM) at every T.
    const int64_t A = (int64_t)c->max_tokens * c->top_k;
    if (c->act_dtype != LMOE_BF16 || c->expert_wdtype != LMOE_BF16 || c->d_pooled % 256 || c->d_ff % 128 ||
        A * c->d_ff * 2 >= ((int64_t)1 << 31) || A * c->d_pooled * 2 >= ((int64_t)1 << 31) ||
        (int64_t)4 * c->d_ff * c->d_pooled >= ((int64_t)1 << 31))
      return fail(LMOE_E_UNSUPPORTED,
                  "packed expert weights need bf16 activations and experts, d_pooled a multiple of 256, d_ff a "
                  "multiple of 128 and 32-bit byte offsets at max_tokens");
  }
  return LMOE_OK;
}

// Checks of one forward call's arguments against its configuration (before
// anything is enqueued).
lmoe_status check_forward_args(const lmoe_config& c, const void* x, void* out, int32_t T,
                               const lmoe_aux* aux) {
  if (T < 0 || T > c.max_tokens)
    return fail(LMOE_E_INVAL, "T = " + std::to_string(T) + " outside [0, max_tokens = " +
                                  std::to_string(c.max_tokens) + "]");
  if (T == 0) return LMOE_OK;
  if (!x || !out) return fail(LMOE_E_INVAL, "x or out is NULL");
  if (!aligned16(x) || !aligned16(out)) return fail(LMOE_E_INVAL, "x or out is not 16-byte aligned");
  const bool bf16 = c.act_dtype == LMOE_BF16;
  const bool out_f32 = c.out_dtype == LMOE_F32;
  const size_t x_bytes = (size_t)T * c.d_model * (bf16 ? 2 : 4);
  const size_t o_bytes = (size_t)T * c.d_model * (out_f32 ? 4 : 2);
  const uintptr_t xb = reinterpret_cast<uintptr_t>(x), ob = reinterpret_cast<uintptr_t>(out);
  if (xb < ob + o_bytes && ob < xb + x_bytes) return fail(LMOE_E_INVAL, "out overlaps x");
  if (aux) {
    const void* ap[] = {aux->logits, aux->topk_ids, aux->topk_w, aux->expert_offsets, aux->sorted_assign};
    for (const void* q : ap)
      if (q && !aligned4(q)) return fail(LMOE_E_INVAL, "aux pointer is not 4-byte aligned");
  }
  return LMOE_OK;
}

// Validation of the weight pointers against a configuration.
lmoe_status check_weights(const lmoe_config* cfg, const lmoe_weights* w) {
  if (!w) return fail(LMOE_E_INVAL, "weights is NULL");
  const void* req[] = {w->w_router, w->w_pool, w->g_pool, w->w_gate_up, w->w_down, w->g_expert,
                       w->w_unpool};
  const char* names[] = {"w_router", "w_pool", "g_pool", "w_gate_up", "w_down", "g_expert", "w_unpool"};
  for (int i = 0; i < 7; ++i) {
    if (!req[i]) return fail(LMOE_E_INVAL, std::string(names[i]) + " is NULL");
    if (!aligned16(req[i])) return fail(LMOE_E_INVAL, std::string(names[i]) + " is not 16-byte aligned");
  }
  const bool has_bias = (cfg->flags & LMOE_FLAG_ROUTER_BIAS) != 0;
  if (has_bias != (w->b_router != nullptr))
    return fail(LMOE_E_INVAL, "b_router must be given iff LMOE_FLAG_ROUTER_BIAS is set");
  if (w->b_router && !aligned4(w->b_router)) return fail(LMOE_E_INVAL, "b_router is misaligned");
  if (cfg->expert_wdtype == LMOE_MXFP4) {
    if (!w->s_gate_up || !w->s_down) return fail(LMOE_E_INVAL, "MXFP4 experts need s_gate_up and s_down");
    if (!aligned16(w->s_gate_up) || !aligned16(w->s_down))
      return fail(LMOE_E_INVAL, "s_gate_up / s_down are not 16-byte aligned");
  } else if (w->s_gate_up || w->s_down) {
    return fail(LMOE_E_INVAL, "MX scale pointers must be NULL unless expert_wdtype is LMOE_MXFP4");
  }

  return LMOE_OK;
}

// The fused expert kernel runs the streamed experts (1..64 rows each) whole,
// one per workgroup, when there are at least this many of them (counted on
// the device); otherwise the single-wave weight-streaming launches run them.
// Each whole expert gets one compute unit, so that needs about as many
// streamed experts as compute units (3/4 of them). The environment variable
// LMOE_FUSED_EXPERTS = 1 (always whole experts) or 0 (never) overrides it.
constexpr int kAllStreamedT = 128;

int fused_whole_min(int n_cu) {
  const char* env = getenv("LMOE_FUSED_EXPERTS");
  if (env && env[0] == '1') return 0;
  if (env && env[0] == '0') return INT32_MAX;
  return (3 * n_cu + 3) / 4;
}

// The launch sequence of one forward pass on stream s, over the workspace ws
// laid out by pl (sized for at least T tokens). Arguments are already checked.
// masks_dirty: whether the chunk masks may hold bits (they are cleared first
// then); it is left true only if the call stopped between the top-k and the
// sort. ev: null, or LMOE_NUM_STAGES + 1 created events recorded around the
// stages. Returns the first failed launch's error (nothing more is enqueued
// after it).
hipError_t enqueue_forward(const lmoe_config& c, const lmoe_weights& W, const Plan& pl, unsigned char* ws,
                           int n_cu, bool& masks_dirty, hipEvent_t* ev, const void* x, void* out,
                           int32_t T, hipStream_t s, const lmoe_aux* aux) {
  const bool bf16 = c.act_dtype == LMOE_BF16;
  const bool out_f32 = c.out_dtype == LMOE_F32;
  // expert weights in the packed layout (create checked that only the
  // weight-streaming and tiled grouped kernels run the expert GEMMs then)
  const int packed = (c.flags & LMOE_FLAG_PACKED_EXPERTS) ? 1 : 0;
  const int E = c.n_experts, k = c.top_k, D = c.d_model, Dp = c.d_pooled, F = c.d_ff;
  float* P = reinterpret_cast<float*>(ws + pl.P);
  float* logits = (aux && aux->logits) ? aux->logits : reinterpret_cast<float*>(ws + pl.logits);
  int32_t* ids = (aux && aux->topk_ids) ? aux->topk_ids : reinterpret_cast<int32_t*>(ws + pl.ids);
  float* tw = (aux && aux->topk_w) ? aux->topk_w : reinterpret_cast<float*>(ws + pl.w);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + pl.offsets);
  int32_t* sorted_assign = reinterpret_cast<int32_t*>(ws + pl.sorted_assign);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + pl.tiles);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(ws + pl.n_tiles);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + pl.inv);
  int32_t* row_tok = reinterpret_cast<int32_t*>(ws + pl.row_tok);
  void* xp = ws + pl.xp;
  void* H = ws + pl.H;
  uint8_t* xq = ws + pl.xq;
  uint8_t* xs = ws + pl.xs;
  uint8_t* hq = ws + pl.hq;
  uint8_t* hs = ws + pl.hs;
  const bool mx = c.expert_wdtype == LMOE_MXFP4;
  void* Y = ws + pl.Y;
  float* ss = reinterpret_cast<float*>(ws + pl.ss);
  void* u = ws + pl.u;
  const int slots = slots_for(T, k, E);
  // Experts with few rows go to the weight-streaming kernels (bf16, K multiple of 128).
  // The grouped kernels' buffer loads take 32-bit byte offsets: the activations
  // (xp, H) and one expert's weights must each stay below 2 GiB.
  const bool off32_ok = (int64_t)T * k * F * 2 < ((int64_t)1 << 31) &&
                        (int64_t)T * k * Dp * 2 < ((int64_t)1 << 31) &&
                        (int64_t)2 * F * Dp * 2 < ((int64_t)1 << 31);
  const bool stream_ok = bf16 && !mx && Dp % 128 == 0 && F % 128 == 0 && off32_ok;
  // The fused expert kernel (Dp a multiple of 256: whole groups of 4 waves),
  // launched when the streamed experts may reach its threshold (there are at
  // most T k of them); it and the single-wave launches then decide on the
  // device which of them runs.
  const int whole_min = fused_whole_min(n_cu);
  const bool fused = stream_ok && Dp % 256 == 0 && (int64_t)T * k >= whole_min;
  // MXFP4 experts: the create-time checks (Dp and F multiples of 1024, 32-bit
  // byte extents) are all the MX weight-streaming kernel needs.
  // A batch of at most kAllStreamedT tokens gives no expert more than that many
  // rows (the k experts of a token are distinct); then the weight-streaming
  // kernels take every expert, in passes of their row limit, and the tiled
  // kernels are not launched (their launches cost more than the rare extra
  // pass over an expert's weights).
  const int pass_rows = stream_ok ? stream_max_rows() : (mx ? stream_mx_max_rows() : 0);
  const int small_max = pass_rows > 0 && T <= kAllStreamedT ? kAllStreamedT : pass_rows;
  const bool tiled = T > small_max;
  // Experts with many rows: the tiled grouped GEMM (bf16, Dp % 256 == 0, F % 128 == 0).
  const bool big_ok = bf16 && !mx && Dp % 256 == 0 && F % 128 == 0 && off32_ok;
  int32_t* mt_off = reinterpret_cast<int32_t*>(ws + pl.mt_off);
  const int64_t A_ = (int64_t)T * k;
  // Row tiles (at least 256 rows each) over the experts with more than small_max rows: at most
  // floor(A / 256) full ones plus one partial per such expert, and there are at
  // most floor(A / (small_max + 1)) such experts. The bound sizes the grid, so a
  // tight one keeps the launch cheap when few or no experts are large (decode).
  const int64_t n_big = A_ / (small_max + 1) < E ? A_ / (small_max + 1) : E;
  const int mtiles_bound = (int)(A_ / 256 + n_big);

  int stage = 0;
  auto mark = [&]() {
    if (ev) (void)hipEventRecord(ev[stage], s);
    ++stage;
  };

  // After the first failed launch nothing more is enqueued (later kernels would
  // read tile lists and offsets that were never written).
  hipError_t err = hipSuccess;
#define run(X)                    \
  do {                            \
    if (err == hipSuccess) err = (X); \
  } while (0)

  // Small batches: the dense projections stream their weights with split-K.
  const bool dense_stream = bf16 && T <= dense_stream_max_tokens();
  float* part = reinterpret_cast<float*>(ws + pl.part);
  const int slices_in = dense_stream_slices(Dp + E, D), slices_un = dense_stream_slices(D, Dp);

  // Larger batches: the dense projections on the tiled kernel (bf16; K a
  // multiple of 128, the pooler's rows a multiple of 256, 32-bit offsets).
  const bool dense256 = bf16 && !dense_stream && D % 128 == 0 && Dp % 256 == 0 &&
                        (int64_t)T * D * 2 < ((int64_t)1 << 31) && (int64_t)T * Dp * 2 < ((int64_t)1 << 31) &&
                        (int64_t)256 * D * 2 < ((int64_t)1 << 31);
  auto dense_params = [&](const void* A, int K, int N) {
    GroupedParams g{};
    g.A = A;
    g.lda = K;
    g.ldb = K;
    g.K = K;
    g.M = T;
    g.N = N;
    g.ntiles_n = (N + 255) / 256;
    g.ntiles_m = gemm_grouped_dense_row_tiles(T, g.ntiles_n, n_cu);
    g.max_tiles = g.ntiles_n * g.ntiles_m;
    g.a_bytes = (uint32_t)((int64_t)T * K * 2);
    return g;
  };

  // The top-k ORs into the chunk masks and the sort clears them; if a previous
  // call stopped between the two, they are cleared before the top-k.
  uint64_t* masks = reinterpret_cast<uint64_t*>(ws + pl.masks);

  // 1. router + pooler: one GEMM over [W_pool; W_router]
  mark();
  bool pooled = false;
  if (dense256) {
    GroupedParams g = dense_params(x, D, Dp + E);
    g.B = W.w_pool;
    g.B1 = W.w_router;
    g.n_split = Dp;
    g.out = P;
    g.ldo = Dp;
    g.out1 = logits;
    g.ldo1 = E;
    g.bias1 = W.b_router;
    run(launch_gemm_grouped(g, EPI_F32, n_cu, s));
  } else if (dense_stream && slices_in > 0) {
    DenseStreamParams d{};
    d.A = x;
    d.lda = D;
    d.B0 = W.w_pool;
    d.B1 = W.w_router;
    d.n_split = Dp;
    d.ldb = D;
    d.T = T;
    d.N = Dp + E;
    d.K = D;
    d.slices = slices_in;
    d.part = part;
    d.out0 = P;
    d.ldo0 = Dp;
    d.out1 = logits;
    d.ldo1 = E;
    d.bias1 = W.b_router;
    // the split-K reduction, the pooled RMSNorm and the MXFP8 quantization of
    // xp (one row per token, so it needs no routing) and the top-k in one pass
    run(launch_dense_stream_partials(d, s));
    if (masks_dirty) {
      run(launch_clear_u64(masks, (int64_t)(pl.chunk_base - pl.masks) / 8, s));
      if (err == hipSuccess) masks_dirty = false;
    }
    const TopkOut tk{ids, tw, masks, k};
    run(launch_splitk_pool_norm(d, W.g_pool, c.eps_pool, mx ? static_cast<void*>(xq) : xp, mx ? 2 : 0, xs, tk, s));
    if (err == hipSuccess) masks_dirty = true;
    pooled = true;
  } else {
    GemmParams g{};
    g.M = T;
    g.N = Dp + E;
    g.K = D;
    g.A = x;
    g.lda = D;
    g.B0 = W.w_pool;
    g.B1 = W.w_router;
    g.n_split = Dp;
    g.ldb = D;
    g.out0 = P;
    g.ldo0 = Dp;
    g.out1 = logits;
    g.ldo1 = E;
    g.bias1 = W.b_router;
    run(launch_gemm(g, EPI_F32, bf16, s));
  }
  // 2. top-k + softmax + chunk masks (done above with the small-batch reduction)
  mark();
  if (!pooled) {
    if (masks_dirty) {
      run(launch_clear_u64(masks, (int64_t)(pl.chunk_base - pl.masks) / 8, s));
      if (err == hipSuccess) masks_dirty = false;
    }
    run(launch_topk(logits, T, E, k, ids, tw, masks, s));
    if (err == hipSuccess) masks_dirty = true;
  }
  // 3. counting sort + tile list
  mark();
  {
    SortParams sp{};
    sp.ids = ids;
    sp.topk_w = tw;
    sp.chunk_masks = masks;
    sp.chunk_base = reinterpret_cast<int32_t*>(ws + pl.chunk_base);
    sp.counts = reinterpret_cast<int32_t*>(ws + pl.counts);
    sp.offsets = offsets;
    sp.sorted_assign = sorted_assign;
    sp.inv = inv;
    sp.row_tok = row_tok;
    sp.tiles = tiles;
    sp.n_tiles = n_tiles;
    sp.T = T;
    sp.E = E;
    sp.k = k;
    sp.tile_m = kGemmBM;
    sp.small_max = small_max;
    sp.mt_off = mt_off;
    sp.tile_m2 = mx ? gemm_grouped_mx_tile_m() : gemm_grouped_tile_m();
    if (fused) {
      sp.stream_items = reinterpret_cast<int32_t*>(ws + pl.stream_items);
      sp.n_stream = reinterpret_cast<int32_t*>(ws + pl.n_stream);
      sp.queue = reinterpret_cast<int32_t*>(ws + pl.queue);
    }
    run(launch_sort(sp, s));
    if (err == hipSuccess) masks_dirty = false;
  }
  // 4. pooled RMSNorm (already done with the small-batch reduction)
  mark();
  if (pooled) {
  } else if (mx) {
    run(launch_pool_norm_mx(P, W.g_pool, T, Dp, c.eps_pool, xq, xs, s));
  } else {
    run(launch_pool_norm(P, W.g_pool, T, Dp, c.eps_pool, xp, bf16, s));
  }
  // 5. gate/up grouped GEMM + SwiGLU (with the fused kernel: both streamed GEMMs)
  mark();
  StreamParams sp_down{};
  if (stream_ok) {
    sp_down.A = H;
    sp_down.lda = F;
    sp_down.B = W.w_down;
    sp_down.ldb = F;
    sp_down.b_expert_stride = (int64_t)Dp * F;
    sp_down.b_packed = packed;
    sp_down.offsets = offsets;
    sp_down.n_experts = E;
    sp_down.groups = Dp / 64;
    sp_down.max_rows = small_max;
    sp_down.K = F;
    sp_down.F = F;
    sp_down.a_bytes = (uint32_t)(A_ * F * 2);
    sp_down.b_bytes = (uint32_t)((int64_t)Dp * F * 2);
    sp_down.out = Y;
    sp_down.ldo = Dp;
    sp_down.ss_out = ss;
    sp_down.ss_ld = Dp / 64;
    if (fused) {
      sp_down.fused_n = reinterpret_cast<const int32_t*>(ws + pl.n_stream);
      sp_down.whole_min = whole_min;
    }
  }
  if (stream_ok) {
    StreamParams sp{};
    sp.A = xp;
    sp.lda = Dp;
    sp.a_rows = row_tok;
    sp.B = W.w_gate_up;
    sp.ldb = Dp;
    sp.b_expert_stride = (int64_t)2 * F * Dp;
    sp.b_packed = packed;
    sp.offsets = offsets;
    sp.n_experts = E;
    sp.groups = F / 32;
    sp.max_rows = small_max;
    sp.K = Dp;
    sp.F = F;
    sp.a_bytes = (uint32_t)((int64_t)T * Dp * 2);
    sp.b_bytes = (uint32_t)((int64_t)2 * F * Dp * 2);
    sp.out = H;
    sp.ldo = F;
    if (fused) {
      FusedStreamParams f{};
      f.gu = sp;
      f.dn = sp_down;
      f.items = reinterpret_cast<const int32_t*>(ws + pl.stream_items);
      f.n_items = reinterpret_cast<const int32_t*>(ws + pl.n_stream);
      f.queue = reinterpret_cast<int32_t*>(ws + pl.queue);
      f.whole_min = whole_min;
      run(launch_fused_stream(f, n_cu, s));
      sp.fused_n = f.n_items;
      sp.whole_min = whole_min;
    }
    run(launch_stream(sp, EPI_SWIGLU, s));
  }
  if (mx) {
    StreamMxParams sp{};
    sp.A = xq;
    sp.As = xs;
    sp.a_rows = row_tok;
    sp.B = static_cast<const uint8_t*>(W.w_gate_up);
    sp.Bs = W.s_gate_up;
    sp.N = 2 * F;
    sp.offsets = offsets;
    sp.n_experts = E;
    sp.groups = F / 32;
    sp.max_rows = small_max;
    sp.K = Dp;
    sp.F = F;
    sp.a_bytes = (uint32_t)((int64_t)T * Dp);
    sp.as_bytes = (uint32_t)((int64_t)T * Dp / 32);
    sp.b_bytes = (uint32_t)((int64_t)F * Dp);
    sp.bs_bytes = (uint32_t)((int64_t)2 * F * Dp / 32);
    sp.out = hq;
    sp.ldo = F;
    sp.out_scales = hs;
    sp.ldos = F / 32;
    run(launch_stream_mx(sp, EPI_SWIGLU, s));
  }
  if (mx && !tiled) {
  } else if (mx) {
    GroupedMxParams g{};
    g.A = xq;
    g.As = xs;
    g.a_rows = row_tok;
    g.B = static_cast<const uint8_t*>(W.w_gate_up);
    g.Bs = W.s_gate_up;
    g.N = 2 * F;
    g.offsets = offsets;
    g.mt_off = mt_off;
    g.E = E;
    g.ntiles_n = F / 128;
    g.max_tiles = g.ntiles_n * mtiles_bound;
    g.a_bytes = (uint32_t)((int64_t)T * Dp);
    g.as_bytes = (uint32_t)((int64_t)T * Dp / 32);
    g.K = Dp;
    g.F = F;
    g.out = hq;
    g.ldo = F;
    g.out_scales = hs;
    g.ldos = F / 32;
    run(launch_gemm_grouped_mx(g, EPI_SWIGLU, s));
  } else if (big_ok) {
    GroupedParams g{};
    g.A = xp;
    g.lda = Dp;
    g.a_rows = row_tok;
    g.B = W.w_gate_up;
    g.ldb = Dp;
    g.b_expert_stride = (int64_t)2 * F * Dp;
    g.b_packed = packed;
    g.offsets = offsets;
    g.mt_off = mt_off;
    g.E = E;
    g.ntiles_n = F / 128;
    g.max_tiles = g.ntiles_n * mtiles_bound;
    g.a_bytes = (uint32_t)((int64_t)T * Dp * 2);
    g.b_bytes = (uint32_t)((int64_t)2 * F * Dp * 2);
    g.K = Dp;
    g.F = F;
    g.out = H;
    g.ldo = F;
    if (tiled) run(launch_gemm_grouped(g, EPI_SWIGLU, n_cu, s));
  } else {
    GemmParams g{};
    g.N = F;
    g.K = Dp;
    g.A = xp;
    g.lda = Dp;
    g.a_rows = row_tok;
    g.B0 = W.w_gate_up;
    g.ldb = Dp;
    g.b_expert_stride = (int64_t)2 * F * Dp;
    g.tiles = tiles;
    g.n_tiles = n_tiles;
    g.offsets = offsets;
    g.max_slots = slots;
    g.out0 = H;
    g.ldo0 = F;
    g.F = F;
    run(launch_gemm(g, EPI_SWIGLU, bf16, s));
  }
  // 6. down grouped GEMM + sum-of-squares partials
  mark();
  if (stream_ok) run(launch_stream(sp_down, EPI_DOWN, s));
  if (mx) {
    StreamMxParams sp{};
    sp.A = hq;
    sp.As = hs;
    sp.B = static_cast<const uint8_t*>(W.w_down);
    sp.Bs = W.s_down;
    sp.N = Dp;
    sp.offsets = offsets;
    sp.n_experts = E;
    sp.groups = Dp / 64;
    sp.max_rows = small_max;
    sp.K = F;
    sp.F = F;
    sp.a_bytes = (uint32_t)(A_ * F);
    sp.as_bytes = (uint32_t)(A_ * F / 32);
    sp.b_bytes = (uint32_t)((int64_t)Dp * F / 2);
    sp.bs_bytes = (uint32_t)((int64_t)Dp * F / 32);
    sp.out = Y;
    sp.ldo = Dp;
    sp.ss_out = ss;
    sp.ss_ld = Dp / 64;
    run(launch_stream_mx(sp, EPI_DOWN, s));
  }
  if (mx && !tiled) {
  } else if (mx) {
    GroupedMxParams g{};
    g.A = hq;
    g.As = hs;
    g.B = static_cast<const uint8_t*>(W.w_down);
    g.Bs = W.s_down;
    g.N = Dp;
    g.offsets = offsets;
    g.mt_off = mt_off;
    g.E = E;
    g.ntiles_n = Dp / 256;
    g.max_tiles = g.ntiles_n * mtiles_bound;
    g.a_bytes = (uint32_t)(A_ * F);
    g.as_bytes = (uint32_t)(A_ * F / 32);
    g.K = F;
    g.F = F;
    g.out = Y;
    g.ldo = Dp;
    g.ss_out = ss;
    g.ss_ld = Dp / 64;
    run(launch_gemm_grouped_mx(g, EPI_DOWN, s));
  } else if (big_ok) {
    GroupedParams g{};
    g.A = H;
    g.lda = F;
    g.B = W.w_down;
    g.ldb = F;
    g.b_expert_stride = (int64_t)Dp * F;
    g.b_packed = packed;
    g.offsets = offsets;
    g.mt_off = mt_off;
    g.E = E;
    g.ntiles_n = Dp / 256;
    g.max_tiles = g.ntiles_n * mtiles_bound;
    g.a_bytes = (uint32_t)(A_ * F * 2);
    g.b_bytes = (uint32_t)((int64_t)Dp * F * 2);
    g.K = F;
    g.F = F;
    g.out = Y;
    g.ldo = Dp;
    g.ss_out = ss;
    g.ss_ld = Dp / 64;
    if (tiled) run(launch_gemm_grouped(g, EPI_DOWN, n_cu, s));
  } else {
    GemmParams g{};
    g.N = Dp;
    g.K = F;
    g.A = H;
    g.lda = F;
    g.B0 = W.w_down;
    g.ldb = F;
    g.b_expert_stride = (int64_t)Dp * F;
    g.tiles = tiles;
    g.n_tiles = n_tiles;
    g.offsets = offsets;
    g.max_slots = slots;
    g.out0 = Y;
    g.ldo0 = Dp;
    g.ss_out = ss;
    g.ss_ld = Dp / 64;
    run(launch_gemm(g, EPI_DOWN, bf16, s));
  }
  // 7. per-expert RMSNorm + weighted sum
  mark();
  {
    CombineParams cp{};
    cp.y = Y;
    cp.ss = ss;
    cp.inv = inv;
    cp.ids = ids;
    cp.w = tw;
    cp.g_expert = W.g_expert;
    cp.u = u;
    cp.T = T;
    cp.k = k;
    cp.Dp = Dp;
    cp.eps = c.eps_expert;
    run(launch_combine(cp, bf16, s));
  }
  // 8. unpooler
  mark();
  if (dense256) {
    GroupedParams g = dense_params(u, Dp, D);
    g.B = W.w_unpool;
    g.B1 = W.w_unpool;
    g.n_split = D;
    g.out = out;
    g.ldo = D;
    run(launch_gemm_grouped(g, out_f32 ? EPI_F32 : EPI_ACT, n_cu, s));
  } else if (dense_stream && slices_un > 0) {
    DenseStreamParams d{};
    d.A = u;
    d.lda = Dp;
    d.B0 = W.w_unpool;
    d.B1 = W.w_unpool;
    d.n_split = D;
    d.ldb = Dp;
    d.T = T;
    d.N = D;
    d.K = Dp;
    d.slices = slices_un;
    d.part = part;
    d.out0 = out;
    d.ldo0 = D;
    d.out0_bf16 = !out_f32;
    run(launch_dense_stream(d, s));
  } else {
    GemmParams g{};
    g.M = T;
    g.N = D;
    g.K = Dp;
    g.A = u;
    g.lda = Dp;
    g.B0 = W.w_unpool;
    g.ldb = Dp;
    g.out0 = out;
    g.ldo0 = D;
    g.n_split = D;                       // EPI_F32: every column goes to out0 as fp32
    run(launch_gemm(g, out_f32 ? EPI_F32 : EPI_ACT, bf16, s));
  }
  mark();
  if (aux && aux->expert_offsets)
    run(hipMemcpyAsync(aux->expert_offsets, offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToDevice, s));
  if (aux && aux->sorted_assign)
    run(hipMemcpyAsync(aux->sorted_assign, sorted_assign, sizeof(int32_t) * (size_t)T * k,
                       hipMemcpyDeviceToDevice, s));
#undef run
  return err;
}

// Scratch of the no-allocation forward (lmoe_forward_noalloc): a file-scope
// array in the code object's static device memory, so that each GPU the
// library runs on holds its own copy from the code object's load until the
// process ends. In host code the array's name is only a stand-in: kernels and
// copies get the device address that hipGetSymbolAddress returns for the
// current device, taken once per device.
static __device__ __align__(256) unsigned char scratch[LMOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct NoallocDevice {
  std::once_flag once;
  unsigned char* ptr = nullptr;   // device address of this device's scratch
  int n_cu = 0;
  hipError_t err = hipSuccess;
};
NoallocDevice g_noalloc[kMaxDevices];

// Set-up on the device that is current: the scratch's device address and the
// compute-unit count, once per device.
NoallocDevice& noalloc_device(int dev) {
  NoallocDevice& d = g_noalloc[dev];
  std::call_once(d.once, [&d, dev]() {
    void* ptr = nullptr;
    d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (d.err != hipSuccess) return;
    d.ptr = static_cast<unsigned char*>(ptr);
    int n = 0;
    d.n_cu = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n
                                                                                                          : 256;
  });
  return d;
}

}  // namespace

struct lmoe_ctx {
  lmoe_config cfg;
  lmoe_weights w;
  int device;
  Plan plan;
  unsigned char* ws;
  bool timing;
  bool masks_dirty;                 // top-k ran without the sort that clears the masks
  int n_cu;                         // compute units of the device
  std::vector<hipEvent_t> events;   // LMOE_NUM_STAGES + 1 per timed forward
  float acc_ms[LMOE_NUM_STAGES];
  int n_timed;
};

extern "C" {

const char* lmoe_status_str(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "LMOE_OK";
    case LMOE_E_INVAL: return "LMOE_E_INVAL: invalid argument";
    case LMOE_E_UNSUPPORTED: return "LMOE_E_UNSUPPORTED: unsupported configuration";
    case LMOE_E_NOMEM: return "LMOE_E_NOMEM: device allocation failed";
    case LMOE_E_HIP: return "LMOE_E_HIP: HIP runtime error";
  }
  return "unknown lmoe_status";
}

const char* lmoe_last_error(void) { return g_last_error.c_str(); }

lmoe_status lmoe_workspace_bytes(const lmoe_config* cfg, size_t* out) {
  if (!out) return fail(LMOE_E_INVAL, "out is NULL");
  lmoe_status st = check_config(cfg);
  if (st != LMOE_OK) return st;
  *out = make_plan(*cfg).total;
  return LMOE_OK;
}

lmoe_status lmoe_mx_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, uint8_t* scales,
                                  void* hip_stream) {
  g_last_error.clear();
  if (n < 0 || n % 32) return fail(LMOE_E_INVAL, "n must be a non-negative multiple of 32");
  if (n == 0) return LMOE_OK;
  if (!x || !codes || !scales) return fail(LMOE_E_INVAL, "x, codes and scales must not be NULL");
  if (!aligned16(x) || !aligned16(codes)) return fail(LMOE_E_INVAL, "x and codes must be 16-byte aligned");
  if (n / 32 > (int64_t)INT32_MAX) return fail(LMOE_E_UNSUPPORTED, "n too large");
  const hipError_t e = launch_mx_quant(x, n, codes, scales, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(LMOE_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return LMOE_OK;
}

lmoe_status lmoe_nvfp4_to_mxfp4(const uint8_t* codes, const uint8_t* scales16, const float* global_scale,
                                int64_t n_mats, int64_t rows, int64_t cols, uint8_t* out_codes,
                                uint8_t* out_scales, void* hip_stream) {
  g_last_error.clear();
  if (n_mats < 0 || rows < 0 || cols < 0 || cols % 32)
    return fail(LMOE_E_INVAL, "n_mats and rows must be >= 0 and cols a non-negative multiple of 32");
  if (n_mats == 0 || rows == 0 || cols == 0) return LMOE_OK;
  if (!codes || !scales16 || !global_scale || !out_codes || !out_scales)
    return fail(LMOE_E_INVAL, "codes, scales16, global_scale, out_codes and out_scales must not be NULL");
  if (!aligned16(codes) || !aligned16(out_codes) || (reinterpret_cast<uintptr_t>(scales16) & 1) ||
      !aligned4(global_scale))
    return fail(LMOE_E_INVAL, "codes and out_codes must be 16-byte, scales16 2-byte, global_scale 4-byte aligned");
  if (rows > INT64_MAX / n_mats || n_mats * rows > INT64_MAX / cols)
    return fail(LMOE_E_INVAL, "size overflow");
  const int64_t nc = n_mats * rows * (cols / 2), n16 = n_mats * rows * (cols / 16),
                n32 = n_mats * rows * (cols / 32);
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
  };
  if (out_codes != codes && overlap(out_codes, nc, codes, nc))
    return fail(LMOE_E_INVAL, "out_codes must be codes itself or not overlap it");
  if (overlap(out_scales, n32, codes, nc) || overlap(out_scales, n32, scales16, n16) ||
      overlap(out_scales, n32, out_codes, nc) || overlap(out_codes, nc, scales16, n16) ||
      overlap(out_scales, n32, global_scale, 4 * n_mats) || overlap(out_codes, nc, global_scale, 4 * n_mats))
    return fail(LMOE_E_INVAL, "outputs overlap the inputs");
  const hipError_t e = launch_nvfp4_to_mxfp4(codes, scales16, global_scale, n_mats, rows, cols, out_codes,
                                             out_scales, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(LMOE_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return LMOE_OK;
}

lmoe_status lmoe_pack_experts(const void* src, void* dst, int64_t n_mats, int64_t rows, int64_t cols,
                              void* hip_stream) {
  g_last_error.clear();
  if (n_mats < 0 || rows < 0 || cols < 0 || rows % 64 || cols % 64)
    return fail(LMOE_E_INVAL, "n_mats must be >= 0, rows and cols non-negative multiples of 64");
  if (n_mats == 0 || rows == 0 || cols == 0) return LMOE_OK;
  if (!src || !dst) return fail(LMOE_E_INVAL, "src and dst must not be NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(LMOE_E_INVAL, "src and dst must be 16-byte aligned");
  if (rows > INT32_MAX || cols > INT32_MAX || rows > INT64_MAX / n_mats || n_mats * rows > INT64_MAX / (2 * cols))
    return fail(LMOE_E_INVAL, "size overflow");
  const int64_t bytes = n_mats * rows * cols * 2;
  const uintptr_t x = reinterpret_cast<uintptr_t>(src), y = reinterpret_cast<uintptr_t>(dst);
  if (x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes) return fail(LMOE_E_INVAL, "src and dst overlap");
  const hipError_t e = launch_pack_experts(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), n_mats,
                                           (int)rows, (int)cols, static_cast<hipStream_t>(hip_stream));
  if (e == hipErrorInvalidValue) return fail(LMOE_E_INVAL, "too many 64 x 64 blocks for one launch");
  if (e != hipSuccess) return fail(LMOE_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return LMOE_OK;
}

lmoe_status lmoe_create(const lmoe_config* cfg, const lmoe_weights* w, lmoe_handle* out) {
  g_last_error.clear();
  if (!out) return fail(LMOE_E_INVAL, "out is NULL");
  *out = nullptr;
  lmoe_status st = check_config(cfg);
  if (st != LMOE_OK) return st;
  st = check_weights(cfg, w);
  if (st != LMOE_OK) return st;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LMOE_E_HIP, "hipGetDevice failed");
  lmoe_ctx* h = new (std::nothrow) lmoe_ctx();
  if (!h) return fail(LMOE_E_NOMEM, "host allocation failed");
  h->cfg = *cfg;
  h->w = *w;
  h->device = dev;
  h->plan = make_plan(*cfg);
  h->ws = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&h->ws), h->plan.total) != hipSuccess) {
    (void)hipGetLastError();
    const std::string msg = "hipMalloc of " + std::to_string(h->plan.total) + " workspace bytes failed";
    delete h;
    return fail(LMOE_E_NOMEM, msg);
  }
  // The top-k kernel ORs into the chunk masks; the sort clears them after use,
  // so they start at zero once here.
  if (hipMemset(h->ws + h->plan.masks, 0, h->plan.chunk_base - h->plan.masks) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(h->ws);
    delete h;
    return fail(LMOE_E_HIP, "clearing the workspace failed");
  }
  h->timing = false;
  h->masks_dirty = false;
  h->n_cu = 256;
  {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
      h->n_cu = prop.multiProcessorCount;
  }
  memset(h->acc_ms, 0, sizeof(h->acc_ms));
  h->n_timed = 0;
  *out = h;
  return LMOE_OK;
}

lmoe_status lmoe_destroy(lmoe_handle h) {
  if (!h) return LMOE_OK;
  int cur = 0;
  (void)hipGetDevice(&cur);
  if (cur != h->device) (void)hipSetDevice(h->device);
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  hipError_t err = h->ws ? hipFree(h->ws) : hipSuccess;
  if (cur != h->device) (void)hipSetDevice(cur);
  delete h;
  if (err != hipSuccess) return fail(LMOE_E_HIP, std::string("hipFree: ") + hipGetErrorString(err));
  return LMOE_OK;
}

lmoe_status lmoe_set_timing(lmoe_handle h, int enable) {
  if (!h) return fail(LMOE_E_INVAL, "handle is NULL");
  h->timing = enable != 0;
  return LMOE_OK;
}

lmoe_status lmoe_get_timing(lmoe_handle h, float* ms_per_stage, int32_t* n_forward) {
  if (!h || !ms_per_stage || !n_forward) return fail(LMOE_E_INVAL, "NULL argument");
  const size_t per = LMOE_NUM_STAGES + 1;
  for (size_t f = 0; f + per <= h->events.size(); f += per) {
    if (hipEventSynchronize(h->events[f + per - 1]) != hipSuccess)
      return fail(LMOE_E_HIP, "hipEventSynchronize failed");
    for (int s = 0; s < LMOE_NUM_STAGES; ++s) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, h->events[f + s], h->events[f + s + 1]) != hipSuccess)
        return fail(LMOE_E_HIP, "hipEventElapsedTime failed");
      h->acc_ms[s] += ms;
    }
    ++h->n_timed;
  }
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.clear();
  for (int s = 0; s < LMOE_NUM_STAGES; ++s) ms_per_stage[s] = h->acc_ms[s];
  *n_forward = h->n_timed;
  memset(h->acc_ms, 0, sizeof(h->acc_ms));
  h->n_timed = 0;
  return LMOE_OK;
}

lmoe_status lmoe_forward(lmoe_handle h, const void* x, void* out, int32_t T, void* hip_stream,
                         const lmoe_aux* aux) {
  g_last_error.clear();
  if (!h) return fail(LMOE_E_INVAL, "handle is NULL");
  lmoe_status st = check_forward_args(h->cfg, x, out, T, aux);
  if (st != LMOE_OK || T == 0) return st;

  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(LMOE_E_HIP, "hipGetDevice failed");
  if (cur != h->device && hipSetDevice(h->device) != hipSuccess)
    return fail(LMOE_E_HIP, "hipSetDevice failed");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipEvent_t ev[LMOE_NUM_STAGES + 1] = {};
  // Stage timing records events; a stream being captured into a graph gets
  // none (the forward itself captures: kernels only, no allocation, memset or
  // host synchronization).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return fail(LMOE_E_HIP, "hipStreamIsCapturing failed");
  const bool timing = h->timing && cap == hipStreamCaptureStatusNone;
  if (timing)
    for (auto& e : ev)
      if (hipEventCreate(&e) != hipSuccess) return fail(LMOE_E_HIP, "hipEventCreate failed");
  const hipError_t err = enqueue_forward(h->cfg, h->w, h->plan, h->ws, h->n_cu, h->masks_dirty,
                                         timing ? ev : nullptr, x, out, T, s, aux);
  if (timing) h->events.insert(h->events.end(), ev, ev + LMOE_NUM_STAGES + 1);
  if (cur != h->device) (void)hipSetDevice(cur);
  if (err != hipSuccess) return fail(LMOE_E_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  return LMOE_OK;
}

lmoe_status lmoe_forward_noalloc(const lmoe_config* cfg, const lmoe_weights* w, const void* x, void* out,
                                 int32_t T, void* hip_stream, const lmoe_aux* aux) {
  g_last_error.clear();
  lmoe_status st = check_config(cfg);
  if (st != LMOE_OK) return st;
  st = check_weights(cfg, w);
  if (st != LMOE_OK) return st;
  st = check_forward_args(*cfg, x, out, T, aux);
  if (st != LMOE_OK || T == 0) return st;
  // The scratch is laid out for exactly T tokens.
  lmoe_config c = *cfg;
  c.max_tokens = T;
  const Plan pl = make_plan(c);
  if (pl.total > (size_t)LMOE_NOALLOC_SCRATCH_BYTES)
    return fail(LMOE_E_INVAL, "T = " + std::to_string(T) + " needs " + std::to_string(pl.total) +
                                  " bytes of workspace, more than the " +
                                  std::to_string((size_t)LMOE_NOALLOC_SCRATCH_BYTES) +
                                  "-byte scratch of lmoe_forward_noalloc (use lmoe_create + lmoe_forward)");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LMOE_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(LMOE_E_UNSUPPORTED, "device index beyond 63");
  NoallocDevice& d = noalloc_device(dev);
  if (d.err != hipSuccess)
    return fail(LMOE_E_HIP, std::string("hipGetSymbolAddress of the scratch failed: ") + hipGetErrorString(d.err));
  // The scratch keeps whatever the device's previous call (or another layout)
  // left in it: the chunk masks, the only region that must start at zero, are
  // cleared first by a kernel.
  bool masks_dirty = true;
  const hipError_t err = enqueue_forward(c, *w, pl, d.ptr, d.n_cu, masks_dirty, nullptr, x, out, T,
                                         static_cast<hipStream_t>(hip_stream), aux);
  if (err != hipSuccess) return fail(LMOE_E_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  return LMOE_OK;
}

}  // extern "C"
