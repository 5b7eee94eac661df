// Top-k + softmax of one token's router logits by one wave; shared by the
// top-k kernel and the small-batch pooled-norm kernel, which runs it on the
// logits it has just reduced.
#pragma once
#include "common.h"

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

// k rounds of a wave arg-max, each on the lanes' best
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

// Token t's top-k, by the calling wave (all 64 lanes): row points at its E
// logits. Lane j < k writes the j-th selected expert and its weight, and ORs
// the token's bit into its chunk's mask of that expert.
// MAXQ: the slots a lane holds at most (E <= 64 MAXQ); the rounds scan only those.
template <int MAXQ>
__device__ __forceinline__ void topk_token_q(const float* __restrict__ row, int t, int E, int k,
                                             int32_t* __restrict__ ids, float* __restrict__ w,
                                             uint64_t* __restrict__ chunk_masks) {
  const int lane = threadIdx.x & 63;
  const int per = (E + kWave - 1) / kWave;
  float v[MAXQ];
  unsigned taken = 0;
#pragma unroll
  for (int q = 0; q < MAXQ; ++q) {
    const int e = q * kWave + lane;
    const bool ok = q < per && e < E;
    // unconditional load from a clamped (valid) address, masked afterwards
    const float x = row[e < E ? e : E - 1];
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
    for (int q = 0; q < MAXQ; ++q)
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

// Token t's top-k (as topk_token_q), the per-lane slot count picked from E.
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int t, int E, int k,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           uint64_t* __restrict__ chunk_masks) {
  if (E <= 4 * kWave)
    topk_token_q<4>(row, t, E, k, ids, w, chunk_masks);
  else
    topk_token_q<kMaxPerLane>(row, t, E, k, ids, w, chunk_masks);
}

}  // namespace
}  // namespace lmoe
