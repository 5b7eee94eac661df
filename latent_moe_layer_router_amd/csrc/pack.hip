// Load-time copy of bf16 expert weights into the packed expert layout: each
// [rows][cols] row-major matrix becomes a sequence of 8 KiB blocks of 64 rows x
// 64 columns (block (g, s) at element (g * cols / 64 + s) * 4096, its row r at
// r * 64), the order in which the weight-streaming kernels and the tiled
// grouped GEMM read a stage of 64 rows x 64 K-columns. The values are not
// changed; only their order.
//
// One wave per block: 8 steps of 8 rows x 128 bytes (lane i: row i / 8, 16-byte
// chunk i % 8), read and written once each, non-temporal.
#include "common.h"
#include "kernels.h"

namespace lmoe {

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

__global__ __launch_bounds__(64) void pack_experts_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst, int rows, int cols) {
  const int64_t b = blockIdx.x;                  // block index over all matrices
  const int gs = cols / 64;                      // blocks per row group
  const int64_t per_mat = (int64_t)(rows / 64) * gs;
  const int64_t mat = b / per_mat;
  const int64_t in_mat = b - mat * per_mat;
  const int g = (int)(in_mat / gs), s = (int)(in_mat - (int64_t)g * gs);
  const uint16_t* sm = src + mat * (int64_t)rows * cols + (int64_t)(64 * g) * cols + 64 * s;
  uint16_t* db = dst + b * 4096;
  const int lane = threadIdx.x, r0 = lane >> 3, c = (lane & 7) * 8;
  u32x4_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(sm + (int64_t)(8 * i + r0) * cols + c));
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4_t*>(db + (8 * i + r0) * 64 + c));
}

}  // namespace

hipError_t launch_pack_experts(const uint16_t* src, uint16_t* dst, int64_t n_mats, int rows, int cols,
                               hipStream_t s) {
  if (n_mats <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
  if (rows % 64 || cols % 64) return hipErrorInvalidValue;
  const int64_t blocks = n_mats * (int64_t)(rows / 64) * (cols / 64);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_experts_kernel, dim3((unsigned)blocks), dim3(64), 0, s, src, dst, rows, cols);
  return hipGetLastError();
}

}  // namespace lmoe
