// Deterministic top-k index selection for the sparse indexer, for gfx950.
//
// Source: 「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」, sections
// 修改topk结果，输出后排序 and 用 torch.sort 替换 topk，输出对比: the indexer
// keeps the 2048 highest-scoring positions of each row of logits; an unstable
// top-k let equal scores at the edge of the selection fall either way between
// two identical requests, and a stable sort fixed it.  Ties go by position,
// never by where a value happens to sit in a parallel reduction
// (「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈性能」 section 4.2).
//
// Rank order of a row: value descending, equal values by ascending position;
// NaN after every number; -0.0 ties with +0.0.  Each valid position gets one
// 64-bit key, its value mapped to an order-preserving 32-bit code in the high
// half and the bitwise complement of its position in the low half, so that
// "key descending" is exactly the rank order and no two keys are equal.  One
// workgroup sorts a row's keys with a bitonic network in LDS (a fixed
// sequence of compare-exchanges: the result cannot depend on timing) and
// writes the positions of the first k keys.  Positions past the row's span
// get key 0, below every valid key, and come out as -1.
#include "vea_internal.h"

#include <math.h>

namespace vea {
namespace {

constexpr int kTopkThreads = 256;

// Order-preserving code of a float: larger value -> larger code; NaN -> 0
// (below -inf, whose code is 0x007FFFFF); -0.0 is folded into +0.0 first.
__device__ __forceinline__ uint32_t order_code(float x) {
  x = x + 0.0f;                                         // -0.0 + 0.0 = +0.0
  if (x != x) return 0u;
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CAP>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ uint64_t keys[CAP];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  int s = 0, len = p.n;
  if (p.starts != nullptr) s = min(max(p.starts[r], 0), p.n);
  if (p.lens != nullptr) len = min(max(p.lens[r], 0), p.n - s);
  else len = p.n - s;
  int size = 2;                                         // sort width: a power of two >= len
  while (size < len) size <<= 1;

  const float* row = p.logits + (int64_t)r * p.row_stride + s;
  for (int i = tid; i < size; i += kTopkThreads) {
    uint64_t key = 0;
    if (i < len) key = ((uint64_t)order_code(row[i]) << 32) | (uint32_t)~(uint32_t)(s + i);
    keys[i] = key;
  }
  __syncthreads();

  // Bitonic network, descending: for every merge width w and stride j, pair
  // (i, i + j) with i's bit j clear; blocks with bit w clear are put in
  // descending order, the others ascending, so the last merge (w = size)
  // leaves the whole row descending.
  for (int w = 2; w <= size; w <<= 1) {
    for (int j = w >> 1; j > 0; j >>= 1) {
      for (int t = tid; t < (size >> 1); t += kTopkThreads) {
        const int i = 2 * t - (t & (j - 1));
        const uint64_t a = keys[i], b = keys[i + j];
        const bool desc = (i & w) == 0;
        if (desc ? (a < b) : (a > b)) {
          keys[i] = b;
          keys[i + j] = a;
        }
      }
      __syncthreads();
    }
  }

  const int m = min(p.k, len);
  int32_t* out = p.out + (int64_t)r * p.k;
  for (int t = tid; t < p.k; t += kTopkThreads)
    out[t] = t < m ? (int32_t)~(uint32_t)(keys[t] & 0xFFFFFFFFu) : -1;
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  if (p.n < 1 || p.n > kTopkMaxN || p.k < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((topk_kernel<kTopkMaxN>), dim3(p.rows), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace vea
