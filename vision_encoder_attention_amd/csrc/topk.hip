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
// workgroup sorts a row's keys with a bitonic network (a fixed sequence of
// compare-exchanges: the result cannot depend on timing) and writes the
// positions of the first k keys.  Positions past the row's span get key 0,
// below every valid key, and come out as -1.
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

// Bitonic network over CAP = 4096 keys (the row, padded with 0 keys),
// descending, with the compare-exchanges in registers: each thread holds 16
// keys whose indices differ only in a window of 4 consecutive index bits
// [lo, lo + 4), the other 8 bits being its thread id, so the strides 2^lo ..
// 2^(lo+3) pair keys of the same thread.  The keys pass through LDS only when
// the window moves (21 times for 4096 keys instead of a barrier for each of
// the 78 strides).  Every merge width w and stride j pair (i, i + j) with bit
// j of i clear; blocks with bit w clear go descending, the others ascending,
// so the last merge leaves the row descending.
template <int CAP>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  constexpr int E = CAP / kTopkThreads;
  constexpr int LOG = 12;
  static_assert(E == 16 && (1 << LOG) == CAP, "16 keys per thread, 4096 keys");
  __shared__ uint64_t keys[CAP + CAP / 16];             // one pad slot per 16: few bank conflicts
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  int s = 0, len;
  if (p.starts != nullptr) s = min(max(p.starts[r], 0), p.n);
  if (p.lens != nullptr) len = min(max(p.lens[r], 0), p.n - s);
  else len = p.n - s;

  // index of this thread's key e under window [lo, lo + 4)
  auto idx = [&](int lo, int e) { return (tid & ((1 << lo) - 1)) | ((tid >> lo) << (lo + 4)) | (e << lo); };
  auto slot = [](int i) { return i + (i >> 4); };

  uint64_t v[E];
  const float* row = p.logits + (int64_t)r * p.row_stride + s;
#pragma unroll
  for (int e = 0; e < E; ++e) {                         // window [0, 4): index 16 tid + e
    const int i = E * tid + e;
    v[e] = i < len ? ((uint64_t)order_code(row[i]) << 32) | (uint32_t)~(uint32_t)(s + i) : 0ull;
  }
  int lo = 0;
  // Fully unrolled: every window, stride and skip below is a compile-time
  // constant; only the direction bit of a merge block comes from tid.
#pragma unroll
  for (int sb = 1; sb <= LOG; ++sb) {                   // merge width w = 2^sb
    const int w = 1 << sb;
#pragma unroll
    for (int hi = sb - 1; hi >= 0; hi -= 4) {           // strides 2^hi .. 2^max(hi-3, 0)
      const int nlo = max(hi - 3, 0);
      if (nlo != lo) {
        // Each thread writes back exactly the slots it read under the old
        // window, so one barrier (between the writes and the reads) suffices.
#pragma unroll
        for (int e = 0; e < E; ++e) keys[slot(idx(lo, e))] = v[e];
        __syncthreads();
        lo = nlo;
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = keys[slot(idx(lo, e))];
      }
#pragma unroll
      for (int m = 3; m >= 0; --m) {
        if (lo + m > hi) continue;                      // a passenger bit of this window
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & (1 << m)) continue;
          const int e2 = e | (1 << m);
          const bool desc = (idx(lo, e) & w) == 0;
          const uint64_t a = v[e], c = v[e2];
          const bool sw = (a < c) == desc;                // keys are distinct: a > c is !(a < c)
          v[e] = sw ? c : a;
          v[e2] = sw ? a : c;
        }
      }
    }
  }
  // window [0, 4) again: key e of this thread is rank 16 tid + e
  const int m = min(p.k, len);
  int32_t* out = p.out + (int64_t)r * p.k;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = E * tid + e;
    if (t < p.k) out[t] = t < m ? (int32_t)~(uint32_t)(v[e] & 0xFFFFFFFFu) : -1;
  }
  for (int t = CAP + tid; t < p.k; t += kTopkThreads) out[t] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  if (p.n < 1 || p.n > kTopkMaxN || p.k < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((topk_kernel<kTopkMaxN>), dim3(p.rows), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace vea
