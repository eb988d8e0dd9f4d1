// Top-k sparse multi-query attention over a shared latent KV, for gfx950.
//
// Source: 「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」.  The decoder's
// sparse attention reads Q, the KV cache and an index (section 实验方法和结果);
// with the same index SET in another order the bf16 output moved by 2^-8,
// because the blockwise merge of eq. (1)(2) (section 进一步探索) rounds in the
// order the blocks arrive.  Here each row's indices are sorted ascending in
// LDS before use, so the blocks always arrive in one canonical order and the
// output is bitwise independent of the order the caller supplies.
//
// One workgroup = 4 waves = 64 query heads of one query row; all heads share
// the row's gathered latent rows (multi-query).  Per step of BN = 32 sorted
// indices:
//   gather   32 latent rows (d_qk bf16 each) -> LDS, 16-byte loads, double
//            buffered through registers;
//   S^T      = K Q^T over d_qk with v_mfma_f32_16x16x32_bf16, Q^T held in
//            registers (16 heads per wave), fp32 accumulation;
//   softmax  fp32 online update (running max, rescale, running sum);
//   O^T     += V^T P^T over d_v with the same MFMA.  V is the first d_v
//            columns of the gathered rows; V^T operands come straight from the
//            row-major tile with ds_read_b64_tr_b16 (each 16-lane group reads
//            a 4-key x 16-column block and receives it transposed).
// Entries < 0 or >= n_kv are skipped.  No atomics: every output element and
// lse entry has one writer.
#include "vea_internal.h"

#include <float.h>
#include <limits.h>
#include <math.h>

namespace vea {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Transposed LDS read: 8 bytes per lane, 4x16 bf16 blocks transposed within
// each group of 16 lanes.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

constexpr int kMaxK = 4096;

template <int DQK, int DV>
struct SCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 256;
  static constexpr int HPW = 16;                       // heads per wave (MFMA N)
  static constexpr int HEADS = WAVES * HPW;            // heads per workgroup
  static constexpr int BN = 32;                        // sorted indices per step
  static constexpr int KROW = DQK + 8;                 // padded LDS row (bf16)
  static constexpr int TILE = BN * KROW;
  static constexpr int DCH = DQK / 8;                  // 16-byte chunks per latent row
  static constexpr int CPT = BN * DCH / THREADS;       // chunks per thread per tile
  static_assert(BN * DCH % THREADS == 0, "gather split");
  static_assert(DQK % 32 == 0 && DV % 16 == 0 && DV <= DQK, "latent dims");
  static_assert(HEADS == kSparseHeadsPerWG, "host launch shape");
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void sparse_mqa_kernel(SparseParams p) {
  using C = SCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t tile[2 * C::TILE];
  __shared__ int sidx[kMaxK];
  __shared__ int s_nvalid;

  const int row = blockIdx.x / p.head_blocks;
  const int hb = blockIdx.x - row * p.head_blocks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int G = lane >> 4;                              // lane group 0..3

  // ---- canonical order: load the row's indices and sort them ascending
  int n2 = 1;
  while (n2 < p.k) n2 <<= 1;
  if (tid == 0) s_nvalid = 0;
  const int32_t* irow = p.idx + (int64_t)row * p.k;
  for (int i = tid; i < n2; i += C::THREADS) {
    int v = INT_MAX;
    if (i < p.k) {
      const int x = irow[i];
      v = (x >= 0 && x < p.n_kv) ? x : INT_MAX;        // padding / out of range: skipped
    }
    sidx[i] = v;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (n2 >> 1); t += C::THREADS) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const int a = sidx[i], b = sidx[j];
        if ((a > b) == up) { sidx[i] = b; sidx[j] = a; }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n2; i += C::THREADS)
    if (sidx[i] != INT_MAX && (i + 1 == n2 || sidx[i + 1] == INT_MAX)) s_nvalid = i + 1;
  __syncthreads();
  const int nvalid = s_nvalid;

  // ---- Q^T fragment of this wave's 16 heads: Q[row][head][32 ks + 8 G .. +7]
  const int head = hb * C::HEADS + wave * C::HPW + l16;
  const bool hvalid = head < p.heads;
  u32x4 qf[DQK / 32];
  {
    const uint16_t* src = p.q + ((int64_t)row * p.heads + (hvalid ? head : 0)) * DQK + 8 * G;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) {
      const u32x4 v = *(const u32x4*)(src + 32 * ks);
      qf[ks] = hvalid ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  float c = fabsf(p.scale) * kLog2e;
  if (p.scale < 0.f) {
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) qf[ks] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  c = fmaxf(c, FLT_MIN);

  floatx4 o[DV / 16];
#pragma unroll
  for (int nt = 0; nt < DV / 16; ++nt) o[nt] = (floatx4){};
  float m_run = -INFINITY, l_run = 0.f;
  const int n_tiles = (nvalid + C::BN - 1) / C::BN;

  u32x4 greg[C::CPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int cidx = tid + i * C::THREADS;
      const int r = cidx / C::DCH, col = cidx - r * C::DCH;
      const int j = kt * C::BN + r;
      const bool ok = j < nvalid;
      const u32x4 v = *(const u32x4*)(p.kv + (int64_t)(ok ? sidx[j] : 0) * DQK + 8 * col);
      greg[i] = ok ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* dst = tile + buf * C::TILE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int cidx = tid + i * C::THREADS;
      const int r = cidx / C::DCH, col = cidx - r * C::DCH;
      *(u32x4*)(dst + r * C::KROW + 8 * col) = greg[i];
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) load_tile(kt + 1);
    const uint16_t* kt_ = tile + buf * C::TILE;

    // S^T[key 16 kb + 4 G + i][head l16]
    floatx4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (floatx4){};
      const uint16_t* ka = kt_ + (16 * kb + l16) * C::KROW + 8 * G;
#pragma unroll
      for (int ks = 0; ks < DQK / 32; ++ks) {
        const u32x4 a = *(const u32x4*)(ka + 32 * ks);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[ks]), s[kb], 0, 0, 0);
      }
    }
    if ((kt + 1) * C::BN > nvalid) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kt * C::BN + 16 * kb + 4 * G + i >= nvalid) s[kb][i] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mx_sc = (mx == -INFINITY) ? -INFINITY : mx * c;
    const float m_new = fmaxf(m_run, mx_sc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(fmaf(s[kb][i], c, -m_use));
        s[kb][i] = e;
        psum += e;
      }
    l_run = fmaf(alpha, l_run, psum);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int nt = 0; nt < DV / 16; ++nt) o[nt] *= alpha;
    }
    // B operand: k-slot j of lane group G is key 16 (j/4) + 4 G + j%4.
    const u32x4 pb = (u32x4){pack_bf16x2(s[0][0], s[0][1]), pack_bf16x2(s[0][2], s[0][3]),
                             pack_bf16x2(s[1][0], s[1][1]), pack_bf16x2(s[1][2], s[1][3])};
    // A operand V^T[n][keys]: transposed read of rows 16 kb + 4 G .. +3, columns 16 nt .. +15.
    const uint16_t* vb = kt_ + (4 * G + (l16 >> 2)) * C::KROW + 4 * (l16 & 3);
#pragma unroll
    for (int nt = 0; nt < DV / 16; ++nt) {
      const u32x2 lo = lds_read_tr(vb + 16 * nt);
      const u32x2 hi = lds_read_tr(vb + 16 * C::KROW + 16 * nt);
      const u32x4 a = (u32x4){lo[0], lo[1], hi[0], hi[1]};
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pb), o[nt], 0, 0, 0);
    }
    if (kt + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (hvalid) {
    uint16_t* dst = p.out + ((int64_t)row * p.heads + head) * DV + 4 * G;
#pragma unroll
    for (int nt = 0; nt < DV / 16; ++nt)
      *(u32x2*)(dst + 16 * nt) = (u32x2){pack_bf16x2(o[nt][0] * inv, o[nt][1] * inv),
                                         pack_bf16x2(o[nt][2] * inv, o[nt][3] * inv)};
    if (p.lse != nullptr && G == 0)
      p.lse[(int64_t)head * p.rows + row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_sparse_mqa(const SparseParams& p, int d_qk, int d_v, hipStream_t s) {
  if (d_qk != 576 || d_v != 512) return hipErrorInvalidValue;
  if (p.k > kMaxK) return hipErrorInvalidValue;
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL((sparse_mqa_kernel<576, 512>), dim3(p.rows * p.head_blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace vea
