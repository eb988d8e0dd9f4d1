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
// One workgroup = 8 waves = 64 query heads of one query row; all heads share
// the row's gathered latent rows (multi-query).  Per step of BN = 32 sorted
// indices:
//   gather   32 latent rows (d_qk bf16 each) straight into LDS by buffer
//            loads with the LDS bit (per-lane row addresses; entries past the
//            valid count read as zeros through the buffer's record bound),
//            double buffered, 16-byte chunks XOR-swizzled within each row;
//   S^T      = K Q^T over d_qk with v_mfma_f32_16x16x32_bf16, Q^T held in
//            registers; a pair of waves splits d_qk (and later d_v) between
//            them and adds its partial logits through LDS; fp32 accumulation;
//   softmax  fp32 online update with a lazily moved reference max;
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

#include <type_traits>

namespace vea {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2v));
}
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Transposed LDS read: 8 bytes per lane, 4x16 bf16 blocks transposed within
// each group of 16 lanes.
__device__ __forceinline__ u32x2 lds_read_tr(const void* p) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <int DQK, int DV, int MAXK>
struct SCfg {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int HPW = 16;                       // heads per wave pair (MFMA N)
  static constexpr int HEADS = (WAVES / 2) * HPW;      // heads per workgroup
  static constexpr int BN = 32;                        // sorted indices per step
  static constexpr int ROWB = DQK * 2;                 // bytes per latent row (no padding)
  static constexpr int TILE = BN * ROWB;
  static constexpr int CPR = DQK / 8;                  // 16-byte chunks per row
  static constexpr int BLOCKS = TILE / 1024;           // 1 KB DMA blocks per tile
  static constexpr int KS_HALF = DQK / 64;             // 32-wide k-steps per half of d_qk
  static constexpr int NT_HALF = DV / 32;              // 16-wide n-tiles per half of d_v
  static_assert(TILE % 1024 == 0, "tile in whole 1 KB DMA blocks");
  static_assert(CPR % 8 == 0, "swizzle stays inside aligned groups of 8 chunks");
  static_assert(DQK % 64 == 0 && DV % 32 == 0 && DV <= DQK, "latent dims");
  static_assert((DV / 2) % 64 == 0, "each half of d_v starts on an 8-chunk boundary");
  static_assert(HEADS == kSparseHeadsPerWG, "host launch shape");
  // Chunk swizzle.  Rows r and r + 1 sit 32 banks apart (1152-byte rows), so
  // the swizzle works on the row pair x = (r / 2) % 8 and permutes the low 3
  // bits of a chunk index (it stays inside aligned groups of 8 chunks).
  //  * V^T reads (ds_read_b64_tr_b16: 32 lanes per cycle, rows 0..7 x one
  //    chunk pair) need the four rows of one bank half on disjoint chunk
  //    pairs: the permutation must map x = 0..3 (and 4..7) to distinct x / 2.
  //  * K reads (ds_read_b128, 16 rows x one logical chunk) were measured with
  //    the SQ_LDS_BANK_CONFLICT counter for candidate permutations: x ^ (2x & 6)
  //    is conflict-free for both read kinds (the bit reversal and the
  //    rotation, which also satisfy the V^T rule, cost K reads 4 cycles).
  static __device__ __forceinline__ int swz(int r) {
    const int x = (r >> 1) & 7;
    return x ^ ((x << 1) & 6);
  }
};

// One workgroup = 8 waves = 64 heads of one query row.  The two waves of a
// pair serve the same 16 heads: wave half hh computes the logits over its half
// of d_qk and keeps the output for its half of d_v.  After the QK^T MFMAs the
// pair adds its two partial logit tiles through LDS (the sum is commutative,
// so both waves hold bitwise the same logits and run the same softmax).  This
// keeps a wave at 36 Q + 64 O registers.
template <int DQK, int DV, int MAXK>
__global__ __launch_bounds__(512, 1) void sparse_mqa_kernel(SparseParams p) {
  using C = SCfg<DQK, DV, MAXK>;
  __shared__ __attribute__((aligned(1024))) unsigned char tile0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char tile1[C::TILE];
  __shared__ int sidx[MAXK];
  __shared__ float xs[C::WAVES][8][64];                 // partial logits, exchanged within a pair

  const int row = blockIdx.x / p.head_blocks;
  const int hb = blockIdx.x - row * p.head_blocks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) value
  const int hh = wave & 1;                              // which half of d_qk / d_v
  const int pr = wave >> 1;                             // pair: 16 heads
  const int l16 = lane & 15;
  const int G = lane >> 4;                              // lane group 0..3

  // ---- canonical order: load the row's indices and sort them ascending
  int n2 = 1;
  while (n2 < p.k) n2 <<= 1;
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
  // number of valid entries: first position holding INT_MAX (binary search)
  int lo = 0, hi = n2;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sidx[mid] == INT_MAX) hi = mid; else lo = mid + 1;
  }
  const int nvalid = lo;

  // ---- Q^T fragment: this pair's 16 heads, this wave's half of d_qk
  const int head = hb * C::HEADS + pr * C::HPW + l16;
  const bool hvalid = head < p.heads;
  const int dq0 = hh * (DQK / 2);
  u32x4 qf[C::KS_HALF];
  {
    const uint16_t* src = p.q + ((int64_t)row * p.heads + (hvalid ? head : 0)) * DQK + dq0 + 8 * G;
#pragma unroll
    for (int ks = 0; ks < C::KS_HALF; ++ks) {
      const u32x4 v = *(const u32x4*)(src + 32 * ks);
      qf[ks] = hvalid ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  float c = fabsf(p.scale) * kLog2e;
  if (p.scale < 0.f) {
#pragma unroll
    for (int ks = 0; ks < C::KS_HALF; ++ks) qf[ks] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  c = fmaxf(c, FLT_MIN);

  // ---- gather by DMA: 1 KB block bk of a tile is filled by wave bk % 8;
  // slot sl of the tile holds row sl / CPR, physical chunk sl % CPR =
  // logical chunk ^ swz(row).
  const __amdgpu_buffer_rsrc_t kv_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, (short)0, (int)((int64_t)p.n_kv * C::ROWB), 0x00020000);
  auto gather = [&](int kt, unsigned char* dst) {
#pragma unroll
    for (int bi = 0; bi < (C::BLOCKS + C::WAVES - 1) / C::WAVES; ++bi) {
      const int bk = bi * C::WAVES + wave;              // wave-uniform
      if (bk < C::BLOCKS) {
        const int sl = bk * 64 + lane;
        const int r = sl / C::CPR;
        const int col = 16 * ((sl - r * C::CPR) ^ C::swz(r));
        const int j = kt * C::BN + r;
        const unsigned off = j < nvalid ? (unsigned)sidx[j] * C::ROWB + col : 0xFFFFFFF0u;   // past the end: zeros
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, (__attribute__((address_space(3))) void*)(dst + bk * 1024),
                                                 16, off, 0, 0, 0);
      }
    }
  };

  // ---- per-lane LDS read offsets.  The swizzle only permutes the low 3 bits
  // of a chunk index, so chunk 8 a + x (x < 8) sits at 16 (8 a + (x ^ swz)):
  // one per-lane base per x class plus a compile-time 128 a offset.
  const int ksw = C::swz(l16);                           // same for rows l16 and 16 + l16
  int kbase[2];                                          // K chunk dq0/8 + 4 ks + G, ks = 2 a + b
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int c0 = dq0 / 8 + 4 * b + G;                  // chunk at a = 0 (dq0/8 need not be 8-aligned)
    kbase[b] = l16 * C::ROWB + 16 * ((c0 & ~7) | ((c0 & 7) ^ ksw));
  }
  const int vr0 = 4 * G + (l16 >> 2);                    // first of the 4 keys read transposed
  const int vx = (l16 & 3) >> 1;                         // chunk dv0/8 + 2 nt + vx, nt = 4 a + b
  const int dv0 = hh * (DV / 2);
  int vbase0[4], vbase1[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    vbase0[b] = vr0 * C::ROWB + dv0 * 2 + 16 * ((2 * b + vx) ^ C::swz(vr0)) + 8 * (l16 & 1);
    vbase1[b] = (vr0 + 16) * C::ROWB + dv0 * 2 + 16 * ((2 * b + vx) ^ C::swz(vr0 + 16)) + 8 * (l16 & 1);
  }

  floatx4 o[C::NT_HALF];
#pragma unroll
  for (int nt = 0; nt < C::NT_HALF; ++nt) o[nt] = (floatx4){};
  float m_used = -INFINITY, l_run = 0.f;
  const int n_tiles = (nvalid + C::BN - 1) / C::BN;

  auto step = [&](int kt, auto odd_tag) {
    constexpr bool ODD = decltype(odd_tag)::value;
    unsigned char* cur = ODD ? tile1 : tile0;
    unsigned char* nxt = ODD ? tile0 : tile1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this lane's gather of tile kt landed
    __syncthreads();                                   // everyone's landed; tile kt-1 fully consumed
    if (kt + 1 < n_tiles) gather(kt + 1, nxt);

    // partial S^T[key 16 kb + 4 G + i][head l16] over this wave's half of d_qk
    floatx4 s0 = (floatx4){}, s1 = (floatx4){};
#pragma unroll
    for (int ks = 0; ks < C::KS_HALF; ++ks) {
      const unsigned char* kp = cur + kbase[ks & 1] + 128 * (ks >> 1);
      const u32x4 a0 = *(const u32x4*)(kp);
      const u32x4 a1 = *(const u32x4*)(kp + 16 * C::ROWB);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qf[ks]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qf[ks]), s1, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[wave][i][lane] = s0[i];
      xs[wave][4 + i][lane] = s1[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {                      // own + partner: the same sum in both waves
      s0[i] += xs[wave ^ 1][i][lane];
      s1[i] += xs[wave ^ 1][4 + i][lane];
    }
    if ((kt + 1) * C::BN > nvalid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kt * C::BN + 4 * G + i >= nvalid) s0[i] = -INFINITY;
        if (kt * C::BN + 16 + 4 * G + i >= nvalid) s1[i] = -INFINITY;
      }
    }
    float mx = vmax(vmax(s0[0], s0[1]), vmax(s0[2], s0[3]));
    mx = vmax(mx, vmax(vmax(s1[0], s1[1]), vmax(s1[2], s1[3])));
    mx = vmax(mx, __shfl_xor(mx, 16));
    mx = vmax(mx, __shfl_xor(mx, 32));
    const float mx_sc = (mx == -INFINITY) ? -INFINITY : mx * c;
    const bool upd = mx_sc > m_used + 8.0f;            // lazy reference max (P < 2^8)
    if (__any(upd)) {
      asm volatile("; rare: move the reference max, rescale O and l" ::);
      const float m_new = upd ? mx_sc : m_used;
      const float alpha = upd ? fast_exp2(m_used - m_new) : 1.0f;
      m_used = m_new;
#pragma unroll
      for (int nt = 0; nt < C::NT_HALF; ++nt) o[nt] *= alpha;
      l_run *= alpha;
    }
    const float m_use = (m_used == -INFINITY) ? 0.f : m_used;
    float e[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = fast_exp2(fmaf(s0[i], c, -m_use));
      e[4 + i] = fast_exp2(fmaf(s1[i], c, -m_use));
    }
    l_run += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    // B operand: k-slot j of lane group G is key 16 (j/4) + 4 G + j%4.
    const u32x4 pb = (u32x4){pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                             pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
    // A operand V^T[n][keys]: transposed read of rows vr0 (+16), this wave's d_v half.
#pragma unroll
    for (int nt = 0; nt < C::NT_HALF; ++nt) {
      const u32x2 a = lds_read_tr(cur + vbase0[nt & 3] + 128 * (nt >> 2));
      const u32x2 b = lds_read_tr(cur + vbase1[nt & 3] + 128 * (nt >> 2));
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8((u32x4){a[0], a[1], b[0], b[1]}), as_bf16x8(pb),
                                                      o[nt], 0, 0, 0);
    }
  };

  if (n_tiles > 0) gather(0, tile0);
  int kt = 0;
  for (; kt + 2 <= n_tiles; kt += 2) {
    step(kt, std::false_type{});
    step(kt + 1, std::true_type{});
  }
  if (kt < n_tiles) step(kt, std::false_type{});

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (hvalid) {
    uint16_t* dst = p.out + ((int64_t)row * p.heads + head) * DV + dv0 + 4 * G;
#pragma unroll
    for (int nt = 0; nt < C::NT_HALF; ++nt)
      *(u32x2*)(dst + 16 * nt) = (u32x2){pack_bf16x2(o[nt][0] * inv, o[nt][1] * inv),
                                         pack_bf16x2(o[nt][2] * inv, o[nt][3] * inv)};
    if (p.lse != nullptr && G == 0 && hh == 0)
      p.lse[(int64_t)head * p.rows + row] = l_tot > 0.f ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_sparse_mqa(const SparseParams& p, int d_qk, int d_v, hipStream_t s) {
  if (d_qk != 576 || d_v != 512) return hipErrorInvalidValue;
  if (p.k > 4096) return hipErrorInvalidValue;
  if (p.rows == 0) return hipSuccess;
  const dim3 grid(p.rows * p.head_blocks), block(512);
  if (p.k <= 2048) hipLaunchKernelGGL((sparse_mqa_kernel<576, 512, 2048>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((sparse_mqa_kernel<576, 512, 4096>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace vea
