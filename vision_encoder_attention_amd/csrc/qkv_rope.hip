// Fused-QKV split + rotary position embedding for gfx950.
//
// The vision encoder's qkv_rope step (「DeepSeek V4.1 上 4×RTX 3090：视觉链路的两个坑和修复」,
// section 二) rotated Q and K in place, and two threads touched the same
// memory.  This kernel is out-of-place and every output element has exactly
// one writer: a thread owns whole 16-byte chunks (4 rotation pairs), so no
// pair is ever split between threads and nothing needs synchronising except
// the per-token angle table, written before one barrier and read after it.
//
// Layout of the fused projection output ([T, 3*hidden] in
// 「从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash - Prefill」 section 3.1):
// columns [Q heads | K heads | V heads], each head `d` contiguous bf16 values.
// Q and K are contiguous in a row, so the (Hq + Hkv) * d / 8 chunks of a token
// are read as one coalesced run; V is not touched (the attention kernel reads
// it in place through a strided pointer).
//
// Precision (trigonometry in at least fp32:
// 「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈性能」 section 4.1): the
// frequency theta^(-2i/d_r) and the angle pos * freq are formed in fp64, sin and
// cos are taken in fp64 and rounded to fp32, the rotation is done in fp32 and
// the result rounded to bf16 (nearest even).  At position 8191 an fp32 angle
// would carry ~5e-4 rad of error; the fp64 angle keeps it below 1e-11.
#include "vea_internal.h"

#include <math.h>

#include <algorithm>

namespace vea {
namespace {

constexpr int kRopeMaxHalf = 128;   // head_dim <= 256
constexpr int kRopeMaxTokens = 8;   // tokens per workgroup

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// One workgroup rotates `tpw` consecutive tokens (several when a token's row
// is short, so that every thread has work): first their angle tables, then
// their 16-byte chunks.
__global__ __launch_bounds__(256) void qkv_rope_kernel(RopeParams p, int tpw) {
  __shared__ float cs[kRopeMaxTokens][kRopeMaxHalf];
  __shared__ float sn[kRopeMaxTokens][kRopeMaxHalf];
  const int t0 = blockIdx.x * tpw;
  const int nt = min(tpw, p.tokens - t0);                    // tokens of this workgroup
  const int half = p.d >> 1;
  const double log2_theta = log2(p.theta);

  // Angle tables, indexed by (token, pair index inside the head).
  for (int idx = threadIdx.x; idx < nt * half; idx += blockDim.x) {
    const int tk = idx / half, i = idx - tk * half;
    const int t = t0 + tk;
    double pos, expo;
    if (p.pos_dims == 1) {
      pos = (double)p.pos[t];
      expo = -2.0 * (double)i / (double)p.d;                 // span d
    } else {
      const int q4 = p.d >> 2;                               // pairs per half-head
      const int axis = i >= q4 ? 1 : 0;                      // 0: grid row, 1: grid column
      const int ii = i - axis * q4;
      pos = (double)p.pos[2 * (int64_t)t + axis];
      expo = -2.0 * (double)ii / (double)(p.d >> 1);         // span d/2
    }
    const double ang = pos * exp2(expo * log2_theta);
    double sv, cv;
    sincos(ang, &sv, &cv);
    cs[tk][i] = (float)cv;
    sn[tk][i] = (float)sv;
  }
  __syncthreads();

  const int cph = p.d >> 3;                                  // 16-byte chunks per head
  if (p.rot_half) {
    // Rotate-half pairing: pair i of a span joins features i and i + span/2.
    // A thread owns chunk j of a span's first half and its partner chunk in
    // the second half (8 pairs).  1D: one span per head (table entries 0 ..
    // d/2); 2D: two spans of d/2 (entries of the second from d/4 on).
    const int pph = p.d >> 4;                                // chunk pairs per head
    const int spc = p.pos_dims == 1 ? pph : (p.d >> 5);      // chunk pairs per span
    const int npairs = (p.hq + p.hkv) * pph;
    for (int idx = threadIdx.x; idx < nt * npairs; idx += blockDim.x) {
      const int tk = idx / npairs, ci = idx - tk * npairs;
      const int t = t0 + tk;
      const int head = ci / pph;
      const int cp = ci - head * pph;
      const int sp = cp / spc, l = cp - sp * spc;
      const int c0 = sp * 2 * spc + l, c1 = c0 + spc;         // chunks of the first elements and partners
      const int ebase = sp * 8 * spc + 8 * l;                 // table entry of the chunk's first pair
      const uint16_t* src = p.x + (int64_t)t * p.x_stride + (int64_t)head * p.d;
      const u32x4 v0 = *(const u32x4*)(src + 8 * c0);
      const u32x4 v1 = *(const u32x4*)(src + 8 * c1);
      u32x4 o0, o1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e = ebase + 2 * w;
        const float a0 = bf16lo(v0[w]), a1 = bf16hi(v0[w]);
        const float b0 = bf16lo(v1[w]), b1 = bf16hi(v1[w]);
        const float ca = cs[tk][e], sa = sn[tk][e], cb = cs[tk][e + 1], sb = sn[tk][e + 1];
        o0[w] = pack2(fmaf(a0, ca, -(b0 * sa)), fmaf(a1, cb, -(b1 * sb)));
        o1[w] = pack2(fmaf(a0, sa, b0 * ca), fmaf(a1, sb, b1 * cb));
      }
      uint16_t* dst = head < p.hq ? p.q + ((int64_t)t * p.hq + head) * p.d
                                  : p.k + ((int64_t)t * p.hkv + (head - p.hq)) * p.d;
      *(u32x4*)(dst + 8 * c0) = o0;
      *(u32x4*)(dst + 8 * c1) = o1;
    }
    return;
  }
  const int nchunks = (p.hq + p.hkv) * cph;                  // per token
  for (int idx = threadIdx.x; idx < nt * nchunks; idx += blockDim.x) {
    const int tk = idx / nchunks, ci = idx - tk * nchunks;
    const int t = t0 + tk;
    const int head = ci / cph;
    const int ch = ci - head * cph;
    const u32x4 v = *(const u32x4*)(p.x + (int64_t)t * p.x_stride + 8 * ci);
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int pi = 4 * ch + w;                             // pair index inside the head
      const float x0 = bf16lo(v[w]), x1 = bf16hi(v[w]);
      const float c = cs[tk][pi], sv = sn[tk][pi];
      const float y0 = fmaf(x0, c, -(x1 * sv));
      const float y1 = fmaf(x0, sv, x1 * c);
      o[w] = pack2(y0, y1);
    }
    uint16_t* dst = head < p.hq ? p.q + ((int64_t)t * p.hq + head) * p.d + 8 * ch
                                : p.k + ((int64_t)t * p.hkv + (head - p.hq)) * p.d + 8 * ch;
    *(u32x4*)dst = o;
  }
}

}  // namespace

hipError_t launch_qkv_rope(const RopeParams& p, hipStream_t s) {
  if (p.tokens == 0) return hipSuccess;
  // tokens per workgroup: enough 16-byte chunks for about 4 per thread
  const int nchunks = (p.hq + p.hkv) * (p.d >> 3);
  const int tpw = std::max(1, std::min(kRopeMaxTokens, 1024 / std::max(1, nchunks)));
  hipLaunchKernelGGL(qkv_rope_kernel, dim3((p.tokens + tpw - 1) / tpw), dim3(256), 0, s, p, tpw);
  return hipGetLastError();
}

}  // namespace vea
