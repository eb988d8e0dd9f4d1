// Block quantisation of bf16 tensors to OCP FP8 E4M3 for gfx950.
//
// The pages allow FP8 for matrix products and recommend block-wise
// quantisation to make it pay (「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈
// 性能」 sections 4.1 and 5.3).  A block is one (token, head) row, one head, or
// one (head, channel) column of x [tokens, heads, head_dim]:
//   amax  = max |x| over the block
//   scale = fp32(amax / 448),  inv = fp32(1 / scale)   (1 and 1 when amax < 2^-64)
//   code  = e4m3 nearest-even of clamp(fp32(x * inv), -448, 448)
// The conversion is v_cvt_pk_fp8_f32 (OCP E4M3, nearest-even), after the
// clamp: above 448 the instruction would produce NaN rather than saturate.
// Per-head and per-channel scales need the whole tensor.  From 1024 tokens
// on, fp8_amax_partial_kernel takes channel maxima over chunks of 256 tokens
// (one workgroup per (chunk, head)) and fp8_amax_final_kernel combines the
// chunks of a head in chunk order; the partial maxima are staged in the
// output code buffer, which holds at least four times their size and is
// overwritten with the codes afterwards.  Below 1024 tokens fp8_amax_kernel
// scans a head in one workgroup.  Maxima are exact and combined in a fixed
// order: no atomics, bitwise reproducible.  fp8_quant_kernel then codes.
#include "vea_internal.h"

#include <math.h>

namespace vea {
namespace {

constexpr float kE4m3Max = 448.0f;
constexpr float kEmptyAmax = 5.421010862427522e-20f;   // 2^-64

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float scale_of(float amax) { return amax < kEmptyAmax ? 1.0f : amax / kE4m3Max; }

// Two values to two e4m3 codes in the low (HI = false) or high half of w.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t w) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, HI);
}

// Per head (granularity 1) or per (head, channel) (granularity 2): workgroup
// h; thread = (channel chunk of 8, token lane); each thread scans its tokens,
// then the lanes of a chunk are combined in LDS.
__global__ __launch_bounds__(256) void fp8_amax_kernel(QuantParams p) {
  __shared__ float part[256][9];
  const int h = blockIdx.x;
  const int cpr = p.d >> 3;                            // 8-channel chunks per row
  const int c8 = threadIdx.x % cpr, tl = threadIdx.x / cpr, tpp = 256 / cpr;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* base = p.x + (int64_t)h * p.d + 8 * c8;
  for (int t = tl; t < p.tokens; t += tpp) {
    const u32x4 w = *(const u32x4*)(base + (int64_t)t * p.x_stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[2 * j] = fmaxf(m[2 * j], fabsf(bf16_lo(w[j])));
      m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(bf16_hi(w[j])));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[threadIdx.x][j] = m[j];
  __syncthreads();
  if (threadIdx.x < p.d) {                             // channel c = threadIdx.x
    const int c = threadIdx.x, cc = c >> 3, j = c & 7;
    float a = 0.f;
    for (int l = 0; l < tpp; ++l) a = fmaxf(a, part[l * cpr + cc][j]);
    part[c][8] = a;
  }
  __syncthreads();
  if (p.granularity == 2) {
    if (threadIdx.x < p.d) p.scales[(int64_t)h * p.d + threadIdx.x] = scale_of(part[threadIdx.x][8]);
  } else if (threadIdx.x == 0) {
    float a = 0.f;
    for (int c = 0; c < p.d; ++c) a = fmaxf(a, part[c][8]);
    p.scales[h] = scale_of(a);
  }
}

constexpr int kAmaxChunk = 256;                        // tokens per partial maximum

// Channel maxima of one (chunk, head): partial[chunk][h][c].
__global__ __launch_bounds__(256) void fp8_amax_partial_kernel(QuantParams p, float* partial) {
  __shared__ float part[256][9];
  const int ch = blockIdx.x, h = blockIdx.y;
  const int cpr = p.d >> 3;
  const int c8 = threadIdx.x % cpr, tl = threadIdx.x / cpr, tpp = 256 / cpr;
  const int t0 = ch * kAmaxChunk, t1 = min(t0 + kAmaxChunk, p.tokens);
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* base = p.x + (int64_t)h * p.d + 8 * c8;
  for (int t = t0 + tl; t < t1; t += tpp) {
    const u32x4 w = *(const u32x4*)(base + (int64_t)t * p.x_stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[2 * j] = fmaxf(m[2 * j], fabsf(bf16_lo(w[j])));
      m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(bf16_hi(w[j])));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[threadIdx.x][j] = m[j];
  __syncthreads();
  if (threadIdx.x < p.d) {
    const int c = threadIdx.x, cc = c >> 3, j = c & 7;
    float a = 0.f;
    for (int l = 0; l < tpp; ++l) a = fmaxf(a, part[l * cpr + cc][j]);
    partial[((int64_t)ch * p.heads + h) * p.d + c] = a;
  }
}

// Maximum over the chunks of head h (chunk order), then the scales.
__global__ __launch_bounds__(256) void fp8_amax_final_kernel(QuantParams p, const float* partial, int chunks) {
  __shared__ float cm[256];
  const int h = blockIdx.x, c = threadIdx.x;
  float a = 0.f;
  if (c < p.d)
    for (int k = 0; k < chunks; ++k) a = fmaxf(a, partial[((int64_t)k * p.heads + h) * p.d + c]);
  cm[c] = a;
  __syncthreads();
  if (p.granularity == 2) {
    if (c < p.d) p.scales[(int64_t)h * p.d + c] = scale_of(a);
  } else if (c == 0) {
    float b = 0.f;
    for (int j = 0; j < p.d; ++j) b = fmaxf(b, cm[j]);
    p.scales[h] = scale_of(b);
  }
}

// One thread per 8 consecutive values of a (token, head) row; the cpr threads
// of a row are adjacent lanes of one wave.  Granularity 0 reduces the row's
// amax across them and writes the row's scale.
__global__ __launch_bounds__(256) void fp8_quant_kernel(QuantParams p) {
  const int cpr = p.d >> 3;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.tokens * p.heads;
  const bool live = g < rows * cpr;
  const int64_t row = live ? g / cpr : 0;
  const int c8 = (int)(g - (g / cpr) * cpr);
  const int t = (int)(row / p.heads), h = (int)(row - (int64_t)t * p.heads);
  u32x4 w = (u32x4){0u, 0u, 0u, 0u};
  if (live) w = *(const u32x4*)(p.x + (int64_t)t * p.x_stride + (int64_t)h * p.d + 8 * c8);
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_lo(w[j]);
    v[2 * j + 1] = bf16_hi(w[j]);
  }
  float sc;
  if (p.granularity == 0) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
    for (int o = 1; o < cpr; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));   // cpr lanes of the row
    sc = scale_of(a);
    if (live && c8 == 0) p.scales[row] = sc;
  }
  if (!live) return;
  u32x2 out;
  if (p.granularity == 2) {
    const floatx4 s0 = *(const floatx4*)(p.scales + (int64_t)h * p.d + 8 * c8);
    const floatx4 s1 = *(const floatx4*)(p.scales + (int64_t)h * p.d + 8 * c8 + 4);
    const float iv[8] = {1.f / s0[0], 1.f / s0[1], 1.f / s0[2], 1.f / s0[3],
                         1.f / s1[0], 1.f / s1[1], 1.f / s1[2], 1.f / s1[3]};
    out[0] = cvt2<false>(v[0] * iv[0], v[1] * iv[1], 0u);
    out[0] = cvt2<true>(v[2] * iv[2], v[3] * iv[3], out[0]);
    out[1] = cvt2<false>(v[4] * iv[4], v[5] * iv[5], 0u);
    out[1] = cvt2<true>(v[6] * iv[6], v[7] * iv[7], out[1]);
  } else {
    if (p.granularity == 1) sc = p.scales[h];
    const float iv = 1.f / sc;
    out[0] = cvt2<false>(v[0] * iv, v[1] * iv, 0u);
    out[0] = cvt2<true>(v[2] * iv, v[3] * iv, out[0]);
    out[1] = cvt2<false>(v[4] * iv, v[5] * iv, 0u);
    out[1] = cvt2<true>(v[6] * iv, v[7] * iv, out[1]);
  }
  *(u32x2*)(p.out + (row * cpr + c8) * 8) = out;
}

}  // namespace

hipError_t launch_quant_fp8(const QuantParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.tokens * p.heads * (p.d >> 3);
  if (p.heads == 0) return hipSuccess;
  if (p.granularity != 0) {
    if (p.tokens >= 1024) {
      // partial maxima [chunks][heads][d] floats in the code buffer
      // ([tokens][heads][d] bytes >= 4 x that size from 1024 tokens on)
      const int chunks = (p.tokens + kAmaxChunk - 1) / kAmaxChunk;
      float* partial = (float*)p.out;
      hipLaunchKernelGGL(fp8_amax_partial_kernel, dim3(chunks, p.heads), dim3(256), 0, s, p, partial);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(fp8_amax_final_kernel, dim3(p.heads), dim3(256), 0, s, p, (const float*)partial, chunks);
    } else {
      hipLaunchKernelGGL(fp8_amax_kernel, dim3(p.heads), dim3(256), 0, s, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_quant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace vea
