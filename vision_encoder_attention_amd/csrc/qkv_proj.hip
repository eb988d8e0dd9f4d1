// Fused QKV projection with a rotary-embedding epilogue, for gfx950.
//
// The projection that feeds qkv_rope multiplies the tokens by one fused
// weight holding Wq | Wk | Wv side by side ([hidden, 3 * hidden] in
// 「从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash - Prefill」 section
// 3.1; here [hidden, (Hq + 2 Hkv) d]).  The pages advise fusing the
// memory-bound work around such a product into it
// (「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈性能」 section 5.2, fourth
// point): here the rotation of Q and K is applied to the fp32 accumulators
// before anything is stored, so the projection output never makes the round
// trip through HBM that a separate qkv_rope step costs, and it is rounded to
// bf16 once instead of twice.
//
// Product: C^T = W^T X^T on v_mfma_f32_32x32x16_bf16, so that the accumulator
// of a lane holds one token and, for each block of 32 features, four runs of
// four consecutive features: every rotation pair (2i, 2i + 1) sits in one
// lane and the epilogue needs no exchange between lanes.
//   * Workgroup tile: 256 features x 256 tokens; 8 waves as 2 x 4, each
//     128 features x 64 tokens (4 x 2 accumulator blocks, 128 registers),
//     two waves per SIMD.  The tile moves 128 flops per byte from L2 to LDS.
//   * Contraction in steps of 32 through a four-stage LDS ring (128 KB)
//     filled by buffer loads straight into LDS; a step's loads are issued
//     three steps before use, one barrier per step.
//   * W stage [32 k][256 features] (512-byte rows, 16-byte chunks XOR-swizzled
//     by 4 * (k % 4)): the W^T operand comes from ds_read_b64_tr_b16, 4 rows x
//     4 chunks per 32 lanes, all 64 banks once.
//   * X stage [256 tokens][32 k] (64-byte rows, chunks swizzled by
//     (token / 4) % 4): the X^T operand is one 16-byte read per lane, 16 rows
//     per 16 lanes on distinct banks.
//   * Workgroups are numbered so that consecutive tiles (the feature tiles of
//     one token block) land on the same XCD and share its L2.
// Epilogue per accumulator block: bias (optional), then the rotation with the
// per-token (cos, sin) table, then bf16 (nearest even); the two lane halves
// trade half-runs so that each lane stores whole 16-byte runs of 8 features
// into q, k or v.  A block
// of 32 features never straddles a head or the Q | K | V boundaries (head_dim
// is a multiple of 32), so the branch is uniform.
//
// The table (rope_cos_sin_kernel) holds, per token and pair, the cosine and
// sine of the pair's angle, formed and evaluated in fp64 and rounded to fp32
// (trigonometry in at least fp32: 「AMD MI250部署DeepSeek-V4-Flash：先修正确性
// 再谈性能」 section 4.1), the same values qkv_rope computes.  The positions
// are the same for every layer of an encoder, so a caller builds it once.
#include "vea_internal.h"

#include <math.h>

namespace vea {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ds_read_b64_tr_b16: each lane of a 16-lane group reads 8 bytes (row i/4,
// columns 4(i%4)..+3 of a 4 x 16 bf16 block) and receives column i of the
// block (its 4 rows, in row order).
__device__ __forceinline__ u32x2 lds_read_tr(const void* p) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

constexpr int kPF = kProjTileF;              // features per workgroup
constexpr int kPT = kProjTileT;              // tokens per workgroup
constexpr int kPK = kProjStepK;              // contraction per stage
constexpr int kThreads = 512;                // 8 waves
constexpr int kWTile = kPK * kPF * 2;        // 16 KB
constexpr int kXTile = kPT * kPK * 2;        // 16 KB
constexpr int kWLoads = kWTile / (kThreads * 16); // 16-byte DMA loads per lane
constexpr int kXLoads = kXTile / (kThreads * 16);
static_assert(kWLoads == 2 && kXLoads == 2, "the step's vmcnt below counts 4 loads per lane");
constexpr unsigned kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit format

// The table, bias and outputs also come as separate restrict-qualified
// arguments: the compiler may then issue the epilogue's table and bias loads
// ahead of its stores instead of one load-use round trip per block.
__global__ __launch_bounds__(kThreads, 1) void qkv_proj_kernel(ProjParams p, const float* __restrict__ cs_tab,
                                                               const uint16_t* __restrict__ bias,
                                                               uint16_t* __restrict__ out_q,
                                                               uint16_t* __restrict__ out_k,
                                                               uint16_t* __restrict__ out_v) {
  __shared__ __attribute__((aligned(1024))) unsigned char w0[kWTile];
  __shared__ __attribute__((aligned(1024))) unsigned char w1[kWTile];
  __shared__ __attribute__((aligned(1024))) unsigned char w2[kWTile];
  __shared__ __attribute__((aligned(1024))) unsigned char w3[kWTile];
  __shared__ __attribute__((aligned(1024))) unsigned char x0[kXTile];
  __shared__ __attribute__((aligned(1024))) unsigned char x1[kXTile];
  __shared__ __attribute__((aligned(1024))) unsigned char x2[kXTile];
  __shared__ __attribute__((aligned(1024))) unsigned char x3[kXTile];

  // Workgroup b runs on XCD b % 8; give each XCD a contiguous range of tiles.
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int per = nblk >> 3, rem = nblk & 7, xcd = bid & 7, slot = bid >> 3;
  const int lid = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int tt = lid / p.ftiles, ft = lid - tt * p.ftiles;
  const int t0 = tt * kPT, n0 = ft * kPF;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;

  // ---- DMA: lane slot sl of the wave's 1 KB blocks holds one 16-byte chunk.
  const int64_t xsb = p.x_stride * 2, wsb = p.w_stride * 2;
  int xoff[kXLoads], woff[kWLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int sl = (wave * kXLoads + i) * 64 + lane;
    const int r = sl >> 2, lc = (sl & 3) ^ ((r >> 2) & 3);
    xoff[i] = (int)(r * xsb) + 16 * lc;
  }
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) {
    const int sl = (wave * kWLoads + i) * 64 + lane;
    const int r = sl >> 5, lc = (sl & 31) ^ (4 * (r & 3));
    woff[i] = (int)(r * wsb) + 16 * lc;
  }
  // Bytes from the tile's first element to the end of the last valid one:
  // token rows past the end and the tail of W read as zeros.
  const unsigned char* xbase = (const unsigned char*)p.x + (int64_t)t0 * xsb;
  const int64_t xlast = (int64_t)(p.tokens - t0 - 1) * xsb + (int64_t)p.hidden * 2;
  const unsigned char* wbase = (const unsigned char*)p.w + (int64_t)n0 * 2;
  const int64_t wlast = (int64_t)(p.hidden - 1) * wsb + (int64_t)(p.n_feat - n0) * 2;
  // A step past the contraction (s >= nk) gets zero-sized buffers: its loads
  // touch no memory and fill the stage with zeros, which add nothing.
  const int nk = p.hidden / kPK;
  auto issue = [&](int s, unsigned char* wd, unsigned char* xd) {
    const bool real = s < nk;
    const int64_t kb = (int64_t)s * kPK * 2, wb = (int64_t)s * kPK * wsb;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(xbase + (real ? kb : 0)), (short)0, real ? (int)(xlast - kb) : 0, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(wbase + (real ? wb : 0)), (short)0, real ? (int)(wlast - wb) : 0, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (__attribute__((address_space(3))) void*)(wd + (wave * kWLoads + i) * 1024), 16, (unsigned)woff[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (__attribute__((address_space(3))) void*)(xd + (wave * kXLoads + i) * 1024), 16, (unsigned)xoff[i], 0, 0, 0);
  };

  // ---- per-lane LDS read offsets (loop invariant)
  // X^T operand of token block tb, k-step ks: token row 64 wt + 32 tb + l32,
  // logical chunk 2 ks + g2 (k = 16 ks + 8 g2 .. + 7).
  int xrd[2][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int r = 64 * wt + 32 * tb + l32;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) xrd[tb][ks] = r * 64 + 16 * ((2 * ks + g2) ^ ((r >> 2) & 3));
  }
  // W^T operand of feature block fb (features 128 wf + 32 fb + l32): the
  // 16-lane group reads k rows 16 ks + 8 g2 + (i16 / 4) (slots 0..3) and the
  // same + 4 (slots 4..7), so slot j of the lane holds k = 16 ks + 8 g2 + j,
  // the k that slot j of the X^T operand holds.
  const int i16 = lane & 15, nhalf = (lane >> 4) & 1;
  const int wrow = (8 * g2 + (i16 >> 2)) * (kPF * 2);
  int wrd[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) {
    const int lc = 4 * (4 * wf + fb) + 2 * nhalf + ((i16 & 3) >> 1);
    wrd[fb] = wrow + 16 * (lc ^ (4 * ((i16 >> 2) & 3))) + 8 * (i16 & 1);
  }

  floatx16 acc[4][2];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) acc[fb][tb] = (floatx16){};

  auto compute = [&](const unsigned char* ws_, const unsigned char* xs_) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 b[2], a[4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) b[tb] = *(const u32x4*)(xs_ + xrd[tb][ks]);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const unsigned char* pa = ws_ + ks * 16 * (kPF * 2) + wrd[fb];
        const u32x2 lo = lds_read_tr(pa);
        const u32x2 hi = lds_read_tr(pa + 4 * (kPF * 2));
        a[fb] = (u32x4){lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[fb]), as_bf16x8(b[tb]), acc[fb][tb], 0, 0, 0);
    }
  };

  // ---- four-stage pipeline: step s reads stage s % 4, then refills the
  // stage of step s - 1 with step s + 3.  Stages are distinct arrays and the
  // loop body (four steps, a multiple of four in all, the extra ones on zero
  // stages) has no branch, so the compiler can tell which stage each DMA
  // writes.
  auto step = [&](const unsigned char* wr_, const unsigned char* xr_) {
    // This lane's loads of this step have landed (the eight issued after
    // them, for the next two steps, may still be in flight); its reads of
    // the previous step are done.  After the barrier the same holds for every wave, and
    // the previous step's stage may be refilled.  (s_waitcnt through the
    // builtin, so that the compiler's own wait placement takes it into
    // account; the expcnt field stays at its maximum, 7.)
    __builtin_amdgcn_s_waitcnt(0x0078);                   // vmcnt(8) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    compute(wr_, xr_);
  };
  issue(0, w0, x0);
  issue(1, w1, x1);
  issue(2, w2, x2);
  for (int s = 0; s < nk; s += 4) {
    step(w0, x0);
    issue(s + 3, w3, x3);
    step(w1, x1);
    issue(s + 4, w0, x0);
    step(w2, x2);
    issue(s + 5, w1, x1);
    step(w3, x3);
    issue(s + 6, w2, x2);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);                     // the last (zero) loads: vmcnt(0)

  // ---- epilogue, block by block (8 blocks of 32 features x 32 tokens per
  // lane set).  The table entries and bias of block i + 1 are loaded while
  // block i is finished, so each round trip to memory is paid about once.
  const int qn = p.hq * p.d, kn = (p.hq + p.hkv) * p.d;
  const int half = p.d >> 1;
  struct Blk {
    bool live, rot;
    int t, base, heads, f0, dd0;
    uint16_t* out;
  };
  auto blk = [&](int i) {
    const int tb = i >> 2, fb = i & 3;
    Blk b;
    const int nb = n0 + 128 * wf + 32 * fb;               // first feature of the block (uniform)
    b.t = t0 + 64 * wt + 32 * tb + l32;
    b.live = nb < p.n_feat;
    if (nb < qn) {
      b.out = out_q; b.base = 0; b.heads = p.hq;
    } else if (nb < kn) {
      b.out = out_k; b.base = qn; b.heads = p.hkv;
    } else {
      b.out = out_v; b.base = kn; b.heads = p.hkv;
    }
    b.rot = cs_tab != nullptr && nb < kn;
    b.f0 = nb - b.base;                                   // feature inside the region
    b.dd0 = b.f0 % p.d;                                   // inside the head (multiple of 32)
    return b;
  };
  const bool rh = p.rot_span != 0 && cs_tab != nullptr;   // rotate-half pairing (pre-pass below)
  // Operands of one block: (cos, sin) of pair entries e, e + 1 of each run a
  // (e = (dd0 + 8a + 4 g2) / 2) and the bias of the run's 4 features.
  struct Ops {
    floatx4 cs[4];
    u32x2 bb[4];
  };
  auto load_ops = [&](const Blk& b, Ops& o) {
    if (!b.live || rh) return;
    const int tc = b.t < p.tokens ? b.t : p.tokens - 1;
    if (b.rot) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        o.cs[a] = *(const floatx4*)(cs_tab + ((int64_t)tc * half + ((b.dd0 + 8 * a + 4 * g2) >> 1)) * 2);
    }
    if (bias != nullptr) {
#pragma unroll
      for (int a = 0; a < 4; ++a) o.bb[a] = *(const u32x2*)(bias + b.base + b.f0 + 8 * a + 4 * g2);
    }
  };
  // Rotate-half pairs (f, f + span/2): a head lies inside the wave's 128
  // features (d 64 or 128), so the partner of a first element sits in this
  // lane, span/2 / 32 blocks on at the same register (span/2 >= 32) or two
  // runs on in the same block (span/2 = 16).  In that mode this pass adds the
  // bias and rotates in the accumulators, and the blocks below only store.
  if (rh) {
    const int span = p.rot_span, hs = span >> 1;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const Blk b0 = blk(4 * tb);
      const int tc = b0.t < p.tokens ? b0.t : p.tokens - 1;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const Blk b = blk(4 * tb + fb);
        if (!b.live || bias == nullptr) continue;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x2 bb = *(const u32x2*)(bias + b.base + b.f0 + 8 * a + 4 * g2);
          acc[fb][tb][4 * a] += bf16_lo(bb[0]);
          acc[fb][tb][4 * a + 1] += bf16_hi(bb[0]);
          acc[fb][tb][4 * a + 2] += bf16_lo(bb[1]);
          acc[fb][tb][4 * a + 3] += bf16_hi(bb[1]);
        }
      }
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const Blk b = blk(4 * tb + fb);
        if (!b.live || !b.rot) continue;
        auto turn = [&](floatx16& A, int ia, floatx16& B, int ib, int e) {
          const float2 cv = *(const float2*)(cs_tab + ((int64_t)tc * half + e) * 2);
          const float x0 = A[ia], x1 = B[ib];
          A[ia] = x0 * cv.x - x1 * cv.y;
          B[ib] = x0 * cv.y + x1 * cv.x;
        };
        if (hs >= 32) {
          if (b.dd0 % span >= hs) continue;               // a block of second elements
          // partner block fb + hs / 32 (< 4: the head is in the wave), chosen
          // by a compile-time index so that the accumulators stay in registers
          const int e0 = (b.dd0 / span) * hs + b.dd0 % span + 4 * g2;
          if (hs == 32) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                turn(acc[fb][tb], 4 * a + q, acc[fb < 3 ? fb + 1 : 3][tb], 4 * a + q, e0 + 8 * a + q);
          } else {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                turn(acc[fb][tb], 4 * a + q, acc[fb < 2 ? fb + 2 : 3][tb], 4 * a + q, e0 + 8 * a + q);
          }
        } else {                                          // span 32: partners two runs on
          const int e0 = (b.dd0 / span) * hs + 4 * g2;
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int q = 0; q < 4; ++q) turn(acc[fb][tb], 4 * a + q, acc[fb][tb], 4 * (a + 2) + q, e0 + 8 * a + q);
        }
      }
    }
  }
  auto finish = [&](const Blk& b, const Ops& o, const floatx16& c) {
    if (!b.live) return;
    uint32_t pk[4][2];                                    // bf16 of run a: 4 features 8a + 4 g2 + (0..3)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float y0 = c[4 * a], y1 = c[4 * a + 1], y2 = c[4 * a + 2], y3 = c[4 * a + 3];
      if (bias != nullptr && !rh) {
        y0 += bf16_lo(o.bb[a][0]);
        y1 += bf16_hi(o.bb[a][0]);
        y2 += bf16_lo(o.bb[a][1]);
        y3 += bf16_hi(o.bb[a][1]);
      }
      if (b.rot && !rh) {
        const floatx4 cs = o.cs[a];
        const float r0 = y0 * cs[0] - y1 * cs[1], r1 = y0 * cs[1] + y1 * cs[0];
        const float r2 = y2 * cs[2] - y3 * cs[3], r3 = y2 * cs[3] + y3 * cs[2];
        y0 = r0; y1 = r1; y2 = r2; y3 = r3;
      }
      pk[a][0] = pack_bf16x2(y0, y1);
      pk[a][1] = pack_bf16x2(y2, y3);
    }
    // Lanes l and l + 32 hold the two halves of every 8-feature run.  Swap so
    // that the low lane gets runs 1 and 3 whole and the high lane runs 0 and 2
    // (permlane32_swap(x, y): lanes 32..63 of x trade with lanes 0..31 of y).
    uint32_t run[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {                         // run pair (2h, 2h + 1)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(pk[2 * h + 1][j], pk[2 * h][j], false, false);
        run[h][j] = r[0];                                 // low: run 2h+1 features 0..3; high: run 2h 0..3
        run[h][2 + j] = r[1];                             // low: run 2h+1 features 4..7; high: run 2h 4..7
      }
    }
    if (b.t < p.tokens) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int fo = b.f0 + 8 * (2 * h + 1 - g2);
        *(u32x4*)(b.out + (int64_t)b.t * b.heads * p.d + fo) = (u32x4){run[h][0], run[h][1], run[h][2], run[h][3]};
      }
    }
  };
  Ops ops[2];
  Blk cur = blk(0);
  load_ops(cur, ops[0]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    Blk nxt;
    if (i + 1 < 8) {
      nxt = blk(i + 1);
      load_ops(nxt, ops[(i + 1) & 1]);
    }
    finish(cur, ops[i & 1], acc[i & 3][i >> 2]);
    cur = nxt;
  }
}

// One thread per (token, pair): the angle pos * theta^(-2i/span) and its sine
// and cosine in fp64, stored as fp32 (cos, sin).  1D: span d, pair i = e.  2D:
// pairs [0, d/4) turn with the grid row, [d/4, d/2) with the grid column, span
// d/2, pair i = e mod d/4.
__global__ __launch_bounds__(256) void rope_cos_sin_kernel(RopeTableParams p) {
  const int half = p.d >> 1;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.tokens * half) return;
  const int t = (int)(idx / half), e = (int)(idx - (int64_t)t * half);
  double pos, expo;
  if (p.pos_dims == 1) {
    pos = (double)p.pos[t];
    expo = -2.0 * (double)e / (double)p.d;
  } else {
    const int q4 = p.d >> 2;
    const int axis = e >= q4 ? 1 : 0;
    pos = (double)p.pos[2 * (int64_t)t + axis];
    expo = -2.0 * (double)(e - axis * q4) / (double)(p.d >> 1);
  }
  const double ang = pos * exp2(expo * log2(p.theta));
  double sv, cv;
  sincos(ang, &sv, &cv);
  *(float2*)(p.out + 2 * idx) = make_float2((float)cv, (float)sv);
}

}  // namespace

hipError_t launch_qkv_proj(const ProjParams& p, hipStream_t s) {
  if (p.tokens == 0) return hipSuccess;
  if (p.hidden % kPK != 0 || p.hidden < kPK || p.d % 32 != 0 || p.ftiles != (p.n_feat + kPF - 1) / kPF)
    return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)p.ftiles * ((p.tokens + kPT - 1) / kPT);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qkv_proj_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, p, p.cs, p.bias, p.q, p.k, p.v);
  return hipGetLastError();
}

hipError_t launch_rope_cos_sin(const RopeTableParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.tokens * (p.d >> 1);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_cos_sin_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace vea
