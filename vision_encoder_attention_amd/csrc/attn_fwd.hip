// Blockwise scaled-dot-product attention forward for gfx950 (CDNA4, wave64).
//
// What is computed (per sequence b of a cu_seqlens-packed batch, query head h,
// key/value head g = h / (Hq/Hkv), query row i):
//   o_i = sum_j softmax_j(scale * q_i.k_j) v_j over the allowed keys j,
//   lse_i = ln sum_j exp(scale * q_i.k_j)
// Page titles cited:
//   [3090]   「DeepSeek V4.1 上 4×RTX 3090：视觉链路的两个坑和修复」
//   [MI250]  「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈性能」
//   [SGLang] 「从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash - Prefill」
//   [V32]    「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」
//
// Structure (bf16 path):
//   * One workgroup = 4 waves = BM (128) query rows of one (sequence, piece,
//     head).  Query pieces of qb rows are the scheduling unit of [3090]
//     section 三; a tile never straddles a piece and all addressing inside a
//     piece is relative to the piece's own rows (there is no S/P buffer in
//     global memory at all: S and P live in registers).
//   * The key loop walks BN = 64 keys per step up to the sequence's own key
//     bound (the varlen loop of [SGLang] section 3.2), K and V tiles staged
//     through LDS, double buffered, with 16-byte coalesced global loads.
//   * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32
//     accumulation, [MI250] sections 3.1 / 4.1): the accumulator layout gives
//     each lane ONE query row and 32 of the step's keys, so the row max needs
//     a single cross-lane exchange and the row sum is lane-local until the end.
//   * Online softmax in fp32 ([V32] section 进一步探索 eq. (1)(2)): running max
//     m, rescale alpha = 2^(m_old - m_new), running sum l; exponentials via
//     v_exp_f32 with log2(e) folded into the scale.  The reference max moves
//     lazily and is not recomputed per tile: P is formed with the current
//     reference and a tile whose P grows too large (or a row still without
//     a reference) takes a rare path that recomputes its logits, moves the
//     reference and rescales O and l.
//   * O^T += V^T P^T with the same MFMA; P is rounded to bf16 (RNE) in
//     registers, V is stored transposed in LDS so each lane reads 4 keys of one
//     column as one 8-byte LDS read.  O^T's layout again gives each lane one
//     query row, so the per-row rescale touches only the lane's own registers.
//   * Masking excludes keys (weight exactly 0) rather than adding a bias
//     ([MI250] section 3.3); only tiles that cross the causal diagonal or the
//     key tail evaluate the mask.
//   * No atomics; each output element and each lse entry has one writer, so
//     runs are bitwise reproducible ([MI250] section 3.2).
#include "vea_internal.h"

#include <float.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

#include "../../include/vea.h"

namespace vea {
namespace {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // Round-to-nearest-even conversion of a pair: one v_cvt_pk_bf16_f32.
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2v));
}

// IEEE maximum (NaN-propagating); maps to v_maximum3_f32 without the
// canonicalising moves fmaxf needs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Decode the workgroup id into (sequence b, query head h, tile t).  Tiles are
// issued heaviest-first (largest tile index first: under a causal mask it has
// the most keys).  With xcd_map, all query heads of one key/value head are
// kept on one XCD (workgroups are dispatched round-robin over the 8 XCDs), so
// the workgroups that stream the same K/V share that XCD's L2.
__device__ __forceinline__ void decode_unit(const DenseParams& p, int id, int& b, int& h, int& t) {
  int trev;
  if (p.xcd_map) {
    const int xcd = id & 7, j = id >> 3;
    const int nh = p.hq >> 3;
    const int per_t = p.batch * nh;
    trev = j / per_t;
    const int rem = j - trev * per_t;
    b = rem / nh;
    const int hl = rem - b * nh;
    const int a = hl / p.group, gi = hl - a * p.group;
    h = (xcd + 8 * a) * p.group + gi;
  } else {
    const int per_t = p.batch * p.hq;
    trev = id / per_t;
    const int rem = id - trev * per_t;
    b = rem / p.hq;
    h = rem - b * p.hq;
  }
  t = p.tiles_per_seq - 1 - trev;
}

struct TileRange {
  int qs, ks, len_q, len_k;   // sequence base rows and lengths
  int row0, row_end;          // local query rows [row0, row_end) of this tile
  int kend;                   // keys [0, kend) are needed by some row
  int kfull;                  // keys [0, kfull) are allowed for every row
};

__device__ __forceinline__ bool tile_range(const DenseParams& p, int b, int t, int bm, bool causal, TileRange& r) {
  const int qs = clampi(p.cu_q[b], 0, p.total_q);
  const int qe = clampi(p.cu_q[b + 1], qs, p.total_q);
  const int ks = clampi(p.cu_k[b], 0, p.total_k);
  const int ke = clampi(p.cu_k[b + 1], ks, p.total_k);
  r.qs = qs;
  r.ks = ks;
  r.len_q = qe - qs;
  r.len_k = ke - ks;
  const int piece = t / p.tiles_per_piece;
  const int tip = t - piece * p.tiles_per_piece;
  const int pbase = piece * p.qb;                       // piece-local row base
  const int row_lim = min(pbase + p.qb, r.len_q);
  r.row0 = pbase + tip * bm;
  if (r.row0 >= row_lim) return false;
  r.row_end = min(r.row0 + bm, row_lim);
  if (causal) {
    const int off = r.len_k - r.len_q;                  // bottom-right alignment
    r.kend = clampi(r.row_end + off, 0, r.len_k);
    r.kfull = clampi(r.row0 + off + 1, 0, r.len_k);
  } else {
    r.kend = r.len_k;
    r.kfull = r.len_k;
  }
  return true;
}

// Decode units (one query token per sequence): unit (sequence b, key/value
// head h) has as rows the dec_group query heads of that key/value head, which
// all read the same K/V; the keys are the sequence's cache, all visible.
__device__ __forceinline__ void decode_range(const DenseParams& p, int b, TileRange& r) {
  const int ks = clampi(p.cu_k[b], 0, p.total_k);
  const int ke = clampi(p.cu_k[b + 1], ks, p.total_k);
  r.qs = b;
  r.ks = ks;
  r.len_q = p.dec_group;
  r.len_k = ke - ks;
  r.row0 = 0;
  r.row_end = p.dec_group;
  r.kend = r.len_k;
  r.kfull = r.len_k;
}

// =============================================================== bf16 path

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Transposed LDS read: within each group of 16 lanes, lane i points at 8 bytes
// (row i/4, columns 4(i%4)..+3 of a 4 x 16 bf16 block) and receives column i
// of that block (its 4 rows).
__device__ __forceinline__ u32x2 lds_read_tr(const void* p) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float lane_swap_max(float x) {
  // max with the lane 32 apart (the other half of the wave holds the same row)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_swap_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct Cfg {
  static constexpr int BM = kDenseBM;                   // 4 waves x 32 query rows
  static constexpr int BN = 64;                         // keys per step
  static constexpr int THREADS = 256;
  static constexpr int CPR = D / 8;                     // 16-byte chunks per K/V row
  static constexpr int TILE = BN * D * 2;               // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;                // K + V
  static constexpr int LOADS = TILE / (THREADS * 16);   // 16-byte DMA loads per lane per tile
  static_assert(LOADS == 2 || LOADS == 4, "tile split");
  // XOR swizzle of the 16-byte chunks of a row.  The LDS has 64 four-byte
  // banks and a ds_read_b64_tr_b16 serves 32 lanes per cycle.
  //  * V^T reads: 4 rows x 4 logical chunks per 32 lanes; rows r and r + 2
  //    (same bank half for d = 64; for d = 128 every row spans all banks)
  //    need disjoint physical chunk sets, so their swizzles differ in a bit
  //    above the low two.
  //  * K reads (ds_read_b128): 16 rows x one logical chunk, each row pair on
  //    a distinct chunk.
  // Both read kinds measure zero SQ_LDS_BANK_CONFLICT cycles with these
  // swizzles (the plain (r / 2) % 8 and r % 16 cost every V^T read 2 and 6).
  // The period is 16 rows, so rows r, r + 16 and r + 32 share a swizzle.
  static __device__ __forceinline__ int swz(int r) {
    if (D == 64) {
      const int x = (r >> 1) & 7;                       // bit-reversed row pair
      return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
    }
    return ((r & 3) << 2) | ((r >> 2) & 3);
  }
};

template <int D, bool CAUSAL, bool PAGED, bool DECODE = false>
__global__ __launch_bounds__(256, (D == 64 ? 3 : 2)) void attn_fwd_bf16_kernel(DenseParams p) {
  using C = Cfg<D>;
  // Two K stages and two V stages in distinct arrays: the compiler can then see
  // that a DMA into one stage never aliases reads of another, and does not wait.
  __shared__ __attribute__((aligned(1024))) unsigned char kst0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char kst1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vst0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vst1[C::TILE];

  // unit, and for a split unit of the last round, its key-range chunk
  const int slot = wg_slot(blockIdx.x, p.grid, p.wg_perm);
  int id = slot, chunk = 0;
  const bool split = id >= p.full_units;
  if (split) {
    const int u2 = id - p.full_units;
    const int tu = u2 / p.nsplit;
    chunk = u2 - tu * p.nsplit;
    id = p.full_units + tu;
  }
  int b, h, t;
  decode_unit(p, id, b, h, t);
  TileRange tr;
  if constexpr (DECODE) {
    decode_range(p, b, tr);
  } else {
    if (!tile_range(p, b, t, C::BM, CAUSAL, tr)) return;   // uniform over the workgroup
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g2 = lane >> 5;                 // which half of the wave
  const int kvh = h / p.group;

  // ---- this lane's query row (local index in the sequence)
  const int qi = tr.row0 + wave * 32 + l32;
  const bool qvalid = qi < tr.row_end;
  // A wave whose 32 rows are all past the tile's end (the short last tile of
  // a piece) still issues its share of the K/V DMA and meets every barrier,
  // but skips the MFMA and softmax work.  Only where the branch costs no
  // extra spills: elsewhere (d 128, causal, decode) it measured no faster.
  constexpr bool SKIP_DEAD = !CAUSAL && D == 64 && !DECODE;
  const bool live = !SKIP_DEAD || tr.row0 + __builtin_amdgcn_readfirstlane(wave) * 32 < tr.row_end;

  // ---- Q fragment (B operand of S^T = K Q^T): Q[qi][16 ks + 8 g2 .. +7]
  u32x4 qf[D / 16];
  {
    // decode: row qi of unit (b, h) is query head h * dec_group + qi of token b
    const uint16_t* src = DECODE ? (const uint16_t*)p.q + (int64_t)b * p.q_stride +
                                       (int64_t)(h * p.dec_group + (qvalid ? qi : 0)) * D + 8 * g2
                                 : (const uint16_t*)p.q + (int64_t)(tr.qs + (qvalid ? qi : tr.row0)) * p.q_stride +
                                       (int64_t)h * D + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 v = *(const u32x4*)(src + 16 * ks);
      qf[ks] = qvalid ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  // Negative scale: negate Q (exact sign-bit flip) so the exponent scale is positive.
  float c = fabsf(p.scale) * kLog2e;
  if (p.scale < 0.f) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  c = fmaxf(c, FLT_MIN);   // scale 0: every logit becomes ~0, masked ones stay -inf

  const int kend_i = CAUSAL ? clampi(qi + tr.len_k - tr.len_q + 1, 0, tr.len_k) : tr.len_k;

  // Key tiles [kt0, kt0 + n_tiles) of this workgroup: all of them, or its
  // chunk's share of a split unit.  Below, kt counts tiles from kt0.
  const int n_all = (tr.kend + C::BN - 1) / C::BN;
  int kt0 = 0, n_tiles = n_all;
  if (split) {
    kt0 = (n_all * chunk) / p.nsplit;
    n_tiles = (n_all * (chunk + 1)) / p.nsplit - kt0;
  }

  // ---- DMA of K/V tiles straight into LDS (buffer loads, no register staging).
  // Lane slot sl of the wave's 1 KB destination block holds row sl / CPR,
  // physical chunk sl % CPR = logical chunk ^ swz(row).  Rows past the needed
  // key range read as zeros (beyond the buffer's record count).
  const int64_t ksb = p.k_stride * 2, vsb = p.v_stride * 2;
  int voff_k[C::LOADS], voff_v[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int sl = (wave * C::LOADS + i) * 64 + lane;
    const int r = sl / C::CPR, ch = (sl % C::CPR) ^ C::swz(r);
    voff_k[i] = (int)(r * ksb) + 16 * ch;
    voff_v[i] = (int)(r * vsb) + 16 * ch;
  }
  // Key row j of this sequence: row tr.ks + j of the packed K/V, or, for a
  // paged cache, row j's page looked up in the sequence's block-table row.
  const unsigned char* kbase_ptr =
      (const unsigned char*)p.k + ((PAGED ? 0 : (int64_t)tr.ks * p.k_stride) + (int64_t)kvh * D) * 2;
  const unsigned char* vbase_ptr =
      (const unsigned char*)p.v + ((PAGED ? 0 : (int64_t)tr.ks * p.v_stride) + (int64_t)kvh * D) * 2;
  // Physical row of the sequence's key j.  A tile never spans two pages (page
  // sizes are multiples of the tile height).
  auto phys_row = [&](int j) -> int64_t {
    if constexpr (!PAGED) return j;
    const int64_t page = p.block_table[(int64_t)b * p.max_pages + (j >> p.page_shift)];
    return (page << p.page_shift) | (j & ((1 << p.page_shift) - 1));
  };
  auto row_ptr = [&](const unsigned char* base, int64_t sb, int j) -> const unsigned char* {
    return base + phys_row(j) * sb;
  };
  // First physical row of tile kt, 0 past the key range (such a tile is never
  // loaded).  The paged pipeline below reads these block-table entries two
  // tiles ahead of their DMA, so the lookup's latency stays off the issue.
  auto tile_row = [&](int kt) -> int64_t {
    const int j = (kt0 + kt) * C::BN;
    return j < tr.kend ? phys_row(j) : 0;
  };
  auto issue_tile = [&](int kt, int64_t row0, const unsigned char* base, int64_t sb, const int* voff,
                        unsigned char* stage) {
    const int rows = min(tr.kend - (kt0 + kt) * C::BN, C::BN);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + row0 * sb), (short)0, (int)(rows * sb), 0x00020000);
    unsigned char* dst = stage + wave * C::LOADS * 1024;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                               (unsigned)voff[i], 0, 0, 0);
  };
  // rows of tiles kt, kt + 1, kt + 2 at the top of iteration kt (paged only)
  int64_t rv = 0, rk = 0, rn = 0;
  auto row_of = [&](int kt, int64_t pre) -> int64_t {
    if constexpr (PAGED) return pre;
    else return (int64_t)(kt0 + kt) * C::BN;
  };
  auto issue_k = [&](int kt, int64_t pre, unsigned char* stage) {
    issue_tile(kt, row_of(kt, pre), kbase_ptr, ksb, voff_k, stage);
  };
  auto issue_v = [&](int kt, int64_t pre, unsigned char* stage) {
    issue_tile(kt, row_of(kt, pre), vbase_ptr, vsb, voff_v, stage);
  };

  // ---- per-lane LDS read offsets (loop invariant)
  const int sw = C::swz(l32);                         // same for rows l32 and 32 + l32
  int koff[D / 16];                                   // K rows l32 (+32), chunk 2 ks + g2
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = l32 * D * 2 + 16 * ((2 * ks + g2) ^ sw);
  const int i16 = lane & 15, G16 = lane >> 4, nhalf = G16 & 1;
  const int vr0 = 4 * g2 + (i16 >> 2);                // key row of the first 4-key read (+ 16 st)
  int voff0[D / 32], voff1[D / 32];                   // V rows vr0 and vr0 + 8
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    const int chunk = 4 * nb + 2 * nhalf + ((i16 & 3) >> 1);
    voff0[nb] = vr0 * D * 2 + 16 * (chunk ^ C::swz(vr0)) + 8 * (i16 & 1);
    voff1[nb] = (vr0 + 8) * D * 2 + 16 * (chunk ^ C::swz(vr0 + 8)) + 8 * (i16 & 1);
  }

  floatx16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = (floatx16){};
  float m_used = -INFINITY;  // max used for exponentiation (times c, log2 domain)
  float l_run = 0.f;         // lane-partial sum of P
  float m_use = 0.f;         // m_used, or 0 while the row has none

  const int n_full = min(n_all, tr.kfull / C::BN) - kt0;   // (local) tiles no row needs masked

  // S^T = K Q^T for one tile: two independent 32-key accumulators, interleaved.
  auto qk = [&](const unsigned char* ks_, floatx16& s0, floatx16& s1) {
    s0 = (floatx16){};
    s1 = (floatx16){};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 a0 = *(const u32x4*)(ks_ + koff[ks]);
      const u32x4 a1 = *(const u32x4*)(ks_ + 32 * D * 2 + koff[ks]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qf[ks]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(qf[ks]), s1, 0, 0, 0);
    }
  };
  // Keys past a row's bound (tail of the sequence, causal diagonal) -> -inf.
  auto mask = [&](int kt, floatx16& s0, floatx16& s1) {
    const int j0 = (kt0 + kt) * C::BN + 4 * g2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + (r & 3);
      if (j >= kend_i) s0[r] = -INFINITY;
      if (j + 32 >= kend_i) s1[r] = -INFINITY;
    }
  };
  // Online softmax, part 1: row max of a finished tile's logits and the
  // (rare) move of the reference max.  The reference max of a row moves
  // lazily: only when the tile max exceeds it by more than 8 (log2 units), so
  // P stays below 2^8; the final lse uses the same reference, so the result
  // is exact in real arithmetic.  Returns the reference to subtract.
  auto softmax_ref = [&](const floatx16& s0, const floatx16& s1) -> float {
    float mx = vmax(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = vmax(vmax(mx, s0[r]), s1[r]);
    mx = lane_swap_max(mx);
    const float mx_sc = (mx == -INFINITY) ? -INFINITY : mx * c;
    const bool upd = mx_sc > m_used + 8.0f;
    if (__any(upd)) {
      asm volatile("; rare: move the reference max, rescale O and l" ::);
      const float m_new = upd ? mx_sc : m_used;
      const float alpha = upd ? fast_exp2(m_used - m_new) : 1.0f;
      m_used = m_new;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
      l_run *= alpha;
    }
    return (m_used == -INFINITY) ? 0.f : m_used;
  };
  // Common part: P = 2^(s c - m) with the current reference, rounded to
  // bf16 and packed, and this lane's fp32 sum of the tile's P.  A lane sum
  // above 2^13 (so some P above 2^8) or a row without a reference sends the
  // wave to the rare part, which recomputes the tile's logits from K in
  // global memory (they are not kept), moves the reference and recomputes
  // P.  k-slot j of lane half g2 in step st is key 16 st + 8 (j / 4) + 4 g2 +
  // j % 4 for both operands.
  auto softmax_p = [&](const floatx16& s0, const floatx16& s1, float mu, u32x4* pb) -> float {
    float tq[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const floatx16& sv = kb == 0 ? s0 : s1;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t w[4];
        float pr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e0 = fast_exp2(fmaf(sv[8 * hf + 2 * q], c, -mu));
          const float e1 = fast_exp2(fmaf(sv[8 * hf + 2 * q + 1], c, -mu));
          pr[q] = e0 + e1;
          w[q] = pack_bf16x2(e0, e1);
        }
        tq[2 * kb + hf] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
        pb[2 * kb + hf] = (u32x4){w[0], w[1], w[2], w[3]};
      }
    }
    return (tq[0] + tq[1]) + (tq[2] + tq[3]);
  };
  // S^T of key tile kt from K in global memory (rows past the key bound
  // clamped to the last one; they are masked).
  auto qk_global = [&](int kt, floatx16& s0, floatx16& s1) {
    const int r0 = (kt0 + kt) * C::BN;
    const unsigned char* pa = row_ptr(kbase_ptr, ksb, min(r0 + l32, tr.kend - 1)) + 16 * g2;
    const unsigned char* pb2 = row_ptr(kbase_ptr, ksb, min(r0 + 32 + l32, tr.kend - 1)) + 16 * g2;
    s0 = (floatx16){};
    s1 = (floatx16){};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 a0 = *(const u32x4*)(pa + 32 * ks);
      const u32x4 a1 = *(const u32x4*)(pb2 + 32 * ks);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qf[ks]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(qf[ks]), s1, 0, 0, 0);
    }
  };
  // O^T += V^T P^T with V read transposed from a V stage.
  auto pv = [&](const u32x4* pb, const unsigned char* vs_) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        const u32x2 lo = lds_read_tr(vs_ + st * 16 * D * 2 + voff0[nb]);
        const u32x2 hi = lds_read_tr(vs_ + st * 16 * D * 2 + voff1[nb]);
        const u32x4 a = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb[st]), o[nb], 0, 0, 0);
      }
    }
  };

  // ---- software pipeline over key tiles.  Iteration kt (1 <= kt <= n_tiles)
  // computes S of tile kt while it finishes tile kt-1 (softmax + P V), so the
  // QK^T MFMAs run under the softmax VALU work of the same wave.  K is staged
  // one tile ahead of V: iteration kt reads K(kt) and V(kt-1), and its DMA
  // refills the K stage of tile kt-1 with K(kt+1) and the V stage of tile
  // kt-2 with V(kt).  Stage parity is static per iteration (unrolled by two),
  // so the compiler sees that the DMA never aliases the stages being read.
  floatx16 sp0, sp1;                                  // logits of the tile being finished
  auto iter = [&](int kt, auto odd_tag, auto has_s_tag) {
    constexpr bool ODD = decltype(odd_tag)::value;      // parity of kt
    constexpr bool HAS_S = decltype(has_s_tag)::value;  // kt < n_tiles
    unsigned char* k_rd = ODD ? kst1 : kst0;          // K(kt)
    unsigned char* k_wr = ODD ? kst0 : kst1;          // K(kt+1)
    unsigned char* v_rd = ODD ? vst0 : vst1;          // V(kt-1)
    unsigned char* v_wr = ODD ? vst1 : vst0;          // V(kt)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this lane's DMA of K(kt), V(kt-1) landed
    __syncthreads();                                  // everyone's landed; the stages refilled below are consumed
    floatx16 sn0, sn1;
    if constexpr (HAS_S) {
      if (kt + 1 < n_tiles) issue_k(kt + 1, rk, k_wr);
      issue_v(kt, rv, v_wr);
      if constexpr (PAGED) {
        rv = rk;
        rk = rn;
        rn = tile_row(kt + 3);
      }
    }
    // QK^T of tile kt under the softmax of tile kt-1, then P V of tile kt-1
    if constexpr (HAS_S) {
      if (live) {
        qk(k_rd, sn0, sn1);
      } else {
        sn0 = (floatx16){};
        sn1 = (floatx16){};
      }
    }
    if (live) {
      u32x4 pb[4];
      float t = softmax_p(sp0, sp1, m_use, pb);
      if (__any(t > 8192.f || m_used == -INFINITY)) {
        asm volatile("; rare: recompute the logits, move the reference max, recompute P" ::);
        floatx16 r0, r1;
        qk_global(kt - 1, r0, r1);
        if (kt - 1 >= n_full) mask(kt - 1, r0, r1);
        m_use = softmax_ref(r0, r1);
        t = softmax_p(r0, r1, m_use, pb);
      }
      l_run += t;
      pv(pb, v_rd);
    }
    if constexpr (HAS_S) {
      if (kt >= n_full) {
        asm volatile("; masked tile" ::);
        mask(kt, sn0, sn1);
      }
      sp0 = sn0;
      sp1 = sn1;
    }
  };

  if (n_tiles > 0) {
    if constexpr (PAGED) rv = tile_row(0);
    issue_k(0, rv, kst0);
    issue_v(0, rv, vst0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (PAGED) {
      rv = tile_row(1);
      rk = tile_row(2);
      rn = tile_row(3);
    }
    if (1 < n_tiles) issue_k(1, rv, kst1);
    qk(kst0, sp0, sp1);
    if (0 >= n_full) mask(0, sp0, sp1);
    m_use = softmax_ref(sp0, sp1);                      // reference from the first tile
    int kt = 1;
    for (; kt + 1 < n_tiles; kt += 2) {                // kt odd here
      iter(kt, std::true_type{}, std::true_type{});
      iter(kt + 1, std::false_type{}, std::true_type{});
    }
    if (kt < n_tiles) {                                // one more tile with S (odd), then drain (even)
      iter(kt, std::true_type{}, std::true_type{});
      iter(kt + 1, std::false_type{}, std::false_type{});
    } else {                                           // drain at an odd kt
      iter(kt, std::true_type{}, std::false_type{});
    }
  }

  // ---- epilogue: O / l (bf16 RNE), lse = ln 2 * (m + log2 l)
  const float l_tot = lane_swap_add(l_run);
  if (split) {
    // partial result of this key range, per tile row: unnormalized O
    // (fp32), reference max m (log2 domain) and sum l
    const int wr = DECODE ? p.ws_rows : C::BM;          // rows per chunk
    float* w = p.ws + (size_t)(slot - p.full_units) * (wr * (D + 2));
    const int rl = wave * 32 + l32;                     // row within the tile
    if (DECODE && !qvalid) return;                      // decode: only the few real rows are merged
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(floatx4*)(w + rl * D + 32 * nb + 8 * r4 + 4 * g2) =
            (floatx4){o[nb][4 * r4], o[nb][4 * r4 + 1], o[nb][4 * r4 + 2], o[nb][4 * r4 + 3]};
    if (g2 == 0) {
      w[wr * D + rl] = m_used;
      w[wr * D + wr + rl] = l_tot;
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    uint16_t* dst = DECODE ? (uint16_t*)p.out + (int64_t)b * p.o_stride + (int64_t)(h * p.dec_group + qi) * D + 4 * g2
                           : (uint16_t*)p.out + (int64_t)(tr.qs + qi) * p.o_stride + (int64_t)h * D + 4 * g2;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const floatx16& ov = o[nb];
        const u32x2 w = (u32x2){pack_bf16x2(ov[4 * r4 + 0] * inv, ov[4 * r4 + 1] * inv),
                                pack_bf16x2(ov[4 * r4 + 2] * inv, ov[4 * r4 + 3] * inv)};
        *(u32x2*)(dst + 32 * nb + 8 * r4) = w;
      }
    const int64_t li = DECODE ? (int64_t)(h * p.dec_group + qi) * p.total_q + b : (int64_t)h * p.total_q + tr.qs + qi;
    if (p.lse != nullptr && g2 == 0) p.lse[li] = l_tot > 0.f ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ============================================ bf16, head_dim 64, non-causal
// The image case (non-causal, packed or paged K/V, no decode units).  At
// head_dim 64 a 64-key step holds 16 MFMAs per 32 query rows but the same
// softmax work per logit as at 128, so the kernel is bound by instruction
// issue and by the K/V staging rather than by the matrix cores.  Here a
// workgroup is 4 waves x 64 query rows (a 256-row tile: half the K/V DMA per
// flop of a 128-row tile), and each wave holds two independent 32-row
// blocks:
//   * every K and V^T operand read from LDS feeds two MFMAs (one per block),
//     half the LDS traffic per flop of a 32-row wave;
//   * the two blocks' logit -> softmax -> P V chains are independent, so one
//     block's exponentials issue while the other's MFMAs run.
// K and V of one step are staged together (double-buffered, one barrier per
// step).  The fast path forms P = 2^(s c) with no reference at all and
// checks that fp32 held (every lane sum of a tile below 2^100, every row sum
// at least 2^-100); a workgroup where it did not recomputes its key range on
// the careful path, the other kernel's lazily moved reference.
constexpr int kD64Threads = 256;                         // 4 waves x 64 rows = kD64BM

template <bool PAGED>
__global__ __launch_bounds__(kD64Threads, 2) void attn_fwd_d64_kernel(DenseParams p) {
  constexpr int D = 64, BN = 64, CPR = D / 8;
  constexpr int TILE = BN * D * 2;                       // 8 KB: one K (or V) tile
  constexpr int LOADS = TILE / (kD64Threads * 16);       // 16-byte DMA loads per lane per tile
  static_assert(LOADS == 2 && kD64Threads / 64 * 64 == kD64BM, "tile split");
  using C = Cfg<D>;                                      // swizzle of the 16-byte chunks
  __shared__ __attribute__((aligned(1024))) unsigned char kst0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char kst1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vst0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vst1[TILE];

  const int slot = wg_slot(blockIdx.x, p.grid, p.wg_perm);
  int id = slot, chunk = 0;
  const bool split = id >= p.full_units;
  if (split) {
    const int u2 = id - p.full_units;
    const int tu = u2 / p.nsplit;
    chunk = u2 - tu * p.nsplit;
    id = p.full_units + tu;
  }
  int b, h, t;
  decode_unit(p, id, b, h, t);
  TileRange tr;
  if (!tile_range(p, b, t, kD64BM, false, tr)) return;     // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  const int kvh = h / p.group;
  const int rw0 = tr.row0 + wave * 64;                   // first row of this wave
  // A wave whose 64 rows all lie past the tile's end (the short last tile of
  // a piece) issues its DMA share and meets every barrier, nothing else.
  const bool live = rw0 < tr.row_end;

  // ---- Q fragments of the two blocks: Q[row][16 ks + 8 g2 .. +7]
  u32x4 qf[2][D / 16];
  bool qvalid[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int qi = rw0 + 32 * r + l32;
    qvalid[r] = qi < tr.row_end;
    const uint16_t* src = (const uint16_t*)p.q + (int64_t)(tr.qs + (qvalid[r] ? qi : tr.row0)) * p.q_stride +
                          (int64_t)h * D + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 v = *(const u32x4*)(src + 16 * ks);
      qf[r][ks] = qvalid[r] ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  float c = fabsf(p.scale) * kLog2e;
  if (p.scale < 0.f) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[r][ks] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  c = fmaxf(c, FLT_MIN);

  const int n_all = (tr.kend + BN - 1) / BN;
  int kt0 = 0, n_tiles = n_all;
  if (split) {
    kt0 = (n_all * chunk) / p.nsplit;
    n_tiles = (n_all * (chunk + 1)) / p.nsplit - kt0;
  }
  const int n_full = tr.kend / BN - kt0;                 // (local) tiles without the key tail

  // ---- DMA of K/V tiles into LDS (see the other kernel)
  const int64_t ksb = p.k_stride * 2, vsb = p.v_stride * 2;
  int voff_k[LOADS], voff_v[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int sl = (wave * LOADS + i) * 64 + lane;
    const int r = sl / CPR, ch = (sl % CPR) ^ C::swz(r);
    voff_k[i] = (int)(r * ksb) + 16 * ch;
    voff_v[i] = (int)(r * vsb) + 16 * ch;
  }
  // Key row j of this sequence: row tr.ks + j of the packed K/V, or for a
  // paged cache row j's page from the sequence's block-table row (a 64-key
  // tile never spans two pages).
  const unsigned char* kbase =
      (const unsigned char*)p.k + ((PAGED ? 0 : (int64_t)tr.ks * p.k_stride) + (int64_t)kvh * D) * 2;
  const unsigned char* vbase =
      (const unsigned char*)p.v + ((PAGED ? 0 : (int64_t)tr.ks * p.v_stride) + (int64_t)kvh * D) * 2;
  auto phys_row = [&](int j) __attribute__((always_inline)) -> int64_t {
    if constexpr (!PAGED) return j;
    const int64_t page = p.block_table[(int64_t)b * p.max_pages + (j >> p.page_shift)];
    return (page << p.page_shift) | (j & ((1 << p.page_shift) - 1));
  };
  auto issue = [&](int kt, const unsigned char* base, int64_t sb, const int* voff, unsigned char* stage) __attribute__((always_inline)) {
    const int j0 = (kt0 + kt) * BN;
    const int rows = min(tr.kend - j0, BN);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + phys_row(j0) * sb), (short)0, (int)(rows * sb), 0x00020000);
    unsigned char* dst = stage + wave * LOADS * 1024;
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                               (unsigned)voff[i], 0, 0, 0);
  };

  // ---- per-lane LDS read offsets (the other kernel's)
  const int sw = C::swz(l32);
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = l32 * D * 2 + 16 * ((2 * ks + g2) ^ sw);
  const int i16 = lane & 15, G16 = lane >> 4, nhalf = G16 & 1;
  const int vr0 = 4 * g2 + (i16 >> 2);
  int voff0[D / 32], voff1[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    const int ch = 4 * nb + 2 * nhalf + ((i16 & 3) >> 1);
    voff0[nb] = vr0 * D * 2 + 16 * (ch ^ C::swz(vr0)) + 8 * (i16 & 1);
    voff1[nb] = (vr0 + 8) * D * 2 + 16 * (ch ^ C::swz(vr0 + 8)) + 8 * (i16 & 1);
  }

  floatx16 o[2][D / 32];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[r][nb] = (floatx16){};
  float m_used[2] = {-INFINITY, -INFINITY};   // reference max (times c, log2 domain)
  float m_use[2] = {0.f, 0.f};                // m_used, or 0 while a row has none
  float l_run[2] = {0.f, 0.f};                // lane-partial sums of P

  auto mask = [&](int kt, floatx16& s0, floatx16& s1) __attribute__((always_inline)) {
    const int j0 = (kt0 + kt) * BN + 4 * g2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + (r & 3);
      if (j >= tr.len_k) s0[r] = -INFINITY;
      if (j + 32 >= tr.len_k) s1[r] = -INFINITY;
    }
  };
  // P = 2^(s c - m), packed bf16 for the P V product; returns the lane's fp32 sum
  auto softmax_p = [&](const floatx16& s0, const floatx16& s1, float mu, u32x4* pb) __attribute__((always_inline)) -> float {
    float tq[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const floatx16& sv = kb == 0 ? s0 : s1;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t w[4];
        float pr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e0 = fast_exp2(fmaf(sv[8 * hf + 2 * q], c, -mu));
          const float e1 = fast_exp2(fmaf(sv[8 * hf + 2 * q + 1], c, -mu));
          pr[q] = e0 + e1;
          w[q] = pack_bf16x2(e0, e1);
        }
        tq[2 * kb + hf] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
        pb[2 * kb + hf] = (u32x4){w[0], w[1], w[2], w[3]};
      }
    }
    return (tq[0] + tq[1]) + (tq[2] + tq[3]);
  };
  // Rare part of block r: the tile's row max moves the reference where it
  // exceeds it by more than 8 (log2 units), with O and l rescaled.
  auto move_ref = [&](int r, const floatx16& s0, const floatx16& s1) __attribute__((always_inline)) {
    float mx = vmax(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = vmax(vmax(mx, s0[i]), s1[i]);
    mx = lane_swap_max(mx);
    const float mx_sc = (mx == -INFINITY) ? -INFINITY : mx * c;
    const bool upd = mx_sc > m_used[r] + 8.0f;
    const float m_new = upd ? mx_sc : m_used[r];
    const float alpha = upd ? fast_exp2(m_used[r] - m_new) : 1.0f;
    m_used[r] = m_new;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[r][nb] *= alpha;
    l_run[r] *= alpha;
    m_use[r] = (m_new == -INFINITY) ? 0.f : m_new;
  };
  // S^T of block r for tile kt from K in global memory: the same operands in
  // the same order as the LDS path (rows past the key bound clamp to the last
  // one; they are masked).
  auto qk_global = [&](int r, int kt, floatx16& s0, floatx16& s1) __attribute__((always_inline)) {
    const int j0 = (kt0 + kt) * BN;
    const unsigned char* pa = kbase + phys_row(min(j0 + l32, tr.kend - 1)) * ksb + 16 * g2;
    const unsigned char* pb2 = kbase + phys_row(min(j0 + 32 + l32, tr.kend - 1)) * ksb + 16 * g2;
    s0 = (floatx16){};
    s1 = (floatx16){};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 a0 = *(const u32x4*)(pa + 32 * ks);
      const u32x4 a1 = *(const u32x4*)(pb2 + 32 * ks);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qf[r][ks]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(qf[r][ks]), s1, 0, 0, 0);
    }
  };
  // Careful key step (the fallback, practically never taken): one block at a
  // time, with the rare-path check before its P V, so a tile whose P would
  // grow past 2^8 moves the reference first.  MASK: the step holds the key
  // tail (only the last step of a range).
  auto step_careful = [&](int kt, const unsigned char* ks_, const unsigned char* vs_, auto mask_tag)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      floatx16 s0 = (floatx16){}, s1 = (floatx16){};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 a0 = *(const u32x4*)(ks_ + koff[ks]);
        const u32x4 a1 = *(const u32x4*)(ks_ + 32 * D * 2 + koff[ks]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qf[r][ks]), s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(qf[r][ks]), s1, 0, 0, 0);
      }
      if constexpr (MASK) mask(kt, s0, s1);
      u32x4 pb[4];
      float t = softmax_p(s0, s1, m_use[r], pb);
      if (__any(t > 8192.f || m_used[r] == -INFINITY)) {
        asm volatile("; rare: recompute the logits, move the reference max, recompute P" ::);
        floatx16 r0, r1;
        qk_global(r, kt, r0, r1);
        if constexpr (MASK) mask(kt, r0, r1);
        move_ref(r, r0, r1);
        t = softmax_p(r0, r1, m_use[r], pb);
      }
      l_run[r] += t;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const u32x2 lo = lds_read_tr(vs_ + st * 16 * D * 2 + voff0[nb]);
          const u32x2 hi = lds_read_tr(vs_ + st * 16 * D * 2 + voff1[nb]);
          const u32x4 vop = (u32x4){lo[0], lo[1], hi[0], hi[1]};
          o[r][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vop), as_bf16x8(pb[st]), o[r][nb], 0, 0, 0);
        }
    }
  };

  bool bad = false;
  // P of one 32-key half (accumulator s) with reference mu: two packed
  // operands (k-steps 2h, 2h + 1) and the lane's fp32 sum.
  auto half_p = [&](const floatx16& sv, u32x4* pb) __attribute__((always_inline)) -> float {
    float tq[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint32_t w[4];
      float pr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float e0 = fast_exp2(sv[8 * hf + 2 * q] * c);
        const float e1 = fast_exp2(sv[8 * hf + 2 * q + 1] * c);
        pr[q] = e0 + e1;
        w[q] = pack_bf16x2(e0, e1);
      }
      tq[hf] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
      pb[hf] = (u32x4){w[0], w[1], w[2], w[3]};
    }
    return tq[0] + tq[1];
  };
  // Fast key step: no branch and no per-row reference: P = 2^(s c) (one
  // multiply before each exponential).  Each tile records (in `bad`, per
  // lane) a lane sum that is not below 2^100, where some P may have
  // overflowed, and the range ends by recording a row sum below 2^-100,
  // where the row's significant P may have left the normal range.  A
  // workgroup with any such lane recomputes its range with the careful step.
  // Without either, every P that matters is a normal fp32 / bf16 number, and
  // these keep their relative precision at any exponent, so the missing
  // reference changes no result; the lse is log(l) with reference 0.
  auto step_fast = [&](int kt, const unsigned char* ks_, const unsigned char* vs_, auto mask_tag)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // Two 32-key halves, rotated so that every block's softmax issues under
    // about eight MFMAs of the other block or of the next half:
    //   S_A0 | S_B0 + sm A0 | P_A0 V, S_A1 + sm B0 | P_B0 V, S_B1 + sm A1 |
    //   P_A1 V + sm B1 | P_B1 V
    auto kread = [&](int hh, u32x4* kop) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) kop[ks] = *(const u32x4*)(ks_ + hh * 32 * D * 2 + koff[ks]);
    };
    auto vread = [&](int hh, u32x4 (*vop)[D / 32]) __attribute__((always_inline)) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const int st = 2 * hh + s2;
          const u32x2 lo = lds_read_tr(vs_ + st * 16 * D * 2 + voff0[nb]);
          const u32x2 hi = lds_read_tr(vs_ + st * 16 * D * 2 + voff1[nb]);
          vop[s2][nb] = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        }
    };
    auto qk = [&](int r, const u32x4* kop) __attribute__((always_inline)) -> floatx16 {
      floatx16 acc = (floatx16){};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop[ks]), as_bf16x8(qf[r][ks]), acc, 0, 0, 0);
      return acc;
    };
    auto pv = [&](int r, u32x4 (*vop)[D / 32], const u32x4* pb) __attribute__((always_inline)) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb)
          o[r][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vop[s2][nb]), as_bf16x8(pb[s2]), o[r][nb], 0,
                                                             0, 0);
    };
    auto mask_half = [&](int hh, floatx16& sa, floatx16& sb) __attribute__((always_inline)) {
      const int j0 = (kt0 + kt) * BN + 32 * hh + 4 * g2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (j0 + 8 * (r >> 2) + (r & 3) >= tr.len_k) {
          sa[r] = -INFINITY;
          sb[r] = -INFINITY;
        }
      }
    };
    u32x4 kop0[D / 16], kop1[D / 16], vop0[2][D / 32], vop1[2][D / 32];
    u32x4 pa0[2], pb0[2], pa1[2], pb1[2];
    kread(0, kop0);
    floatx16 sa0 = qk(0, kop0);
    floatx16 sb0 = qk(1, kop0);
    if constexpr (MASK) mask_half(0, sa0, sb0);
    const float ta0 = half_p(sa0, pa0);
    vread(0, vop0);
    kread(1, kop1);
    pv(0, vop0, pa0);
    floatx16 sa1 = qk(0, kop1);
    const float tb0 = half_p(sb0, pb0);
    pv(1, vop0, pb0);
    floatx16 sb1 = qk(1, kop1);
    if constexpr (MASK) mask_half(1, sa1, sb1);
    const float ta1 = half_p(sa1, pa1);
    vread(1, vop1);
    pv(0, vop1, pa1);
    const float tb1 = half_p(sb1, pb1);
    pv(1, vop1, pb1);
    const float ta = ta0 + ta1, tb = tb0 + tb1;
    bad = bad || !(ta < 0x1p100f) || !(tb < 0x1p100f);   // NaN counts as bad
    l_run[0] += ta;
    l_run[1] += tb;
  };

  // ---- key loop: stage kt % 2 holds K(kt) and V(kt); the DMA of tile kt+1
  // is issued right after the barrier that retires tile kt-1's stage.  Steps
  // before n_full hold no key tail.
  auto iter = [&](int kt, auto odd_tag, auto mask_tag, auto careful_tag) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(odd_tag)::value;
    unsigned char* k_rd = ODD ? kst1 : kst0;
    unsigned char* v_rd = ODD ? vst1 : vst0;
    unsigned char* k_wr = ODD ? kst0 : kst1;
    unsigned char* v_wr = ODD ? vst0 : vst1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // this lane's DMA of tile kt landed
    __syncthreads();                                     // everyone's; tile kt-1's stage is free
    if (kt + 1 < n_tiles) {
      issue(kt + 1, kbase, ksb, voff_k, k_wr);
      issue(kt + 1, vbase, vsb, voff_v, v_wr);
    }
    if (live) {
      if constexpr (decltype(careful_tag)::value) step_careful(kt, k_rd, v_rd, mask_tag);
      else step_fast(kt, k_rd, v_rd, mask_tag);
      if (kt + 1 == n_tiles) {
        // After the range's last MFMAs the compiler may reuse their A/B
        // operand registers right away (register copies where the loop's
        // paths join).  A write that lands before an MFMA still waiting in
        // the matrix pipe has read its operands corrupts that product; the
        // pipe's depth depends on the other wave's MFMAs, so the result
        // would depend on timing.  32 wait states let the pipe drain first.
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  const int n_plain = min(n_tiles, max(n_full, 0));
  auto run = [&](auto careful_tag) __attribute__((always_inline)) {
    using F = std::false_type;
    using T = std::true_type;
    issue(0, kbase, ksb, voff_k, kst0);
    issue(0, vbase, vsb, voff_v, vst0);
    if (n_plain > 0) iter(0, F{}, F{}, careful_tag);
    else iter(0, F{}, T{}, careful_tag);                 // the only step holds the key tail
    int kt = 1;
    for (; kt + 1 < n_plain; kt += 2) {
      iter(kt, T{}, F{}, careful_tag);
      iter(kt + 1, F{}, F{}, careful_tag);
    }
    if (kt < n_plain) {                                  // one more plain step (odd), then the tail (even)
      iter(kt, T{}, F{}, careful_tag);
      if (kt + 1 < n_tiles) iter(kt + 1, F{}, T{}, careful_tag);
    } else if (kt < n_tiles) {                           // the tail step (odd)
      iter(kt, T{}, T{}, careful_tag);
    }
  };
  if (n_tiles > 0) {
    run(std::false_type{});
#pragma unroll
    for (int r = 0; r < 2; ++r) {                        // reference 0 on the fast path
      m_used[r] = 0.f;
      if (live) bad = bad || !(lane_swap_add(l_run[r]) >= 0x1p-100f);   // a wave with no rows has no sums
    }
    // the decision is the workgroup's: the careful pass stages tiles with
    // barriers that every wave must meet
    if (__syncthreads_or(bad ? 1 : 0)) {
      asm volatile("; rare: recompute the range with per-step reference moves" ::);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) o[r][nb] = (floatx16){};
        m_used[r] = -INFINITY;
        m_use[r] = 0.f;
        l_run[r] = 0.f;
      }
      run(std::true_type{});
    }
  }

  // ---- epilogue
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float l_tot = lane_swap_add(l_run[r]);
    const int rl = wave * 64 + 32 * r + l32;             // row within the tile
    if (split) {
      float* w = p.ws + (size_t)(slot - p.full_units) * (kD64BM * (D + 2));
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(floatx4*)(w + rl * D + 32 * nb + 8 * r4 + 4 * g2) =
              (floatx4){o[r][nb][4 * r4], o[r][nb][4 * r4 + 1], o[r][nb][4 * r4 + 2], o[r][nb][4 * r4 + 3]};
      if (g2 == 0) {
        w[kD64BM * D + rl] = m_used[r];
        w[kD64BM * D + kD64BM + rl] = l_tot;
      }
      continue;
    }
    if (!qvalid[r]) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int qi = rw0 + 32 * r + l32;
    uint16_t* dst = (uint16_t*)p.out + (int64_t)(tr.qs + qi) * p.o_stride + (int64_t)h * D + 4 * g2;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const floatx16& ov = o[r][nb];
        const u32x2 w = (u32x2){pack_bf16x2(ov[4 * r4 + 0] * inv, ov[4 * r4 + 1] * inv),
                                pack_bf16x2(ov[4 * r4 + 2] * inv, ov[4 * r4 + 3] * inv)};
        *(u32x2*)(dst + 32 * nb + 8 * r4) = w;
      }
    if (p.lse != nullptr && g2 == 0)
      p.lse[(int64_t)h * p.total_q + tr.qs + qi] = l_tot > 0.f ? (m_used[r] + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// =============================================================== fp8 path
// Attention on OCP FP8 E4M3 inputs (v_mfma_scale_f32_32x32x64_f8f6f4, unit
// scales).  FP8 is allowed for the matrix products, the softmax statistics
// and accumulation stay fp32 (「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈
// 性能」 section 4.1); q carries one dequantisation scale per (token, head),
// k one per head and v one per (head, channel) (the block scales of that
// page's section 5.3).  The q and k scales fold into the per-lane exponent
// factor c, the v scales into the epilogue, so the key loop is the bf16
// kernel's with one MFMA per 64 channels of Q K^T and one per 64 keys of P V.
// P is rounded to E4M3 for the P V product; its fp32 values form l.  The
// max-free softmax of the bf16 kernel is kept, with the rare path taken when
// a lane's tile sum exceeds 448 (the largest E4M3 value; above it the
// conversion gives NaN), which bounds every P below 448.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct CfgF8 {
  static constexpr int BM = kDenseBM;                   // 4 waves x 32 query rows
  static constexpr int BN = 64;                         // keys per step
  static constexpr int THREADS = 256;
  static constexpr int CPR = D / 16;                    // 16-byte chunks per K/V row
  static constexpr int TILE = BN * D;                   // bytes of one K (or V) tile
  static constexpr int LOADS = TILE / (THREADS * 16);   // 16-byte DMA loads per lane per tile
  static_assert(LOADS == 1 || LOADS == 2, "tile split");
  // XOR swizzles of the 16-byte chunks of a row (64 four-byte banks: 16
  // chunk slots per 256 bytes).
  //  * K reads (ds_read_b128): 16 lanes read one logical chunk of 16
  //    consecutive rows; rows fill 4 (d 64) or 2 (d 128) chunk slots each.
  //  * V^T reads (ds_read_b64_tr_b8): 32 lanes read two adjacent logical
  //    chunks of 8 rows {r, r + 1, r + 2, r + 3, r + 8, .., r + 11} (r a
  //    multiple of 4); rows r and r + 8 (and for d 128 rows r and r + 2)
  //    otherwise fall on the same slots.
  static __device__ __forceinline__ int swk(int r) { return D == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swv(int r) {
    return D == 64 ? (((r >> 3) & 1) << 1) : ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2));
  }
};

// ds_read_b64_tr_b8: each lane of a 16-lane group reads 8 bytes (row i/2,
// bytes 8(i%2)..+7 of an 8 x 16 byte block, one row address per lane pair)
// and receives column i of the block (its 8 rows, in row order).
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
  i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ floatx16 mfma_f8(const i32x8& a, const i32x8& b, const floatx16& c) {
  // formats 0/0: E4M3 x E4M3; scale bytes 127: 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <bool HI>
__device__ __forceinline__ uint32_t cvt_f8x2(float a, float b, uint32_t w) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, HI);
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, (D == 64 ? 3 : 2)) void attn_fwd_fp8_kernel(DenseParams p) {
  using C = CfgF8<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char kst0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char kst1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vst0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vst1[C::TILE];

  int b, h, t;
  decode_unit(p, wg_slot(blockIdx.x, p.grid, p.wg_perm), b, h, t);
  TileRange tr;
  if (!tile_range(p, b, t, C::BM, CAUSAL, tr)) return;   // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  const int kvh = h / p.group;
  const int qi = tr.row0 + wave * 32 + l32;
  const bool qvalid = qi < tr.row_end;
  const int64_t qrow = tr.qs + (qvalid ? qi : tr.row0);

  // ---- Q fragment (B operand of S^T = K Q^T): Q[qi][64 ks + 32 g2 .. + 31].
  // A negative scale flips the sign bits (exact).
  i32x8 qf[D / 64];
  {
    const unsigned char* src = (const unsigned char*)p.q + qrow * p.q_stride + (int64_t)h * D + 32 * g2;
    const uint32_t flip = p.scale < 0.f ? 0x80808080u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      u32x4 lo = *(const u32x4*)(src + 64 * ks);
      u32x4 hi = *(const u32x4*)(src + 64 * ks + 16);
      lo ^= flip;
      hi ^= flip;
      if (!qvalid) lo = hi = (u32x4){0u, 0u, 0u, 0u};
      qf[ks] = cat8(lo, hi);
    }
  }
  float c = fabsf(p.scale) * kLog2e * p.q_scale[qrow * p.hq + h] * p.k_scale[kvh];
  c = fmaxf(c, FLT_MIN);   // a zero factor: every logit becomes ~0, masked ones stay -inf

  const int kend_i = CAUSAL ? clampi(qi + tr.len_k - tr.len_q + 1, 0, tr.len_k) : tr.len_k;
  const int n_tiles = (tr.kend + C::BN - 1) / C::BN;

  // ---- DMA of K/V tiles straight into LDS.  Lane slot sl of the wave's 1 KB
  // destination block holds row sl / CPR, physical chunk sl % CPR = logical
  // chunk ^ swizzle(row).  Rows past the key range read as zeros.
  const int64_t ksb = p.k_stride, vsb = p.v_stride;     // bytes per token
  int voff_k[C::LOADS], voff_v[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int sl = (wave * C::LOADS + i) * 64 + lane;
    const int r = sl / C::CPR, ph = sl % C::CPR;
    voff_k[i] = (int)(r * ksb) + 16 * (ph ^ C::swk(r));
    voff_v[i] = (int)(r * vsb) + 16 * (ph ^ C::swv(r));
  }
  const unsigned char* kbase = (const unsigned char*)p.k + (int64_t)tr.ks * ksb + (int64_t)kvh * D;
  const unsigned char* vbase = (const unsigned char*)p.v + (int64_t)tr.ks * vsb + (int64_t)kvh * D;
  auto issue_tile = [&](int kt, const unsigned char* base, int64_t sb, const int* voff, unsigned char* stage) {
    const int rows = min(tr.kend - kt * C::BN, C::BN);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (int64_t)kt * C::BN * sb), (short)0, (int)(rows * sb), 0x00020000);
    unsigned char* dst = stage + wave * C::LOADS * 1024;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                               (unsigned)voff[i], 0, 0, 0);
  };
  auto issue_k = [&](int kt, unsigned char* stage) { issue_tile(kt, kbase, ksb, voff_k, stage); };
  auto issue_v = [&](int kt, unsigned char* stage) { issue_tile(kt, vbase, vsb, voff_v, stage); };

  // ---- per-lane LDS read offsets (loop invariant)
  // K rows l32 (+ 32), logical chunks 4 ks + 2 g2 and + 1 (channels 64 ks +
  // 32 g2 .. + 31, as in the Q fragment).  Rows l32 and l32 + 32 share a swizzle.
  int koff[D / 64][2];
#pragma unroll
  for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[ks][u] = l32 * D + 16 * ((4 * ks + 2 * g2 + u) ^ C::swk(l32));
  // V^T operand of channel block nb: k-slot s of lane half g2 is key
  // kslot(s) = 8 (s / 4) + 4 g2 + s % 4 for s < 16 and 32 + that of s - 16
  // above, the order in which the lane holds P (its S registers of key
  // blocks 0 and 1).  Read m returns slots 8m .. 8m + 7: lane pair (2q,
  // 2q + 1) of a 16-lane group addresses the row of slot 8m + q, both halves
  // of the group's 16-channel chunk (2 nb + nhalf).
  const int i16 = lane & 15, nhalf = (lane >> 4) & 1;
  int voffr[4][D / 32];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int sl = 8 * m + (i16 >> 1);
    const int key = sl < 16 ? 8 * (sl >> 2) + 4 * g2 + (sl & 3) : 32 + 8 * ((sl - 16) >> 2) + 4 * g2 + (sl & 3);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
      voffr[m][nb] = key * D + 16 * ((2 * nb + nhalf) ^ C::swv(key)) + 8 * (i16 & 1);
  }

  floatx16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = (floatx16){};
  float m_used = -INFINITY;  // max used for exponentiation (times c, log2 domain)
  float l_run = 0.f;         // lane-partial sum of P
  float m_use = 0.f;         // m_used, or 0 while the row has none
  const int n_full = min(n_tiles, tr.kfull / C::BN);   // tiles no row needs masked

  auto qk = [&](const unsigned char* ks_, floatx16& s0, floatx16& s1) {
    s0 = (floatx16){};
    s1 = (floatx16){};
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const i32x8 a0 = cat8(*(const u32x4*)(ks_ + koff[ks][0]), *(const u32x4*)(ks_ + koff[ks][1]));
      const i32x8 a1 = cat8(*(const u32x4*)(ks_ + 32 * D + koff[ks][0]), *(const u32x4*)(ks_ + 32 * D + koff[ks][1]));
      s0 = mfma_f8(a0, qf[ks], s0);
      s1 = mfma_f8(a1, qf[ks], s1);
    }
  };
  auto mask = [&](int kt, floatx16& s0, floatx16& s1) {
    const int j0 = kt * C::BN + 4 * g2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + (r & 3);
      if (j >= kend_i) s0[r] = -INFINITY;
      if (j + 32 >= kend_i) s1[r] = -INFINITY;
    }
  };
  // Reference max (moved lazily, as in the bf16 kernel: only when a tile max
  // exceeds it by more than 8 in log2 units, so P stays below 2^8).
  auto softmax_ref = [&](const floatx16& s0, const floatx16& s1) -> float {
    float mx = vmax(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = vmax(vmax(mx, s0[r]), s1[r]);
    mx = lane_swap_max(mx);
    const float mx_sc = (mx == -INFINITY) ? -INFINITY : mx * c;
    const bool upd = mx_sc > m_used + 8.0f;
    if (__any(upd)) {
      asm volatile("; rare: move the reference max, rescale O and l" ::);
      const float m_new = upd ? mx_sc : m_used;
      const float alpha = upd ? fast_exp2(m_used - m_new) : 1.0f;
      m_used = m_new;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
      l_run *= alpha;
    }
    return (m_used == -INFINITY) ? 0.f : m_used;
  };
  // P = 2^(s c - m) with the current reference, rounded to E4M3 in k-slot
  // order (byte s of the operand = slot s), and the lane's fp32 sum of P.
  auto softmax_p = [&](const floatx16& s0, const floatx16& s1, float mu, i32x8& pb) -> float {
    float tq[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const floatx16& sv = w < 4 ? s0 : s1;
      const int r = 4 * (w & 3);
      const float e0 = fast_exp2(fmaf(sv[r], c, -mu));
      const float e1 = fast_exp2(fmaf(sv[r + 1], c, -mu));
      const float e2 = fast_exp2(fmaf(sv[r + 2], c, -mu));
      const float e3 = fast_exp2(fmaf(sv[r + 3], c, -mu));
      tq[w] = (e0 + e1) + (e2 + e3);
      pb[w] = (int)cvt_f8x2<true>(e2, e3, cvt_f8x2<false>(e0, e1, 0u));
    }
    return ((tq[0] + tq[1]) + (tq[2] + tq[3])) + ((tq[4] + tq[5]) + (tq[6] + tq[7]));
  };
  // S^T of key tile kt from K in global memory (rows past the key bound
  // clamped to the last one; they are masked): bitwise the LDS path's logits.
  auto qk_global = [&](int kt, floatx16& s0, floatx16& s1) {
    const int r0 = kt * C::BN;
    const unsigned char* pa = kbase + (int64_t)min(r0 + l32, tr.kend - 1) * ksb + 32 * g2;
    const unsigned char* pb2 = kbase + (int64_t)min(r0 + 32 + l32, tr.kend - 1) * ksb + 32 * g2;
    s0 = (floatx16){};
    s1 = (floatx16){};
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const i32x8 a0 = cat8(*(const u32x4*)(pa + 64 * ks), *(const u32x4*)(pa + 64 * ks + 16));
      const i32x8 a1 = cat8(*(const u32x4*)(pb2 + 64 * ks), *(const u32x4*)(pb2 + 64 * ks + 16));
      s0 = mfma_f8(a0, qf[ks], s0);
      s1 = mfma_f8(a1, qf[ks], s1);
    }
  };
  // O^T += V^T P^T over the tile's 64 keys, one MFMA per 32 channels.
  auto pv = [&](const i32x8& pb, const unsigned char* vs_) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      const u32x2 r0 = lds_read_tr8(vs_ + voffr[0][nb]);
      const u32x2 r1 = lds_read_tr8(vs_ + voffr[1][nb]);
      const u32x2 r2 = lds_read_tr8(vs_ + voffr[2][nb]);
      const u32x2 r3 = lds_read_tr8(vs_ + voffr[3][nb]);
      const i32x8 a = (i32x8){(int)r0[0], (int)r0[1], (int)r1[0], (int)r1[1],
                              (int)r2[0], (int)r2[1], (int)r3[0], (int)r3[1]};
      o[nb] = mfma_f8(a, pb, o[nb]);
    }
  };

  // ---- software pipeline over key tiles, as in the bf16 kernel: iteration
  // kt computes S of tile kt and finishes tile kt - 1; K is staged one tile
  // ahead of V; stage parity is static per iteration.
  floatx16 sp0, sp1;
  auto iter = [&](int kt, auto odd_tag, auto has_s_tag) {
    constexpr bool ODD = decltype(odd_tag)::value;
    constexpr bool HAS_S = decltype(has_s_tag)::value;
    unsigned char* k_rd = ODD ? kst1 : kst0;
    unsigned char* k_wr = ODD ? kst0 : kst1;
    unsigned char* v_rd = ODD ? vst0 : vst1;
    unsigned char* v_wr = ODD ? vst1 : vst0;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    floatx16 sn0, sn1;
    if constexpr (HAS_S) {
      if (kt + 1 < n_tiles) issue_k(kt + 1, k_wr);
      issue_v(kt, v_wr);
      qk(k_rd, sn0, sn1);
    }
    i32x8 pb;
    float tsum = softmax_p(sp0, sp1, m_use, pb);
    if (__any(tsum > 448.f || m_used == -INFINITY)) {
      asm volatile("; rare: recompute the logits, move the reference max, recompute P" ::);
      floatx16 r0, r1;
      qk_global(kt - 1, r0, r1);
      if (kt - 1 >= n_full) mask(kt - 1, r0, r1);
      m_use = softmax_ref(r0, r1);
      tsum = softmax_p(r0, r1, m_use, pb);
    }
    l_run += tsum;
    pv(pb, v_rd);
    if constexpr (HAS_S) {
      if (kt >= n_full) mask(kt, sn0, sn1);
      sp0 = sn0;
      sp1 = sn1;
    }
  };

  if (n_tiles > 0) {
    issue_k(0, kst0);
    issue_v(0, vst0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (1 < n_tiles) issue_k(1, kst1);
    qk(kst0, sp0, sp1);
    if (0 >= n_full) mask(0, sp0, sp1);
    m_use = softmax_ref(sp0, sp1);
    int kt = 1;
    for (; kt + 1 < n_tiles; kt += 2) {
      iter(kt, std::true_type{}, std::true_type{});
      iter(kt + 1, std::false_type{}, std::true_type{});
    }
    if (kt < n_tiles) {
      iter(kt, std::true_type{}, std::true_type{});
      iter(kt + 1, std::false_type{}, std::false_type{});
    } else {
      iter(kt, std::true_type{}, std::false_type{});
    }
  }

  // ---- epilogue: out = O v_scale / l (bf16 RNE), lse = ln 2 (m + log2 l)
  const float l_tot = lane_swap_add(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    uint16_t* dst = (uint16_t*)p.out + (int64_t)(tr.qs + qi) * p.o_stride + (int64_t)h * D + 4 * g2;
    const float* vsc = p.v_scale + (int64_t)kvh * D + 4 * g2;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const floatx4 sv = *(const floatx4*)(vsc + 32 * nb + 8 * r4);
        const floatx16& ov = o[nb];
        const u32x2 w = (u32x2){pack_bf16x2(ov[4 * r4 + 0] * sv[0] * inv, ov[4 * r4 + 1] * sv[1] * inv),
                                pack_bf16x2(ov[4 * r4 + 2] * sv[2] * inv, ov[4 * r4 + 3] * sv[3] * inv)};
        *(u32x2*)(dst + 32 * nb + 8 * r4) = w;
      }
    if (p.lse != nullptr && g2 == 0)
      p.lse[(int64_t)h * p.total_q + tr.qs + qi] = l_tot > 0.f ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge of the split chunks of one unit, in chunk order (fixed, so the result
// is deterministic): with M = max_i m_i, O = sum_i 2^(m_i - M) O_i and
// l = sum_i 2^(m_i - M) l_i, out = O / l (bf16) and lse = ln 2 (M + log2 l):
// the blockwise merge of [V32] eq. (1)(2) with the O update written out.
// Workgroup (tail unit, group of 256 (row, 16-column slice) items).  Empty
// chunks carry m = -inf, l = 0.
template <int D, int NS>
__global__ __launch_bounds__(256) void attn_merge_kernel(DenseParams p) {
  const int tu = blockIdx.x;
  int b, h, t;
  decode_unit(p, p.full_units + tu, b, h, t);
  TileRange tr;
  if (p.dec_group > 0) decode_range(p, b, tr);
  else if (!tile_range(p, b, t, p.bm, false, tr)) return;
  constexpr int SL = D / 16;                            // 16-column slices per row
  const int item = blockIdx.y * 256 + threadIdx.x;
  const int rl = item / SL, sc = item - rl * SL;        // row within the tile, slice
  const int qi = tr.row0 + rl;
  const int wr = p.ws_rows;                             // rows per chunk
  if (rl >= wr || qi >= tr.row_end) return;
  const size_t CF = (size_t)wr * (D + 2);               // floats per chunk
  const float* base = p.ws + (size_t)tu * NS * CF;
  // every chunk's m, l and 16 values loaded up front (one memory latency)
  float mi[NS], li[NS];
  floatx4 vi[NS][4];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const float* c = base + i * CF;
    mi[i] = c[wr * D + rl];
    li[i] = c[wr * D + wr + rl];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) vi[i][q4] = ((const floatx4*)(c + rl * D + 16 * sc))[q4];
  }
  float mmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i) mmax = fmaxf(mmax, mi[i]);
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  float l = 0.f;
  if (mmax != -INFINITY) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (mi[i] == -INFINITY) continue;                 // empty chunk
      const float f = fast_exp2(mi[i] - mmax);
      l = fmaf(f, li[i], l);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * q4 + j] = fmaf(f, vi[i][q4][j], acc[4 * q4 + j]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  u32x4 w[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j >> 2][j & 3] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  const bool dec = p.dec_group > 0;
  uint16_t* dst = dec ? (uint16_t*)p.out + (int64_t)b * p.o_stride + (int64_t)(h * p.dec_group + qi) * D + 16 * sc
                      : (uint16_t*)p.out + (int64_t)(tr.qs + qi) * p.o_stride + (int64_t)h * D + 16 * sc;
  *(u32x4*)dst = w[0];
  *(u32x4*)(dst + 8) = w[1];
  const int64_t lsi = dec ? (int64_t)(h * p.dec_group + qi) * p.total_q + b : (int64_t)h * p.total_q + tr.qs + qi;
  if (sc == 0 && p.lse != nullptr) p.lse[lsi] = l > 0.f ? (mmax + log2f(l)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_merge(const DenseParams& p, dim3 grid, hipStream_t s) {
  switch (p.nsplit) {
    case 2: hipLaunchKernelGGL((attn_merge_kernel<D, 2>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((attn_merge_kernel<D, 3>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((attn_merge_kernel<D, 4>), grid, dim3(256), 0, s, p); break;
    case 5: hipLaunchKernelGGL((attn_merge_kernel<D, 5>), grid, dim3(256), 0, s, p); break;
    case 6: hipLaunchKernelGGL((attn_merge_kernel<D, 6>), grid, dim3(256), 0, s, p); break;
    case 7: hipLaunchKernelGGL((attn_merge_kernel<D, 7>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((attn_merge_kernel<D, 8>), grid, dim3(256), 0, s, p); break;
    case 9: hipLaunchKernelGGL((attn_merge_kernel<D, 9>), grid, dim3(256), 0, s, p); break;
    case 10: hipLaunchKernelGGL((attn_merge_kernel<D, 10>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

// ================================================================ fp32 path
// Same decomposition with v_mfma_f32_32x32x2_f32: each lane holds one k value
// per MFMA, so K and V are read row-major from LDS (no transpose needed).

template <int D>
struct CfgF32 {
  static constexpr int BM = kDenseBM;
  static constexpr int BN = 32;
  static constexpr int THREADS = 256;
  static constexpr int ROW = D + 4;           // floats per LDS row
  static constexpr int DCH = D / 4;           // 16-byte chunks per row
  static constexpr int CPT = BN * DCH / THREADS;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void attn_fwd_f32_kernel(DenseParams p) {
  using C = CfgF32<D>;
  __shared__ __attribute__((aligned(16))) float ksm[C::BN * C::ROW];
  __shared__ __attribute__((aligned(16))) float vsm[C::BN * C::ROW];

  int b, h, t;
  decode_unit(p, wg_slot(blockIdx.x, p.grid, p.wg_perm), b, h, t);
  TileRange tr;
  if (!tile_range(p, b, t, C::BM, CAUSAL, tr)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  const int kvh = h / p.group;
  const float* __restrict__ qg = (const float*)p.q;
  const float* __restrict__ kg = (const float*)p.k;
  const float* __restrict__ vg = (const float*)p.v;

  const int qi = tr.row0 + wave * 32 + l32;
  const bool qvalid = qi < tr.row_end;
  // B operand of the 32x32x2 MFMA: lane holds Q[qi][2 ks + g2]
  float qf[D / 2];
  {
    const float* src = qg + (int64_t)(tr.qs + (qvalid ? qi : tr.row0)) * p.q_stride + (int64_t)h * D + g2;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = qvalid ? src[2 * ks] : 0.f;
  }
  float c = fabsf(p.scale) * kLog2e;
  if (p.scale < 0.f) {
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = -qf[ks];
  }
  c = fmaxf(c, FLT_MIN);
  const int kend_i = CAUSAL ? clampi(qi + tr.len_k - tr.len_q + 1, 0, tr.len_k) : tr.len_k;

  floatx16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = (floatx16){};
  float m_run = -INFINITY, l_run = 0.f;
  const int n_tiles = (tr.kend + C::BN - 1) / C::BN;

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int kbase = kt * C::BN;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int cidx = tid + i * C::THREADS;
      const int r = cidx / C::DCH, dc = cidx % C::DCH;
      const int key = kbase + r;
      const bool ok = key < tr.kend;
      const int64_t row = tr.ks + (ok ? key : 0);
      floatx4 kv = *(const floatx4*)(kg + row * p.k_stride + (int64_t)kvh * D + 4 * dc);
      floatx4 vv = *(const floatx4*)(vg + row * p.v_stride + (int64_t)kvh * D + 4 * dc);
      if (!ok) { kv = (floatx4){}; vv = (floatx4){}; }
      *(floatx4*)(ksm + r * C::ROW + 4 * dc) = kv;
      *(floatx4*)(vsm + r * C::ROW + 4 * dc) = vv;
    }
    __syncthreads();

    floatx16 s = (floatx16){};
    {
      const float* ka = ksm + l32 * C::ROW + g2;
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[2 * ks], qf[ks], s, 0, 0, 0);
    }
    if (kbase + C::BN > tr.kfull) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kbase + 8 * (r >> 2) + 4 * g2 + (r & 3);
        if (j >= kend_i) s[r] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mx_sc = (mx == -INFINITY) ? -INFINITY : mx * c;
    const float m_new = fmaxf(m_run, mx_sc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(s[r], c, -m_use));
      s[r] = e;
      psum += e;
    }
    l_run = fmaf(alpha, l_run, psum);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
    // O^T += V^T P^T: MFMA step r uses key 8 (r/4) + 4 g2 + r%4 in lane half g2.
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g2 + (r & 3);
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vsm[key * C::ROW + 32 * nb + l32], s[r], o[nb], 0, 0, 0);
      }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    float* dst = (float*)p.out + (int64_t)(tr.qs + qi) * p.o_stride + (int64_t)h * D + 4 * g2;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const floatx16& ov = o[nb];
        *(floatx4*)(dst + 32 * nb + 8 * r4) =
            (floatx4){ov[4 * r4] * inv, ov[4 * r4 + 1] * inv, ov[4 * r4 + 2] * inv, ov[4 * r4 + 3] * inv};
      }
    if (p.lse != nullptr && g2 == 0)
      p.lse[(int64_t)h * p.total_q + tr.qs + qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ======================================================= debug probabilities
// P[r][j] = exp(scale q.k - lse) for one piece of one head, written from the
// start of the caller's buffer (piece-local addressing, [3090] section 三).
template <bool BF16>
__global__ __launch_bounds__(256) void attn_probs_kernel(ProbsParams p) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= p.rows || j >= p.len_k) return;
  const int i = p.q0 + r;                                   // local query row
  float* dst = p.p + (int64_t)r * p.p_stride + j;
  if (p.causal && j > i + p.len_k - p.len_q) { *dst = 0.f; return; }
  float dot = 0.f;
  if (BF16) {
    const uint16_t* qq = (const uint16_t*)p.q + (int64_t)(p.seq_q + i) * p.q_stride + (int64_t)p.head * p.d;
    const uint16_t* kk = (const uint16_t*)p.k + (int64_t)(p.seq_k + j) * p.k_stride + (int64_t)p.kv_head * p.d;
    for (int c = 0; c < p.d; ++c)
      dot = fmaf(__uint_as_float((uint32_t)qq[c] << 16), __uint_as_float((uint32_t)kk[c] << 16), dot);
  } else {
    const float* qq = (const float*)p.q + (int64_t)(p.seq_q + i) * p.q_stride + (int64_t)p.head * p.d;
    const float* kk = (const float*)p.k + (int64_t)(p.seq_k + j) * p.k_stride + (int64_t)p.kv_head * p.d;
    for (int c = 0; c < p.d; ++c) dot = fmaf(qq[c], kk[c], dot);
  }
  const float l = p.lse[(int64_t)p.head * p.lse_stride + p.seq_q + i];
  *dst = expf(p.scale * dot - l);
}

// Scratch of vea_attn_fwd_noalloc: the split chunks of the last round of
// workgroups (at most one chunk per resident workgroup).  Host code never
// passes the array's name to a kernel: its device address on the current
// device comes from attn_noalloc_scratch below.
__device__ __align__(256) unsigned char scratch[VEA_ATTN_NOALLOC_SCRATCH_BYTES];

}  // namespace

hipError_t attn_noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<void*> addr;                       // per device, resolved once
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= addr.size()) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

DenseSplit dense_split_plan(int units, int empty, int slots, int key_tiles) {
  // Units go out in grid order, `slots` at a time; the first `empty` have no
  // rows and end at once.  The last round holds (units - empty) % slots real
  // units and would leave most slots idle for a whole unit's time, so each of
  // them is split into as many key ranges as the idle slots allow (at most
  // 10, at most one per key tile; a split below 2 is not worth the merge).
  DenseSplit s{units, 1, 0};
  const int real = units - empty;
  if (slots <= 0 || real <= slots) return s;
  const int tail = real % slots;
  if (tail == 0) return s;
  const int nsplit = std::min(std::min(10, slots / tail), key_tiles);
  if (nsplit < 2) return s;
  s.full_units = units - tail;
  s.nsplit = nsplit;
  s.chunks = tail * nsplit;
  return s;
}

size_t dense_chunk_bytes(int bm, int head_dim) { return (size_t)bm * (head_dim + 2) * sizeof(float); }

int dense_bf16_blocks_per_cu(int head_dim) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  if (head_dim == 64)   // the packed image kernel (the one the split plan serves)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_d64_kernel<false>, kD64Threads, 0);
  else if (head_dim == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_bf16_kernel<128, false, false>, 256, 0);
  return e == hipSuccess ? n : 0;
}

template <int D>
void launch_dense(const DenseParams& p, bool causal, bool paged, dim3 grid, dim3 block, hipStream_t s) {
  // p.bm was chosen by dense_tile_rows for the same (dtype, head_dim, causal)
  if (p.dec_group > 0) {                                // decode units (never causal)
    if (paged) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, false, true>), grid, block, 0, s, p);
    return;
  }
  if (!causal && D == 64) {                             // one kernel for both layouts: paged = packed bitwise
    if (paged) hipLaunchKernelGGL(attn_fwd_d64_kernel<true>, grid, dim3(kD64Threads), 0, s, p);
    else hipLaunchKernelGGL(attn_fwd_d64_kernel<false>, grid, dim3(kD64Threads), 0, s, p);
  } else if (paged) {
    if (causal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, true>), grid, block, 0, s, p);
  } else if (causal) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, false>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, false>), grid, block, 0, s, p);
  }
}

hipError_t launch_attn_fwd_fp8(const DenseParams& p0, int head_dim, bool causal, hipStream_t s) {
  if (p0.nsplit != 1 || p0.full_units != p0.units || p0.block_table != nullptr || p0.bm != kDenseBM)
    return hipErrorInvalidValue;
  const dim3 grid(p0.units), block(256);
  DenseParams p = p0;
  p.grid = p0.units;
  p.wg_perm = wg_order_perm(p.grid);
  if (head_dim == 64) {
    if (causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, false>), grid, block, 0, s, p);
  } else if (head_dim == 128) {
    if (causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false>), grid, block, 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_bf16(const DenseParams& p0, int head_dim, bool causal, hipStream_t s) {
  const int want_bm = p0.dec_group > 0 ? kDenseBM : dense_tile_rows(1, head_dim, causal);
  if (p0.bm != want_bm) return hipErrorInvalidValue;
  const bool split = p0.nsplit > 1;
  if (split ? (causal || p0.ws == nullptr || p0.full_units < 0 || p0.full_units >= p0.units)
            : p0.full_units != p0.units)
    return hipErrorInvalidValue;
  const dim3 grid(p0.full_units + (p0.units - p0.full_units) * p0.nsplit), block(256);
  DenseParams p = p0;
  p.grid = (int)grid.x;
  p.wg_perm = wg_order_perm(p.grid);
  const bool paged = p.block_table != nullptr;
  if (head_dim == 64) {
    launch_dense<64>(p, causal, paged, grid, block, s);
  } else if (head_dim == 128) {
    launch_dense<128>(p, causal, paged, grid, block, s);
  } else {
    return hipErrorInvalidValue;
  }
  if (split) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid(p.units - p.full_units, p.bm * head_dim / 16 / 256);
    const hipError_t me = head_dim == 64 ? launch_merge<64>(p, mgrid, s) : launch_merge<128>(p, mgrid, s);
    if (me != hipSuccess) return me;
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const DenseParams& p0, int head_dim, bool causal, hipStream_t s) {
  if (p0.bm != kDenseBM) return hipErrorInvalidValue;
  const dim3 grid(p0.units), block(256);
  DenseParams p = p0;
  p.grid = p0.units;
  p.wg_perm = wg_order_perm(p.grid);
  if (head_dim != 64) return hipErrorInvalidValue;
  if (causal) hipLaunchKernelGGL((attn_fwd_f32_kernel<64, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_fwd_f32_kernel<64, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_probs(const ProbsParams& p, bool bf16, hipStream_t s) {
  const dim3 grid((p.len_k + 255) / 256, p.rows), block(256);
  if (bf16) hipLaunchKernelGGL((attn_probs_kernel<true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_probs_kernel<false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace vea
