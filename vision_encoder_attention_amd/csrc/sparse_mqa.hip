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
// Per query row r the work is a small dense attention whose "query rows" are
// the heads: S = Q_r K_r^T over d_qk (heads x k), softmax per head, O = P V_r
// over d_v, with K_r the gathered latent rows and V_r their first d_v columns.
//
// One workgroup = 4 waves = 128 heads of one query row, so each latent row is
// gathered once per query row.  Each wave owns 32 heads over the full d_qk and
// d_v, with v_mfma_f32_32x32x16_bf16 tiles whose N dimension is the 32 heads:
// every 16-byte K or V operand read from LDS feeds 32 heads (32 flops per LDS
// byte; a 16-head tile would make the kernel LDS-bound).  Q^T (36 k-steps) sits
// in VGPRs and O^T (16 tiles of 32 d_v x 32 heads) in accumulation registers:
// one wave per SIMD.  Per step of BN = 32 sorted indices:
//   gather   32 latent rows straight into LDS by buffer loads with the LDS bit
//            (per-lane row addresses; entries past the valid count read as
//            zeros through the buffer's record bound), into a ring of stages
//            filled ahead of use, 16-byte chunks XOR-swizzled within each row;
//   S^T      = K Q^T, fp32 accumulation;
//   softmax  fp32 online update with a lazily moved reference max; the
//            softmax of tile t runs on the VALU under the P V MFMAs of tile
//            t-1, so each step is QK^T of tile t, then P V of tile t-1;
//   O^T     += V^T P^T; the V^T operands come straight from the row-major tile
//            with ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x
//            16-column block and receives it transposed).
// Entries < 0 or >= n_kv are skipped.  No atomics: every output element and
// lse entry has one writer.
//
// Workgroups run one per CU, so rows x head blocks units fill whole rounds of
// the chip plus a last, partial one.  With a workspace, each unit of that last
// round is split into nsplit workgroups over consecutive ranges of its SORTED
// tiles (so the split, like the sort, ignores the caller's order); each writes
// its unnormalized O, reference max and sum, and a second kernel merges the
// ranges in range order.
#include "vea_internal.h"

#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

namespace vea {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

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

// The MFMAs are emitted as inline asm so that the register class of each
// accumulator is fixed: O^T in AGPRs (256 of them), S^T in VGPRs next to the
// softmax that reads it.  The compiler does not see these as MFMAs, so the
// wait states the CDNA3/4 ISA requires around matrix instructions are issued
// here by hand (at most 18 for an XDL result read or overwritten by a VALU,
// LDS or memory instruction, 2 for a VALU result read by an XDL instruction;
// a margin on both).  The asm is not volatile, so LDS reads can still be
// scheduled ahead of the MFMAs that use them; every wait is ordered against
// the MFMAs by a register dependency (the wait "rewrites" the registers it
// guards), never by volatility.
__device__ __forceinline__ void mfma_s_first(floatx16& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(floatx16& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o(floatx16& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// XDL result in VGPRs -> any other reader: 20 wait states.
__device__ __forceinline__ void xdl_drain_v(floatx16& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(d));
}
// The 16 O^T accumulators (AGPRs) after the last MFMA that wrote them, before
// anything else reads or writes them: 20 wait states.
#define VEA_O16(o) "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), \
    "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15])
__device__ __forceinline__ void xdl_drain_o(floatx16 (&o)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : VEA_O16(o));
}
// VALU writes of the O^T accumulators -> the next MFMA reading them: 5 wait states.
__device__ __forceinline__ void valu_to_xdl_o(floatx16 (&o)[16]) {
  asm volatile("s_nop 4" : VEA_O16(o));
}
#undef VEA_O16
// VALU result -> XDL operand: 5 wait states.
__device__ __forceinline__ void valu_to_xdl(u32x4& x, u32x4& y) {
  asm volatile("s_nop 4" : "+v"(x), "+v"(y));
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ float lane_swap_max(float x) {
  // max with the lane 32 apart (the other half of the wave holds the same head)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int DQK, int DV, int MAXK>
struct SCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int HPW = 32;                       // heads per wave (MFMA N)
  static constexpr int HEADS = WAVES * HPW;            // heads per workgroup
  static constexpr int BN = 32;                        // sorted indices per step
  static constexpr int ROWB = DQK * 2;                 // bytes per latent row (no padding)
  static constexpr int TILE = BN * ROWB;
  static constexpr int CPR = DQK / 8;                  // 16-byte chunks per row
  static constexpr int BLOCKS = TILE / 1024;           // 1 KB DMA blocks per tile
  static constexpr int BPW = BLOCKS / WAVES;           // DMA blocks per wave per tile
  static constexpr int KSTEPS = DQK / 16;              // k-steps of S^T
  static constexpr int NT = DV / 32;                   // 32-wide d_v tiles of O^T
  // Ring of LDS stages.  The DMA of tile t + DIST is issued at step t, while
  // QK^T reads tile t and P V reads tile t - 1, so NSTAGE = DIST + 2.  Up to
  // 2048 indices the sorted list leaves room for four stages (prefetch two
  // tiles ahead); up to 4096, three.
  static constexpr int NSTAGE = MAXK <= 2048 ? 4 : 3;
  static constexpr int DIST = NSTAGE - 2;
  static_assert(TILE % 1024 == 0 && BLOCKS % WAVES == 0, "tile in whole 1 KB DMA blocks per wave");
  static_assert(CPR % 8 == 0, "swizzle stays inside aligned groups of 8 chunks");
  static_assert(DQK % 32 == 0 && DV % 64 == 0 && DV <= DQK, "latent dims");
  static_assert(HEADS == kSparseHeadsPerWG, "host launch shape");
  static_assert(NT == 16, "the accumulator waits name 16 O^T tiles");
  // Sorted index list: MAXK entries plus DIST tiles of padding, read (never
  // used) by the DMAs of the steps past the last tile.
  static constexpr int SIDX = MAXK + DIST * BN;
  // 32-bit words of LDS left for the counting sort's counts (two per word)
  static constexpr int CNTW = (160 * 1024 - NSTAGE * TILE - SIDX * 4 - WAVES * 4) / 4;
  static_assert(CNTW > 0, "LDS budget");
  // Q through the ring needs a stage per wave (one stage = one wave's Q
  // rows); the three-stage variant loads Q straight into registers.
  static constexpr bool QDMA = NSTAGE >= WAVES;
  static_assert(TILE == HPW * ROWB, "a wave's Q rows fill one stage");
  // Chunk swizzle.  Rows r and r + 1 sit 32 banks apart (1152-byte rows), so
  // the swizzle works on the row pair x = (r / 2) % 8 and permutes the low 3
  // bits of a chunk index (it stays inside aligned groups of 8 chunks; rows r
  // and r + 16 share a swizzle).
  //  * K reads (ds_read_b128, 16 lanes = 16 consecutive rows x one logical
  //    chunk): the swizzle must be a permutation of x = 0..7.
  //  * V^T reads (ds_read_b64_tr_b16, 32 lanes = 4 consecutive rows x 4
  //    logical chunks 4n..4n+3): the two row pairs of an aligned group of 4
  //    rows need swizzles that differ in bit 2.
  // x -> (x & 1) << 2 | x >> 1 satisfies both.
  static __device__ __forceinline__ int swz(int r) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  }
};

// One 16-byte DMA per lane from global memory straight into LDS: lane l's
// chunk lands at lds_block + 16 l.  Written as asm so that the compiler does
// not track it: it would otherwise stop every LDS read of another stage until
// the DMA lands (it cannot tell the stages of the ring apart).  The kernel
// orders these DMAs itself (s_waitcnt vmcnt before the barrier that precedes
// the reads).  Offsets past num_records read as zeros.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_block, uint32_t voffset) {
  // M0 is saved and restored around the DMA (it is a reserved register); one
  // wait state separates the M0 write from the DMA that reads it.
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(lds_block), "s"(rsrc));
}

template <int DQK, int DV, int MAXK>
__global__ __launch_bounds__(256, 1) void sparse_mqa_kernel(SparseParams p) {
  using C = SCfg<DQK, DV, MAXK>;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[C::NSTAGE * C::TILE];
  __shared__ int sidx[C::SIDX];
  __shared__ int wsum[C::WAVES];
  __shared__ uint32_t cntbuf[C::CNTW];

  // workgroup unit (row, head block) and, for a split unit, its chunk
  const int slot = wg_slot(blockIdx.x, p.grid, p.wg_perm);
  int unit = slot, chunk = 0;
  const bool split = unit >= p.full_units;
  if (split) {
    const int u2 = unit - p.full_units;
    const int tu = u2 / p.nsplit;
    chunk = u2 - tu * p.nsplit;
    unit = p.full_units + tu;
  }
  const int row = unit / p.head_blocks;
  const int hb = unit - row * p.head_blocks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) value
  const int l32 = lane & 31;
  const int g2 = lane >> 5;                             // which half of the wave

  // ---- this thread's share of the row's indices (entries tid + THREADS j;
  // entries past k are excluded where they are used), loaded first so their
  // latency overlaps the count buffer's clearing.
  const int32_t* irow = p.idx + (int64_t)row * p.k;
  constexpr int IPT = MAXK / C::THREADS;
  int xi[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) xi[j] = irow[min(tid + C::THREADS * j, p.k - 1)];
  const int head0 = hb * C::HEADS + wave * C::HPW;      // wave-uniform
  const bool active = head0 < p.heads;                  // wave has at least one head
  u32x4 qf[C::KSTEPS];
  if constexpr (!C::QDMA) {
    // Q^T fragments straight from global memory (head l32 of this wave, dims
    // 16 ks + 8 g2 .. +7), issued after the index loads so the sort waits
    // for those alone; heads past the count load head 0 and are zeroed later.
    const int hq = head0 + l32 < p.heads ? head0 + l32 : 0;
    const uint16_t* src = p.q + ((int64_t)row * p.heads + hq) * DQK + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[ks] = *(const u32x4*)(src + 16 * ks);
  }
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  const float c = fmaxf(fabsf(p.scale) * kLog2e, FLT_MIN);   // scale 0: logits ~0, masked ones stay -inf

  // ---- Q of this wave's 32 heads by DMA into stage `wave` of the ring,
  // which is idle until the key loop: 36 fully coalesced 1 KB blocks (the
  // heads of a row are consecutive), laid out like a K tile (head r in
  // place of latent row r, same chunk swizzle), so the Q^T fragments (B
  // operand of S^T = K Q^T: head l32, dims 16 ks + 8 g2 .. +7) are read
  // back exactly like K operands.  Loading them straight into registers
  // would make every load instruction touch 32 rows.  Heads past the count
  // read zeros.  Issued once the sort no longer needs the ring (the
  // counting sort keeps its counts there when they do not fit cntbuf).
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)ring;
  const uint64_t q_addr = (uint64_t)(uintptr_t)(p.q + (int64_t)row * p.heads * DQK);
  const i32x4 q_rsrc = (i32x4){(int)(uint32_t)q_addr, (int)(uint32_t)(q_addr >> 32) & 0xFFFF, p.heads * C::ROWB,
                               0x00020000};
  auto q_dma = [&] {
    if constexpr (!C::QDMA) return;
    const uint32_t dst = ring_lds + (uint32_t)(wave * C::TILE);
#pragma unroll
    for (int bk = 0; bk < C::BLOCKS; ++bk) {
      const int sl = bk * 64 + lane;
      const int r = sl / C::CPR;
      const int ph = sl - r * C::CPR;
      const int col = 16 * ((ph & ~7) | ((ph & 7) ^ C::swz(r)));
      const uint32_t off = __umul24((uint32_t)(head0 + r), (uint32_t)C::ROWB) + (uint32_t)col;
      dma16(q_rsrc, dst + (uint32_t)(bk * 1024), head0 + r < p.heads ? off : 0xFFFFFFF0u);
    }
  };
  bool q_issued = false;

  // ---- canonical order: the row's valid indices in ascending order (with
  // their multiplicity) in sidx[0, nvalid).
  int nvalid;
  if (p.n_kv <= C::NSTAGE * C::TILE / 2) {
    // Counting sort in the stage ring (idle until the key loop): a 16-bit
    // count per latent row (two per word; k <= 4096 cannot overflow one),
    // incremented by LDS atomics (the counts do not depend on their order),
    // then one block-wide exclusive scan over runs of consecutive rows and a
    // scatter of each row's index count times.
    const bool own = p.n_kv <= 2 * C::CNTW;             // counts in cntbuf: the ring is free for Q
    uint32_t* cnt = own ? cntbuf : (uint32_t*)ring;
    const int nw = (p.n_kv + 1) >> 1;
    for (int i = tid; i < nw; i += C::THREADS) cnt[i] = 0u;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int x = xi[j];
      if (tid + C::THREADS * j < p.k && x >= 0 && x < p.n_kv)   // padding / out of range: skipped
        atomicAdd(&cnt[x >> 1], 1u << (16 * (x & 1)));
    }
    lds_barrier();
    if (own) {                                          // the index loads are in: Q's DMAs run under the scan
      q_dma();
      q_issued = true;
    }
    // Each thread owns a run of `per` consecutive rows (even, so the run
    // starts on a count word), read RPT rows (RPT / 2 independent words) at
    // a time; the high half of the last word past n_kv was cleared above.
    constexpr int RPT = 16;
    const int per = ((p.n_kv + C::THREADS - 1) / C::THREADS + 1) & ~1;
    const int v0 = min(tid * per, p.n_kv), v1 = min(v0 + per, p.n_kv);
    auto words = [&](int vb, uint32_t (&w)[RPT / 2]) {
#pragma unroll
      for (int j = 0; j < RPT / 2; ++j) w[j] = vb + 2 * j < v1 ? cnt[(vb >> 1) + j] : 0u;
    };
    int tot = 0;
    for (int vb = v0; vb < v1; vb += RPT) {
      uint32_t w[RPT / 2];
      words(vb, w);
#pragma unroll
      for (int j = 0; j < RPT / 2; ++j) tot += (int)((w[j] & 0xFFFFu) + (w[j] >> 16));
    }
    int incl = tot;                                     // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    lds_barrier();
    int base = incl - tot;
    nvalid = 0;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) {
      if (w < wave) base += wsum[w];
      nvalid += wsum[w];
    }
    for (int vb = v0; vb < v1; vb += RPT) {
      uint32_t w[RPT / 2];
      words(vb, w);
#pragma unroll
      for (int j = 0; j < 2 * (RPT / 2); ++j) {         // row vb + j appears count times
        const int c = (int)((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
        if (c == 1) sidx[base] = vb + j;                // the usual case: distinct indices
        else for (int r = 0; r < c; ++r) sidx[base + r] = vb + j;
        base += c;
      }
    }
    lds_barrier();
  } else {
    // Bitonic sorting network in LDS; padding and out-of-range entries become
    // INT_MAX and sort to the end.
    int n2 = 1;
    while (n2 < p.k) n2 <<= 1;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int i = tid + C::THREADS * j;
      const int x = xi[j];
      if (i < n2) sidx[i] = (i < p.k && x >= 0 && x < p.n_kv) ? x : INT_MAX;
    }
    lds_barrier();
    q_dma();                                            // the network works in sidx only
    q_issued = true;
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (n2 >> 1); t += C::THREADS) {
          const int i = 2 * t - (t & (stride - 1));
          const int j = i + stride;
          const bool up = (i & size) == 0;
          const int a = sidx[i], b = sidx[j];
          if ((a > b) == up) { sidx[i] = b; sidx[j] = a; }
        }
        lds_barrier();
      }
    }
    // number of valid entries: first position holding INT_MAX (binary search)
    int lo = 0, hi = n2;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sidx[mid] == INT_MAX) hi = mid; else lo = mid + 1;
    }
    nvalid = lo;
  }
  // Tiles [t0, t0 + n_tiles) of the sorted list: all of them, or this
  // chunk's share of a split unit.  The key loop sees the list from entry
  // t0 BN on (srow) and the valid count from there (nloc).
  nvalid = __builtin_amdgcn_readfirstlane(nvalid);
  if (!q_issued) q_dma();                               // counts were in the ring
  if (p.page_table != nullptr) {
    // Paged cache: translate the sorted logical positions to physical rows
    // in place.  The order stays that of the logical positions, so the
    // result does not depend on where the pages happen to be.
    const int pmask = (1 << p.page_shift) - 1;
    for (int i = tid; i < nvalid; i += C::THREADS) {
      const int x = sidx[i];
      sidx[i] = (p.page_table[x >> p.page_shift] << p.page_shift) | (x & pmask);
    }
    lds_barrier();
  }
  const int n_all = (nvalid + C::BN - 1) / C::BN;
  // The rest of the last tile holds n_phys: its DMA offset is past the
  // buffer's record bound, so those rows read as zeros.
  for (int i = nvalid + tid; i < n_all * C::BN; i += C::THREADS) sidx[i] = p.n_phys;
  lds_barrier();
  int t0 = 0, n_tiles = n_all;
  if (split) {
    t0 = (n_all * chunk) / p.nsplit;
    n_tiles = (n_all * (chunk + 1)) / p.nsplit - t0;
  }
  const int nloc = nvalid - t0 * C::BN;
  const int* srow = sidx + t0 * C::BN;


  // ---- gather by DMA: 1 KB block bk of a tile is filled by wave bk % WAVES;
  // slot sl of the tile holds row sl / CPR, physical chunk sl % CPR =
  // logical chunk ^ swz(row).
  const uint64_t kv_addr = (uint64_t)(uintptr_t)p.kv;
  const int kv_records = (int)((int64_t)p.n_phys * C::ROWB);
  const i32x4 kv_rsrc = (i32x4){(int)(uint32_t)kv_addr, (int)(uint32_t)(kv_addr >> 32) & 0xFFFF, kv_records,
                                0x00020000};
  // Slot (row, byte column) of each of this lane's DMA blocks, packed
  // row << 16 | column; the same for every tile.
  int g_rc[C::BPW];
#pragma unroll
  for (int bi = 0; bi < C::BPW; ++bi) {
    const int sl = (bi * C::WAVES + wave) * 64 + lane;
    const int r = sl / C::CPR;
    const int ph = sl - r * C::CPR;
    g_rc[bi] = (r << 16) | (16 * ((ph & ~7) | ((ph & 7) ^ C::swz(r))));
  }
  // A gather is issued for every step, also for tiles past this range's
  // n_tiles (those DMAs get a record bound of 0, so they read zeros into a
  // stage no step reads again), so that the key loop has no branch around
  // it and the count of DMAs in flight at each wait is fixed; their index
  // reads stay inside sidx, (t0 + n_tiles + DIST) BN <= SIDX.  The index
  // reads (gather_idx) and the DMAs (gather_dma, one per block) are separate
  // so that the step can spread them between its MFMAs.  g_rc is read
  // through an opaque copy at each use, so that its row and column parts are
  // recomputed there rather than kept live as 18 values.
  auto gather_idx = [&](int kt, int bi) -> int {
    int g = g_rc[bi];
    asm volatile("" : "+v"(g));
    return srow[kt * C::BN + (g >> 16)];
  };
  auto gather_dma = [&](int kt, int x, int bi) {
    const uint32_t dst = ring_lds + (uint32_t)((kt % C::NSTAGE) * C::TILE);
    i32x4 rs = kv_rsrc;
    rs[2] = __builtin_amdgcn_readfirstlane(kt < n_tiles ? kv_records : 0);
    int g = g_rc[bi];
    asm volatile("" : "+v"(g));
    dma16(rs, __builtin_amdgcn_readfirstlane(dst + (uint32_t)((bi * C::WAVES + wave) * 1024)),
          __umul24((uint32_t)x, (uint32_t)C::ROWB) + (uint32_t)(g & 0xFFFF));
  };
  auto gather = [&](int kt) {
    int x[C::BPW];
#pragma unroll
    for (int bi = 0; bi < C::BPW; ++bi) x[bi] = gather_idx(kt, bi);
#pragma unroll
    for (int bi = 0; bi < C::BPW; ++bi) gather_dma(kt, x[bi], bi);
  };


  // ---- per-lane LDS read offsets.  Chunk 8 a + b (b < 8) sits at
  // 16 (8 a + (b ^ swz)): a per-lane base per low-bit class plus 128 a.
  const int ksw = C::swz(l32);                          // same for rows l32 and l32 + 16
  int kb[4];                                            // K row l32, chunk 2 ks + g2, ks = 4 a + b
#pragma unroll
  for (int b = 0; b < 4; ++b) kb[b] = l32 * C::ROWB + 16 * ((2 * b + g2) ^ ksw);
  const int i16 = lane & 15, nh = (lane >> 4) & 1;
  const int vr0 = 4 * g2 + (i16 >> 2);                 // key row of the first 4-key read (+ 16 kst)
  const int vx = 2 * nh + ((i16 & 3) >> 1);            // low chunk bits within a 32-column tile
  int vb0[2], vb1[2];                                   // V rows vr0 and vr0 + 8; nt & 1 selects
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    vb0[e] = vr0 * C::ROWB + 16 * ((4 * e + vx) ^ C::swz(vr0)) + 8 * (i16 & 1);
    vb1[e] = (vr0 + 8) * C::ROWB + 16 * ((4 * e + vx) ^ C::swz(vr0 + 8)) + 8 * (i16 & 1);
  }

  floatx16 o[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    o[nt] = (floatx16){};
    asm("" : "+a"(o[nt]));                              // O^T lives in AGPRs from the start
  }
  float m_used = -INFINITY;  // reference max (times c, log2 domain)
  float l_run = 0.f;         // this lane's partial sum of P

  auto mask_tail = [&](int kt, floatx16& s) {
    if ((kt + 1) * C::BN > nloc) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kt * C::BN + 8 * (r >> 2) + 4 * g2 + (r & 3) >= nloc) s[r] = -INFINITY;
    }
  };
  // ---- one step of the key loop, as an explicitly scheduled sequence of
  // MFMA slots: slots 0..KSTEPS-1 are the QK^T k-steps of tile t (S^T[key
  // 8 (r/4) + 4 g2 + r%4][head l32] accumulates in s), the next 2 NT slots
  // the P V MFMAs of tile t-1 (P already packed in pb).  Each slot issues the
  // LDS read of the operand PD slots ahead and ends in a scheduling barrier,
  // so the register footprint stays fixed (the compiler would otherwise hoist
  // every read of the step).  The softmax of tile t runs on the VALU under
  // the P V MFMAs of tile t-1:
  //   * head max of the tile; the reference max moves only when the tile max
  //     exceeds it by more than 8 (log2 units), so P stays below 2^8 (lazy
  //     rescaling); the final lse uses the same reference, so the result is
  //     exact in real arithmetic;
  //   * l is rescaled at once; O (which P V of tile t-1 is still writing) is
  //     rescaled after the step's last MFMA, in a rare branch;
  //   * P = 2^(s c - m) with an fp32 sum for l, rounded to bf16 and packed:
  //     k-slot j of lane half g2 in P V k-step kst is key 16 kst + 8 (j / 4) +
  //     4 g2 + j % 4, i.e. accumulator entry 8 kst + j, for both the P^T and
  //     the V^T operand.
  constexpr int PD = 4;
  constexpr int NQK = C::KSTEPS, NPV = 2 * C::NT;
  auto load_op = [&](const unsigned char* kst, const unsigned char* vst, auto slot_tag) -> u32x4 {
    constexpr int SL = decltype(slot_tag)::value;
    if constexpr (SL < NQK) {
      return *(const u32x4*)(kst + kb[SL & 3] + 128 * (SL >> 2));
    } else {
      constexpr int J = SL - NQK, KS = J / C::NT, NTI = J % C::NT;
      constexpr int OFF = KS * 16 * C::ROWB + 128 * (NTI >> 1);   // 16 key rows per k-step; 8 chunks per tile pair
      const u32x2 lo = lds_read_tr(vst + vb0[NTI & 1] + OFF);
      const u32x2 hi = lds_read_tr(vst + vb1[NTI & 1] + OFF);
      return (u32x4){lo[0], lo[1], hi[0], hi[1]};
    }
  };
  // Softmax of the tile in s, cut into small VALU pieces that the P V slots
  // interleave, one per slot: with one wave per SIMD nothing else hides the
  // latency of a dependent VALU chain, so each piece only consumes values
  // produced at least one slot earlier.
  struct Soft {
    float mx[4], alpha, m_use;
    bool any_upd;
    float e[16];
    uint32_t w[8];
  };
  auto soft_piece = [&](floatx16& s, Soft& sf, auto piece_tag) {
    constexpr int P = decltype(piece_tag)::value;
    if constexpr (P == 0) {                             // head max: four partial trees
      sf.mx[0] = vmax(vmax(s[0], s[1]), s[2]);
      sf.mx[1] = vmax(vmax(s[3], s[4]), s[5]);
      sf.mx[2] = vmax(vmax(s[6], s[7]), s[8]);
      sf.mx[3] = vmax(vmax(s[9], s[10]), s[11]);
    } else if constexpr (P == 1) {
      sf.mx[0] = vmax(vmax(sf.mx[0], sf.mx[1]), s[12]);
      sf.mx[2] = vmax(vmax(sf.mx[2], sf.mx[3]), vmax(vmax(s[13], s[14]), s[15]));
    } else if constexpr (P == 2) {
      sf.mx[0] = lane_swap_max(vmax(sf.mx[0], sf.mx[2]));
    } else if constexpr (P == 3) {                      // reference update (lazy: only beyond 2^8)
      const float mx_sc = (sf.mx[0] == -INFINITY) ? -INFINITY : sf.mx[0] * c;
      const bool upd = mx_sc > m_used + 8.0f;
      sf.any_upd = __any(upd);
      const float m_new = upd ? mx_sc : m_used;
      sf.alpha = upd ? fast_exp2(m_used - m_new) : 1.0f;
      sf.m_use = (m_new == -INFINITY) ? 0.f : m_new;
      m_used = m_new;
    } else if constexpr (P == 4) {
      l_run *= sf.alpha;
      sf.e[0] = fast_exp2(fmaf(s[0], c, -sf.m_use));
      sf.e[1] = fast_exp2(fmaf(s[1], c, -sf.m_use));
    } else if constexpr (P < 12) {                      // pieces 5..11: two probabilities, pack / sum the previous two
      constexpr int R = 2 * (P - 4);
      sf.e[R] = fast_exp2(fmaf(s[R], c, -sf.m_use));
      sf.e[R + 1] = fast_exp2(fmaf(s[R + 1], c, -sf.m_use));
      sf.w[(R - 2) >> 1] = pack_bf16x2(sf.e[R - 2], sf.e[R - 1]);
      l_run += sf.e[R - 2] + sf.e[R - 1];
    } else if constexpr (P == 12) {
      sf.w[7] = pack_bf16x2(sf.e[14], sf.e[15]);
      l_run += sf.e[14] + sf.e[15];
      asm volatile("" : "+v"(l_run));                   // summed here, not after the step
    }
  };
  auto rescale_o = [&](const Soft& sf) {
    if (sf.any_upd) {
      asm volatile("; rare: the reference max moved, rescale O" ::);
      xdl_drain_o(o);
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {              // one tile at a time through VGPRs
        o[nt] *= sf.alpha;
        asm volatile("" : "+a"(o[nt]));
        __builtin_amdgcn_sched_barrier(0);
      }
      valu_to_xdl_o(o);
    }
  };
  // QK: the QK^T slots of the tile in kst into s, then (PV) the P V slots of
  // the previous tile (pb, V from vst) with the softmax of s under them.
  // Returns the packed P of s in pb.  The gather of tile kg is spread over
  // the step's MFMA slots, one DMA every GSP slots from slot GS on (every
  // slot's worth of DMAs at once would queue behind each other in the
  // texture unit and stall the issuing wave); the index read of each block
  // goes out GS slots before its DMA, so it has returned with the operand
  // reads issued before it.
  constexpr int GS = PD;
  constexpr int GSP_QK = (NQK - GS) / C::BPW;               // step 0: QK^T slots only
  constexpr int GSP_PV = 5;                                 // measured ~1% faster than 4, 6 or 7
  static_assert(GS + (C::BPW - 1) * GSP_PV < NQK + NPV, "the gather fits in the step");
  static_assert(GSP_QK >= 1 && GS + (C::BPW - 1) * GSP_QK < NQK, "the gather fits under the QK^T slots");
  auto step_mma = [&](int kt, int kg, const unsigned char* kst, const unsigned char* vst, floatx16& s, u32x4* pb,
                      Soft& sf, auto pv_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr int LAST = PV ? NQK + NPV : NQK;
    constexpr int GSP = PV ? GSP_PV : GSP_QK;
    u32x4 opr[PD];
    int xg[C::BPW];
    static_for<0, PD>([&](auto i) { opr[i.value] = load_op(kst, vst, i); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, LAST>([&](auto slot_tag) {
      constexpr int SL = decltype(slot_tag)::value;
      const u32x4 a = opr[SL % PD];
      if constexpr (SL + PD < LAST) opr[SL % PD] = load_op(kst, vst, std::integral_constant<int, SL + PD>{});
      if constexpr (SL % GSP == 0 && SL / GSP < C::BPW) xg[SL / GSP] = gather_idx(kg, SL / GSP);
      if constexpr (SL >= GS && (SL - GS) % GSP == 0 && (SL - GS) / GSP < C::BPW)
        gather_dma(kg, xg[(SL - GS) / GSP], (SL - GS) / GSP);
      if constexpr (SL < NQK) {
        // one accumulator: MFMAs that accumulate into the same registers
        // issue back to back at the full rate
        if constexpr (SL == 0) mfma_s_first(s, a, qf[0]);
        else mfma_s(s, a, qf[SL]);
        if constexpr (SL == NQK - 1 && !PV) {
          xdl_drain_v(s);
          mask_tail(kt, s);                             // keys past the valid count -> -inf
        }
      } else {
        constexpr int J = SL - NQK, KS = J / C::NT, NTI = J % C::NT;
        mfma_o(o[NTI], a, pb[KS]);
        if constexpr (J == 0) {                         // under the first P V MFMA: finish S^T
          xdl_drain_v(s);
          mask_tail(kt, s);                             // keys past the valid count -> -inf
        }
        // softmax pieces under P V slots 1 .. 13
        if constexpr (J >= 1 && J <= 13) soft_piece(s, sf, std::integral_constant<int, J - 1>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (!PV) static_for<0, 13>([&](auto piece) { soft_piece(s, sf, piece); });
  };
  auto pack_p = [&](const Soft& sf, u32x4* pb) {
    pb[0] = (u32x4){sf.w[0], sf.w[1], sf.w[2], sf.w[3]};
    pb[1] = (u32x4){sf.w[4], sf.w[5], sf.w[6], sf.w[7]};
    valu_to_xdl(pb[0], pb[1]);
  };
  // Last P V (no QK^T slots).
  static_assert(NQK % PD == 0, "last_pv's operand ring starts where step_mma's left off");
  auto last_pv = [&](const unsigned char* vst, const u32x4* pb) {
    u32x4 opr[PD];
    static_for<0, PD>([&](auto i) { opr[i.value] = load_op(vst, vst, std::integral_constant<int, NQK + i.value>{}); });
    static_for<NQK, NQK + NPV>([&](auto slot_tag) {
      constexpr int SL = decltype(slot_tag)::value;
      const u32x4 a = opr[SL % PD];
      if constexpr (SL + PD < NQK + NPV) opr[SL % PD] = load_op(vst, vst, std::integral_constant<int, SL + PD>{});
      constexpr int J = SL - NQK, KS = J / C::NT, NTI = J % C::NT;
      mfma_o(o[NTI], a, pb[KS]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Wait until this lane's DMA of tile t has landed (with DIST 2 the DMAs
  // of tile t + 1, real or past the range, stay in flight; vector memory
  // loads complete in issue order), then for every wave's.  The barrier also
  // retires the reads of the stage the next DMA refills.
  auto wait_tile = [&](int) {
    if constexpr (C::DIST == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::BPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto stage_ptr = [&](int t) -> const unsigned char* { return ring + (t % C::NSTAGE) * C::TILE; };

  // Q^T fragments from this wave's stage once its own DMAs have landed
  // (nothing else is in flight on the vector memory counter now); every
  // wave is done reading before the first tiles overwrite the stages.
  if constexpr (C::QDMA) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const unsigned char* qst = ring + wave * C::TILE;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[ks] = *(const u32x4*)(qst + kb[ks & 3] + 128 * (ks >> 2));
    lds_barrier();
  }
  if (n_tiles > 0) {
    gather(0);
    if constexpr (C::DIST == 2) gather(1);
  }
  // Q of heads past the count is zero (the DMA reads zeros for them); a
  // negative scale negates Q (exact sign-bit flip) so the exponent scale is
  // positive.
  if constexpr (!C::QDMA) {
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
      if (head0 + l32 >= p.heads) qf[ks] = (u32x4){0u, 0u, 0u, 0u};
  }
  if (p.scale < 0.f) {
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[ks] ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  // Retire the Q reads or loads here: otherwise the compiler waits for them
  // (lgkmcnt(0) or vmcnt(0), which would also drain the operand reads or the
  // tile DMAs in flight) at their first use inside the key loop, on every
  // iteration.
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) asm volatile("" : "+v"(qf[ks]));

  if (n_tiles > 0) {
    u32x4 pb[2];                                        // packed P of the previous tile
    // step 0: QK^T and softmax of tile 0
    wait_tile(0);
    if (active) {
      floatx16 s;
      Soft sf;
      step_mma(0, C::DIST, stage_ptr(0), stage_ptr(0), s, pb, sf, std::false_type{});
      pack_p(sf, pb);
    } else {
      gather(C::DIST);
    }
    // steps 1 .. n_tiles-1: QK^T and softmax of tile t under P V of tile t-1
    for (int t = 1; t < n_tiles; ++t) {
      wait_tile(t);
      if (active) {
        floatx16 s;
        Soft sf;
        step_mma(t, t + C::DIST, stage_ptr(t), stage_ptr(t - 1), s, pb, sf, std::true_type{});
        // P packed before the rare rescale branch: with its uses after the
        // branch the compiler sinks the exponentials past it, out from under
        // the MFMAs of the step
        pack_p(sf, pb);
        rescale_o(sf);
      } else {
        gather(t + C::DIST);
      }
    }
    // last step: P V of tile n_tiles-1
    if (active) last_pv(stage_ptr(n_tiles - 1), pb);
    // the DMAs past the range may still be writing their (unread) stages
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // ---- epilogue: O / l (bf16 RNE), lse = ln 2 * (m + log2 l)
  xdl_drain_o(o);
  float l_tot = l_run;
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_tot), __float_as_uint(l_tot), false, false);
    l_tot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  // The result goes out through LDS: each wave stages SROWS of its 32 rows
  // (heads, 1 KB each) at a time in its own part of the ring, 16-byte chunk
  // c of staged row r at chunk c ^ (r % 16), then writes whole 1 KB rows
  // with one 16-byte store per lane, rather than 32 scattered 8-byte pieces
  // per store.  All waves must be done with the ring first.
  constexpr int SROWS = C::NSTAGE * C::TILE / C::WAVES >= 32 * 1024 ? 32 : 16;
  static_assert(C::WAVES * SROWS * 1024 <= C::NSTAGE * C::TILE, "staging fits the ring");
  lds_barrier();
  // lane values for the epilogue, opaque to the compiler so that nothing
  // derived from them is computed before the key loop and kept live over it
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int l32e = lane_e & 31, g2e = lane_e >> 5;
  unsigned char* stg = ring + wave * SROWS * 1024;
  const int sr = l32e % SROWS;                           // this lane's staged row, in its pass
  const int hsw = sr & 15;
  const int hl0 = wave * C::HPW;                        // first head of this wave within the workgroup
  if (split) {
    // partial result of this key range: unnormalized O^T in fp32 (a row is
    // two 1 KB halves, staged one half at a time), reference max m (log2
    // domain) and sum l, per head of the workgroup
    float* w = p.ws + (size_t)(slot - p.full_units) * (C::HEADS * (DV + 2));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int ps = 0; ps < C::HPW / SROWS; ++ps) {
        if (l32e / SROWS == ps) {
#pragma unroll
          for (int nt = 8 * half; nt < 8 * half + 8; ++nt) {
            // a fresh AGPR value per tile, so the reads stay in this branch
            // and in tile order (hoisted they would need 256 VGPRs at once)
            asm volatile("" : "+a"(o[nt]));
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int ch = 8 * (nt - 8 * half) + 2 * r4 + g2e;   // 16-byte chunk of the half-row
              *(floatx4*)(stg + sr * 1024 + 16 * (ch ^ hsw)) =
                  (floatx4){o[nt][4 * r4], o[nt][4 * r4 + 1], o[nt][4 * r4 + 2], o[nt][4 * r4 + 3]};
            }
          }
        }
#pragma unroll 4
        for (int h = 0; h < SROWS; ++h) {
          const floatx4 v = *(const floatx4*)(stg + h * 1024 + 16 * (lane_e ^ (h & 15)));
          *(floatx4*)(w + (hl0 + ps * SROWS + h) * DV + 256 * half + 4 * lane_e) = v;
        }
      }
    }
    if (g2e == 0) {
      w[C::HEADS * DV + hl0 + l32e] = m_used;
      w[C::HEADS * DV + C::HEADS + hl0 + l32e] = l_tot;
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* dst = p.out + ((int64_t)row * p.heads + head0) * DV + 8 * lane_e;
  const int nrows = min(C::HPW, p.heads - head0);       // rows of this wave that exist
#pragma unroll
  for (int ps = 0; ps < C::HPW / SROWS; ++ps) {
    if (l32e / SROWS == ps) {
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        asm volatile("" : "+a"(o[nt]));                // as in the split branch
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(u32x2*)(stg + sr * 1024 + 16 * ((4 * nt + r4) ^ hsw) + 8 * g2e) =
              (u32x2){pack_bf16x2(o[nt][4 * r4] * inv, o[nt][4 * r4 + 1] * inv),
                      pack_bf16x2(o[nt][4 * r4 + 2] * inv, o[nt][4 * r4 + 3] * inv)};
      }
    }
    const int hn = min(SROWS, nrows - ps * SROWS);
#pragma unroll 4
    for (int h = 0; h < hn; ++h)
      *(u32x4*)(dst + (ps * SROWS + h) * DV) = *(const u32x4*)(stg + h * 1024 + 16 * (lane_e ^ (h & 15)));
  }
  if (head0 + l32e < p.heads) {
    if (p.lse != nullptr && g2e == 0)
      p.lse[(int64_t)(head0 + l32e) * p.rows + row] = l_tot > 0.f ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge of the split chunks of one workgroup unit, in chunk order (fixed, so
// the result is deterministic): with M = max_i m_i,
//   O = sum_i 2^(m_i - M) O_i,  l = sum_i 2^(m_i - M) l_i,
//   out = O / l (bf16),  lse = ln 2 (M + log2 l),
// the blockwise merge of eq. (1)(2) (page above, section 进一步探索) with the
// O update written out.  Workgroup (tail unit, group of HPG heads); one
// thread per (head, 16-column slice).  Empty chunks carry m = -inf, l = 0.
template <int DV, int HEADS, int HPG, int NS>
__global__ __launch_bounds__(256) void sparse_merge_kernel(SparseParams p) {
  const int tu = blockIdx.x;                            // tail unit
  const int unit = p.full_units + tu;
  const int row = unit / p.head_blocks;
  const int hb = unit - row * p.head_blocks;
  constexpr size_t CF = (size_t)HEADS * (DV + 2);       // floats per chunk
  constexpr int SLICES = DV / 16;
  static_assert(HPG * SLICES == 256, "one item per thread");
  const float* base = p.ws + (size_t)tu * NS * CF;
  const int hl = blockIdx.y * HPG + threadIdx.x / SLICES;
  const int sc = threadIdx.x % SLICES;
  const int head = hb * HEADS + hl;
  if (head >= p.heads) return;
  // every chunk's m, l and 16 values loaded up front (one memory latency)
  float mi[NS], li[NS];
  floatx4 vi[NS][4];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const float* c = base + i * CF;
    mi[i] = c[HEADS * DV + hl];
    li[i] = c[HEADS * DV + HEADS + hl];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) vi[i][q4] = ((const floatx4*)(c + hl * DV + 16 * sc))[q4];
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
  uint16_t* dst = p.out + ((int64_t)row * p.heads + head) * DV + 16 * sc;
  *(u32x4*)dst = w[0];
  *(u32x4*)(dst + 8) = w[1];
  if (sc == 0 && p.lse != nullptr)
    p.lse[(int64_t)head * p.rows + row] = l > 0.f ? (mmax + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

SparseSplit sparse_split_plan(int units, int k, int cus) {
  // Units are dispatched in order, one workgroup per CU: the last round holds
  // units % cus of them and would leave the other CUs idle for a whole row's
  // time.  Each unit of that round is split into as many key ranges as the
  // idle CUs allow (at most 8, and at most one range per 32-index tile; a
  // split below 2 is not worth the merge).
  SparseSplit s{units, 1, 0};
  if (cus <= 0 || units <= 0) return s;
  const int tail = units % cus;
  if (tail == 0) return s;
  const int nsplit = std::min(std::min(8, cus / tail), (k + 31) / 32);
  if (nsplit < 2) return s;
  s.full_units = units - tail;
  s.nsplit = nsplit;
  s.chunks = tail * nsplit;
  return s;
}

size_t sparse_chunk_bytes(int d_v) { return (size_t)kSparseHeadsPerWG * (d_v + 2) * sizeof(float); }

hipError_t launch_sparse_mqa(const SparseParams& p0, int d_qk, int d_v, hipStream_t s) {
  if (d_qk != 576 || d_v != 512) return hipErrorInvalidValue;
  if (p0.k > 4096) return hipErrorInvalidValue;
  if (p0.rows == 0) return hipSuccess;
  const int units = p0.rows * p0.head_blocks;
  if (p0.nsplit > 1 ? (p0.ws == nullptr || p0.full_units < 0 || p0.full_units >= units) : p0.full_units != units)
    return hipErrorInvalidValue;
  const int tail = units - p0.full_units;
  const dim3 grid(p0.full_units + tail * p0.nsplit), block(256);
  SparseParams p = p0;
  p.grid = (int)grid.x;
  p.wg_perm = wg_order_perm(p.grid);
  if (p.k <= 2048) hipLaunchKernelGGL((sparse_mqa_kernel<576, 512, 2048>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((sparse_mqa_kernel<576, 512, 4096>), grid, block, 0, s, p);
  if (tail > 0 && p.nsplit > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid(tail, kSparseHeadsPerWG / 8);
    switch (p.nsplit) {
      case 2: hipLaunchKernelGGL((sparse_merge_kernel<512, kSparseHeadsPerWG, 8, 2>), mgrid, dim3(256), 0, s, p); break;
      case 3: hipLaunchKernelGGL((sparse_merge_kernel<512, kSparseHeadsPerWG, 8, 3>), mgrid, dim3(256), 0, s, p); break;
      case 4: hipLaunchKernelGGL((sparse_merge_kernel<512, kSparseHeadsPerWG, 8, 4>), mgrid, dim3(256), 0, s, p); break;
      case 5: hipLaunchKernelGGL((sparse_merge_kernel<512, kSparseHeadsPerWG, 8, 5>), mgrid, dim3(256), 0, s, p); break;
      case 6: hipLaunchKernelGGL((sparse_merge_kernel<512, kSparseHeadsPerWG, 8, 6>), mgrid, dim3(256), 0, s, p); break;
      case 7: hipLaunchKernelGGL((sparse_merge_kernel<512, kSparseHeadsPerWG, 8, 7>), mgrid, dim3(256), 0, s, p); break;
      case 8: hipLaunchKernelGGL((sparse_merge_kernel<512, kSparseHeadsPerWG, 8, 8>), mgrid, dim3(256), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace vea
