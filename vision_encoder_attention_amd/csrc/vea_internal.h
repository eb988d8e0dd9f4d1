// Internal declarations shared by the HIP kernels and the C ABI layer.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vea {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ launch params
struct DenseParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;                // nullable
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t q_stride, k_stride, v_stride, o_stride;   // elements per token
  int batch, total_q, total_k;
  int hq, hkv, group;        // group = hq / hkv
  int qb;                    // rows per piece (> 0, already resolved)
  int bm;                    // query rows per tile (kDenseBM, or kD64BM for the head_dim 64 image kernel)
  int tiles_per_piece, tiles_per_seq;
  int units;                 // batch * tiles_per_seq * hq
  int xcd_map;               // 1: spread kv heads over the 8 XCDs
  float scale;
  // Key-range split of the units of the last, partial round (bf16 path):
  // units [0, full_units) run whole; each later unit is split into nsplit
  // workgroups over consecutive ranges of its key tiles, which write partial
  // (O, m, l) to ws (kDenseBM x (d + 2) floats per chunk), merged after.
  int full_units;
  int nsplit;                // 1: no split
  float* ws;                 // nullable when nsplit == 1
  // Paged K/V (bf16 path): k and v are caches of pages of 2^page_shift token
  // rows (>= the 64-key tile, so a tile never straddles a page); key row j
  // of sequence b is token row block_table[b * max_pages + (j >> page_shift)]
  // << page_shift | (j & (page size - 1)).  cu_k then only gives lengths.
  const int32_t* block_table;   // nullable: K/V packed by cu_k
  int page_shift;
  int max_pages;
  // FP8 path: q, k, v hold e4m3 codes; dequantisation scales per (query
  // token, head) [total_q, hq], per key/value head [hkv] and per (key/value
  // head, channel) [hkv, d].
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  // Decode units (> 0): unit (b, h) covers query heads h * dec_group ..
  // + dec_group - 1 of token b (q, out [batch, ...] with stride q/o_stride,
  // lse [Hq, batch]); hq then counts key/value heads and group is 1.
  int dec_group;
  // Rows per split chunk in ws: kDenseBM, or for decode units dec_group
  // rounded up to a multiple of 4 (only those rows are ever written).
  int ws_rows;
  // Order check (VEA_DEBUG_WG_ORDER): workgroup i of the grid of `grid`
  // workgroups takes grid slot wg_slot(i, grid, wg_perm); 0 is the identity.
  int grid;
  int wg_perm;
};

struct RopeParams {
  const uint16_t* x;
  const int32_t* pos;
  uint16_t* q;
  uint16_t* k;
  int64_t x_stride;
  int tokens, hq, hkv, d, pos_dims;
  int rot_half;              // 1: pairs (i, i + span/2) instead of (2i, 2i + 1)
  double theta;
};

// Grid slot of workgroup i under an order-check permutation of the grid:
// perm 0 the identity, 1 the reverse order, otherwise i * perm mod grid (perm
// coprime to grid, so a bijection).  Results must not depend on it: every
// slot is one independent unit with its own output.
__host__ __device__ inline int wg_slot(int i, int grid, int perm) {
  if (perm == 0) return i;
  if (perm == 1) return grid - 1 - i;
  return (int)(((int64_t)i * perm) % grid);
}

// Device address of the calling device's static scratch of
// vea_attn_fwd_noalloc (VEA_ATTN_NOALLOC_SCRATCH_BYTES), resolved once per
// device; hipSuccess or the runtime's error.
hipError_t attn_noalloc_scratch(void** ptr);

// The permutation VEA_DEBUG_WG_ORDER asks for ("reverse" or "stride"; unset
// or anything else: 0) for a grid of `grid` workgroups.
int wg_order_perm(int grid);

struct SparseParams {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  uint16_t* out;
  float* lse;                // nullable
  int rows, heads, n_kv, k;
  int head_blocks;           // ceil(heads / heads per workgroup)
  float scale;
  // Key-range split of the workgroup units of the last, partial round:
  // units [0, full_units) (unit = row * head_blocks + head block) run whole;
  // each later unit is split into nsplit workgroups over consecutive ranges
  // of its sorted tiles, which write partial (O, m, l) to ws, merged after.
  int full_units;
  int nsplit;                // 1: no split
  float* ws;                 // nullable when nsplit == 1
  // Paged cache: logical position j is physical row
  // page_table[j >> page_shift] << page_shift | (j & (page size - 1)).
  const int32_t* page_table; // nullable: kv holds the logical rows
  int page_shift;
  int n_phys;                // rows of kv (the buffer bound); n_kv when not paged
  // Order check (VEA_DEBUG_WG_ORDER), as in DenseParams.
  int grid;
  int wg_perm;
};

// Split plan of the dense bf16 kernel for one non-causal sequence: `units`
// grid units of which the first `empty` have no rows, `slots` workgroups
// resident at once, `key_tiles` key tiles per unit.
struct DenseSplit {
  int full_units, nsplit, chunks;
};
DenseSplit dense_split_plan(int units, int empty, int slots, int key_tiles);
// Bytes of workspace per split chunk: bm x (d + 2) floats.
size_t dense_chunk_bytes(int bm, int head_dim);
// Workgroups of the dense bf16 kernel resident per CU (0 if unknown).
int dense_bf16_blocks_per_cu(int head_dim);

// Split plan of the sparse kernel for `units` workgroup units of k indices
// each, on a device with `cus` compute units (one workgroup per CU at a time).
struct SparseSplit {
  int full_units, nsplit, chunks;   // chunks = (units - full_units) * nsplit, 0 without a split
};
SparseSplit sparse_split_plan(int units, int k, int cus);
// Bytes of workspace per split chunk: HEADS x (d_v + 2) floats.
size_t sparse_chunk_bytes(int d_v);

struct ProbsParams {
  const void* q;
  const void* k;
  const float* lse;
  float* p;
  int64_t q_stride, k_stride, lse_stride, p_stride;
  int head, kv_head, d;
  int seq_q, len_q, seq_k, len_k, q0, rows, causal;
  float scale;
};

// Launchers (one per kernel family).  Each returns the hipError_t of the launch.
hipError_t launch_attn_fwd_bf16(const DenseParams& p, int head_dim, bool causal, hipStream_t s);
hipError_t launch_attn_fwd_f32(const DenseParams& p, int head_dim, bool causal, hipStream_t s);
hipError_t launch_attn_fwd_fp8(const DenseParams& p, int head_dim, bool causal, hipStream_t s);
hipError_t launch_qkv_rope(const RopeParams& p, hipStream_t s);
hipError_t launch_sparse_mqa(const SparseParams& p, int d_qk, int d_v, hipStream_t s);
hipError_t launch_attn_probs(const ProbsParams& p, bool bf16, hipStream_t s);

struct TopkParams {
  const float* logits;       // [rows, row_stride] fp32
  int64_t row_stride;        // elements
  const int32_t* starts;     // nullable: 0
  const int32_t* lens;       // nullable: n - start
  int32_t* out;              // [rows, k]
  int rows, n, k;
};
constexpr int kTopkMaxN = 4096;   // positions per row the LDS sort holds
hipError_t launch_topk(const TopkParams& p, hipStream_t s);

// Fused QKV projection: out = x w (+ bias), Q and K rotated by the per-token
// (cos, sin) table cs [tokens, d/2, 2] (nullable: no rotation).
struct ProjParams {
  const uint16_t* x;         // bf16 [tokens, x_stride]
  const uint16_t* w;         // bf16 [hidden, w_stride], columns [Q | K | V]
  const uint16_t* bias;      // bf16 [n_feat] or null
  const float* cs;           // [tokens, d/2, 2] or null
  uint16_t* q;               // bf16 [tokens, hq, d]
  uint16_t* k;               // bf16 [tokens, hkv, d]
  uint16_t* v;               // bf16 [tokens, hkv, d]
  int64_t x_stride, w_stride;   // elements
  int tokens, hidden, hq, hkv, d;
  int n_feat;                // (hq + 2 hkv) d
  int ftiles;                // ceil(n_feat / kProjTileF)
  int rot_span;              // 0: adjacent pairs; d or d/2: rotate-half pairs within spans of that width
};
constexpr int kProjTileF = 256;   // features per workgroup tile
constexpr int kProjTileT = 256;   // tokens per workgroup tile
constexpr int kProjStepK = 32;    // hidden is a multiple of this
hipError_t launch_qkv_proj(const ProjParams& p, hipStream_t s);

struct RopeTableParams {
  const int32_t* pos;        // [tokens] or [tokens, 2]
  float* out;                // [tokens, d/2, 2]
  int tokens, d, pos_dims;
  double theta;
};
hipError_t launch_rope_cos_sin(const RopeTableParams& p, hipStream_t s);

// Block quantisation to OCP FP8 E4M3: granularity 0 one scale per (token,
// head) [tokens, heads]; 1 per head [heads]; 2 per (head, channel) [heads, d].
struct QuantParams {
  const uint16_t* x;         // bf16 [tokens, x_stride], heads x d per token
  int64_t x_stride;          // elements
  uint8_t* out;              // e4m3 [tokens, heads, d], contiguous
  float* scales;
  int tokens, heads, d, granularity;
};
hipError_t launch_quant_fp8(const QuantParams& p, hipStream_t s);

// Tile shape of the dense bf16/f32 kernels (query rows per workgroup); the
// host uses it to size the launch.
constexpr int kDenseBM = 128;
// The head_dim 64 non-causal bf16 kernel (packed or paged) covers 256 rows.
constexpr int kD64BM = 256;
// Query rows per tile of a bf16/f32 (non-decode) launch of these parameters.
inline int dense_tile_rows(int dtype_bf16, int head_dim, int causal) {
  return (dtype_bf16 && head_dim == 64 && !causal) ? kD64BM : kDenseBM;
}
constexpr int kSparseHeadsPerWG = 128;

}  // namespace vea
