/*
 * vea.h — C ABI of the MI355X (gfx950) tiled-attention forward library.
 *
 * Operations (page titles used in the citations below):
 *   [3090]   「DeepSeek V4.1 上 4×RTX 3090：视觉链路的两个坑和修复」
 *   [MI250]  「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈性能」
 *   [SGLang] 「从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash - Prefill」
 *   [V32]    「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *     The library allocates nothing and keeps no state between calls; a call
 *     that can use scratch memory takes it as a caller workspace.
 *   - Strides are in ELEMENTS.  Within a token, heads are contiguous and each
 *     head holds head_dim contiguous elements.
 *   - 16-byte vector loads are used: every tensor pointer must be 16-byte
 *     aligned and every token stride a multiple of 16 bytes.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call is asynchronous on that stream; nothing synchronises the host
 *     unless the environment variable VEA_CHECK=1 is set.
 *   - Return value: VEA_OK (0) or a negative vea_status.  Arguments are
 *     validated before anything is launched; on an error nothing runs.  A
 *     launch failure is reported as VEA_EHIP and never swallowed.  A fault
 *     inside a kernel surfaces at the caller's next synchronisation (an
 *     asynchronous illegal access is reported by the NEXT GPU call, as the
 *     cuBLAS "status 13" of [3090] section 三 shows); VEA_CHECK=1 synchronises
 *     after every call and additionally checks device-side index data on the
 *     host (cu_seqlens monotone and consistent with the totals, top-k indices
 *     below n_kv), returning VEA_ERANGE on a violation.
 *   - Results are bitwise identical from run to run: no kernel uses global
 *     atomics, and every output element has exactly one writer.
 */
#ifndef VEA_H
#define VEA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vea_status {
  VEA_OK = 0,
  VEA_EINVAL = -1,       /* null pointer, non-finite scale/theta, misaligned pointer or stride */
  VEA_EDTYPE = -2,       /* dtype not supported by this call */
  VEA_ESHAPE = -3,       /* inconsistent sizes (negative counts, Hq % Hkv != 0, short stride) */
  VEA_EUNSUPPORTED = -4, /* valid request outside the compiled kernel set (e.g. head_dim) */
  VEA_ERANGE = -5,       /* VEA_CHECK only: bad cu_seqlens or top-k index found on the host */
  VEA_EWORKSPACE = -6,   /* caller workspace smaller than the call needs, or misaligned */
  VEA_EHIP = -7,         /* the HIP runtime reported an error (launch or VEA_CHECK sync) */
  VEA_ESCRATCH = -8      /* vea_attn_fwd_noalloc: the call needs more than the static scratch */
} vea_status;

typedef enum vea_dtype { VEA_F32 = 0, VEA_BF16 = 1 } vea_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* vea_status_str(int status);

/* Library version string, e.g. "vea 0.1.0 gfx950". */
const char* vea_version(void);

/*
 * vea_attn_fwd — blockwise scaled-dot-product attention forward over a packed
 * variable-length batch.
 *
 * Computes, for every sequence b, query head h and query row i of b,
 *     o_i = softmax_j( scale * q_i . k_j  over allowed j ) . V,
 *     lse_i = ln sum_{allowed j} exp(scale * q_i . k_j)     (natural log)
 * with the key/value head g = h / (num_heads_q / num_heads_kv).
 * Sources: query pieces with piece-local S/P addressing [3090] section 三;
 * fp32 accumulation of Q K^T and P V and fp32 softmax statistics [MI250]
 * sections 3.1 and 4.1; masked keys excluded (not an additive bias) [MI250]
 * section 3.3; cu_seqlens varlen entry and per-sequence key bound, the
 * softmax_lse output [SGLang] sections 2.2 and 3.2; the online-softmax merge
 * [V32] section 进一步探索 eq. (1)(2).
 *
 *   dtype          VEA_BF16 (head_dim 64 or 128) or VEA_F32 (head_dim 64).
 *   q              [total_q, num_heads_q, head_dim], token stride q_tok_stride.
 *   k, v           [total_k, num_heads_kv, head_dim], token strides k/v_tok_stride
 *                  (v may be a strided view into a fused QKV buffer).
 *   cu_seqlens_q/k device int32 [batch+1], non-decreasing, cu[0] = 0,
 *                  cu_q[batch] = total_q, cu_k[batch] = total_k.  Values are
 *                  clamped to [0, total] inside the kernels, so malformed
 *                  offsets cannot cause out-of-bounds accesses.
 *   max_seqlen_q   >= every query length (sizes the launch; a shorter value
 *                  leaves the rows beyond it unwritten).  max_seqlen_k is
 *                  accepted for symmetry and checked under VEA_CHECK.
 *   causal         0: every key of the sequence is allowed.  1: bottom-right
 *                  aligned causal mask: row i (0-based in its sequence) sees
 *                  keys j <= i + (L_k - L_q).  A row that sees no key gets
 *                  o = 0 and lse = -inf.
 *   scale          finite float (any sign, 0 allowed).
 *   piece_rows     query rows per piece (qb); 0 = one piece per sequence.
 *                  Pieces are [p*qb, (p+1)*qb) within each sequence; no tile
 *                  straddles a piece.  Without a workspace the result is
 *                  bitwise independent of qb; with one, qb changes which rows
 *                  are split (below) and so their rounding.
 *   out            [total_q, num_heads_q, head_dim] of dtype, stride out_tok_stride.
 *   lse            float [num_heads_q, total_q] or NULL (not written).
 *   workspace      NULL (workspace_bytes ignored), or device memory of at
 *                  least vea_attn_fwd_workspace_size bytes for the same sizes
 *                  on the current device, 16-byte aligned; else
 *                  VEA_EWORKSPACE.  Contents need no initialisation and are
 *                  garbage afterwards.  It is used for bf16, batch 1,
 *                  non-causal calls (one image): the query tiles of the last,
 *                  partial round of workgroups over the device are split into
 *                  key ranges that run on otherwise idle CUs and are merged in
 *                  range order with the same merge.  The rounding of those
 *                  rows then depends on the sizes and the CU count; without a
 *                  workspace a row's bits depend only on its sequence.  Both
 *                  are deterministic.  Calls that share a workspace must be
 *                  ordered (same stream).
 */
int vea_attn_fwd(int dtype,
                 const void* q, int64_t q_tok_stride,
                 const void* k, int64_t k_tok_stride,
                 const void* v, int64_t v_tok_stride,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                 int batch, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                 int num_heads_q, int num_heads_kv, int head_dim,
                 int causal, float scale, int piece_rows,
                 void* out, int64_t out_tok_stride, float* lse,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * vea_attn_fwd_paged — vea_attn_fwd (bf16) with K and V in paged caches.
 * Sources: a paged KV cache of fixed-size pages [SGLang] section 2.2; KV rows
 * fetched through a page table [V32] section 实验方法和结果.
 *
 *   k_cache, v_cache  bf16 [num_pages * page_size, num_heads_kv, head_dim],
 *                     token strides k/v_tok_stride.
 *   block_table       device int32 [batch, max_pages_per_seq]: key position j
 *                     of sequence b (0 <= j < its key length, from
 *                     cu_seqlens_k) is token row
 *                     block_table[b][j / page_size] * page_size + j % page_size
 *                     of the caches.  Used entries must lie in [0, num_pages)
 *                     (VEA_ERANGE under VEA_CHECK).
 *   page_size         a power of two, 64 .. 65536 (a 64-key tile never spans
 *                     two pages).  max_pages_per_seq >= ceil(max_seqlen_k /
 *                     page_size).
 * Every other argument as vea_attn_fwd (the same workspace size); total_k is
 * the sum of the key lengths.  The result is bitwise that of vea_attn_fwd on
 * the same logical K/V, wherever the pages are.
 */
int vea_attn_fwd_paged(const void* q, int64_t q_tok_stride,
                       const void* k_cache, int64_t k_tok_stride,
                       const void* v_cache, int64_t v_tok_stride,
                       const int32_t* block_table, int max_pages_per_seq, int page_size, int num_pages,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int batch, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                       int num_heads_q, int num_heads_kv, int head_dim,
                       int causal, float scale, int piece_rows,
                       void* out, int64_t out_tok_stride, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * vea_attn_fwd_noalloc — vea_attn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and the same kernels, with the
 * split of the last round of workgroups using a static scratch array inside
 * the library instead of a caller workspace.  Nothing is allocated by the
 * call (no hipMalloc, hipFree or allocating library routine); the caller
 * passes inputs and outputs as for vea_attn_fwd.
 *
 *   Arguments    as vea_attn_fwd, without workspace / workspace_bytes.
 *   Scratch      VEA_ATTN_NOALLOC_SCRATCH_BYTES (36 MiB) of device memory per
 *                GPU the library runs on, held until the process ends.  It
 *                holds partial results of split rows; nothing in it needs to
 *                start at zero.  A call whose split needs more than that
 *                (vea_attn_fwd_workspace_size reports more; not reachable on
 *                a 256-CU MI355X, where every shape needs at most 34.1 MB)
 *                returns VEA_ESCRATCH and launches nothing.
 *   Result       bitwise that of vea_attn_fwd with a workspace of
 *                vea_attn_fwd_workspace_size bytes (the same split plan).
 *   Concurrency  every call on one GPU shares that GPU's scratch and leaves
 *                its last contents there: calls that overlap on one GPU
 *                (different streams, or several host threads) race and must
 *                be ordered by the caller, e.g. on one stream.
 */
#define VEA_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)36 << 20)
int vea_attn_fwd_noalloc(int dtype,
                         const void* q, int64_t q_tok_stride,
                         const void* k, int64_t k_tok_stride,
                         const void* v, int64_t v_tok_stride,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int batch, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                         int num_heads_q, int num_heads_kv, int head_dim,
                         int causal, float scale, int piece_rows,
                         void* out, int64_t out_tok_stride, float* lse, void* stream);

/*
 * vea_attn_fwd_workspace_size — bytes of workspace vea_attn_fwd uses for these
 * sizes on the current HIP device (0 when it splits nothing).  Validates the
 * shape arguments like vea_attn_fwd; VEA_EHIP if the device cannot be queried.
 */
int vea_attn_fwd_workspace_size(int dtype, int batch, int total_q, int total_k, int max_seqlen_q,
                                int max_seqlen_k, int num_heads_q, int num_heads_kv, int head_dim,
                                int causal, int piece_rows, size_t* bytes);

/*
 * vea_attn_decode — bf16 attention of one new query token per sequence over
 * that sequence's cached keys and values (the decode step: every cached key
 * is visible), packed or paged.
 * Sources: the scaled dot-product attention and its lse as vea_attn_fwd; a
 * paged KV cache of fixed-size pages [SGLang] section 2.2; KV rows fetched
 * through a page table [V32] section 实验方法和结果; the blockwise merge of
 * partial results over key ranges [V32] eq. (1)(2).
 *
 *   q             bf16 [batch, num_heads_q, head_dim], sequence stride
 *                 q_seq_stride elements (>= num_heads_q * head_dim).
 *   k, v          block_table NULL: bf16 [total_k, num_heads_kv, head_dim]
 *                 packed by cu_seqlens_k.  Otherwise caches as in
 *                 vea_attn_fwd_paged (page_size a power of two 64 .. 65536,
 *                 block_table [batch, max_pages_per_seq], num_pages pages).
 *   cu_seqlens_k  device int32 [batch + 1]: sequence b has keys
 *                 [cu[b], cu[b+1]) (positions 0 .. len - 1 in the cache).
 *                 A sequence with no keys gets zeros and lse -inf.
 *   total_k       packed: rows of k/v (= cu[batch]); paged: the sum of the key
 *                 lengths (= cu[batch]).  Key offsets are clamped to total_k,
 *                 so a total_k above the rows k/v hold reads past them: it
 *                 is a contract violation (VEA_ERANGE under VEA_CHECK when
 *                 cu[batch] != total_k).  max_seqlen_k bounds every key length.
 *   num_heads_q / num_heads_kv   a divisor; query head h reads key/value head
 *                 h / (num_heads_q / num_heads_kv); that ratio <= 128.
 *   head_dim      64 or 128.
 *   out           bf16 [batch, num_heads_q, head_dim], stride out_seq_stride.
 *   lse           nullable; float [num_heads_q, batch], natural log.
 *   workspace     nullable; with at least vea_attn_decode_workspace_size bytes
 *                 each (sequence, key/value head) is cut into up to 8 key
 *                 ranges whose partial results are merged in range order (the
 *                 result does not depend on the timing of the ranges; it may
 *                 differ in the last bits from a call without workspace).
 * One workgroup handles all query heads of one key/value head of one sequence,
 * so every cached key is read once per (sequence, key/value head).
 * Errors as vea_attn_fwd; VEA_EUNSUPPORTED for head_dim or a head ratio out of
 * range.  Nothing is written on error.  Asynchronous on stream.
 */
int vea_attn_decode(const void* q, int64_t q_seq_stride,
                    const void* k, int64_t k_tok_stride,
                    const void* v, int64_t v_tok_stride,
                    const int32_t* block_table, int max_pages_per_seq, int page_size, int num_pages,
                    const int32_t* cu_seqlens_k, int batch, int total_k, int max_seqlen_k,
                    int num_heads_q, int num_heads_kv, int head_dim, float scale,
                    void* out, int64_t out_seq_stride, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * vea_attn_decode_workspace_size — bytes of workspace vea_attn_decode uses for
 * these sizes on the current HIP device (0: it splits nothing).
 */
int vea_attn_decode_workspace_size(int batch, int max_seqlen_k, int num_heads_q, int num_heads_kv,
                                   int head_dim, size_t* bytes);

/*
 * vea_qkv_rope — split a fused QKV projection output and apply rotary position
 * embedding to its Q and K heads (V is left in place for vea_attn_fwd to read
 * through a strided pointer).
 * Sources: the vision encoder's qkv_rope step [3090] section 二; the fused
 * [T, 3*hidden] projection output [SGLang] section 3.1; trigonometry in at
 * least fp32 [MI250] section 4.1 (here: angle and sin/cos in fp64, rotation in
 * fp32, bf16 round-to-nearest-even output).
 *
 * Rotation: pair i of a rotated span of width d_r, (x[2i], x[2i+1]), turns by
 * phi = pos * theta^(-2i/d_r).  pos_dims = 1: one span over the whole head,
 * pos = positions[t].  pos_dims = 2 (patch grid): dims [0, d/2) turn with
 * positions[t][0] (grid row), dims [d/2, d) with positions[t][1] (grid
 * column), each a span of width d/2.
 *
 *   x_qkv       bf16 [num_tokens, (Hq + 2 Hkv) * head_dim] with columns
 *               [Q heads | K heads | V heads], token stride x_tok_stride.
 *   positions   device int32 [num_tokens] or [num_tokens, 2].
 *   head_dim    even (pos_dims 1) or a multiple of 4 (pos_dims 2), and a
 *               multiple of 8; at most 256.
 *   theta       finite, > 0.
 *   rotate_half 0: the pairs above; 1: rotate-half pairing, pair i of a span
 *               of width d_r joins features i and i + d_r/2 (same angles);
 *               head_dim a multiple of 32.
 *   q, k        bf16 outputs [num_tokens, Hq, head_dim] and
 *               [num_tokens, Hkv, head_dim], contiguous; must not overlap x_qkv.
 */
int vea_qkv_rope(const void* x_qkv, int64_t x_tok_stride,
                 const int32_t* positions, int pos_dims,
                 int num_tokens, int num_heads_q, int num_heads_kv, int head_dim, float theta,
                 int rotate_half, void* q, void* k, void* stream);

/*
 * vea_sparse_mqa_fwd — multi-query attention of each query row over its own
 * top-k set of latent KV rows (all heads of a row share the gathered rows).
 * Sources: sparse attention taking Q, the KV cache and an index [V32] section
 * 实验方法和结果; the result depends on the index set, the order only changes
 * rounding [V32] sections 结论 and 进一步探索 eq. (1)(2).  Each row's indices
 * are sorted ascending on the device before use, so the output is bitwise
 * invariant to the order of the indices within a row.
 *
 *   q          bf16 [num_rows, num_heads, d_qk], contiguous.
 *   kv_latent  bf16 [n_kv, d_qk], contiguous; V is columns [0, d_v).
 *   topk_idx   device int32 [num_rows, k].  Entries < 0 are padding and are
 *              skipped; entries >= n_kv are skipped as well (and reported as
 *              VEA_ERANGE under VEA_CHECK).  Repeated entries count with their
 *              multiplicity.  A row with no valid entry gets o = 0, lse = -inf.
 *   d_qk, d_v  compiled for d_qk = 576, d_v = 512.
 *   k          1 .. 4096.
 *   out        bf16 [num_rows, num_heads, d_v]; lse float [num_heads, num_rows]
 *              or NULL.
 *   workspace  NULL (workspace_bytes ignored), or device memory of at least
 *              vea_sparse_mqa_workspace_size bytes for the same sizes on the
 *              current device, 16-byte aligned; else VEA_EWORKSPACE.  Its
 *              contents need no initialisation and are garbage afterwards.
 *              With a workspace, the (row, 128-head block) units of the last,
 *              partial round of workgroups over the device's CUs are split
 *              into key ranges of the sorted indices that run on otherwise
 *              idle CUs and are merged in range order (the same merge).  The
 *              rounding of those rows then depends on num_rows, num_heads and
 *              the CU count; without a workspace every row is computed alone,
 *              so a row's bits do not depend on the rest of the batch.  Both
 *              modes are deterministic and order-invariant.  Calls that share
 *              a workspace must be ordered (same stream).
 */
int vea_sparse_mqa_fwd(const void* q, const void* kv_latent, const int32_t* topk_idx,
                       int num_rows, int num_heads, int n_kv, int d_qk, int d_v, int k,
                       float scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * vea_sparse_mqa_paged_fwd — vea_sparse_mqa_fwd over a paged latent cache.
 * Sources: the sparse attention fetches its KV rows through a page table
 * [V32] section 实验方法和结果; the prefill path keeps a paged KV cache
 * [SGLang] section 2.2.
 *
 *   kv_cache    bf16 [num_pages * page_size, d_qk]: num_pages physical pages
 *               of page_size rows, contiguous.
 *   page_table  device int32 [ceil(n_kv / page_size)]: logical position j
 *               (the values in topk_idx, 0 <= j < n_kv) is row
 *               page_table[j / page_size] * page_size + j % page_size of
 *               kv_cache.  Entries must lie in [0, num_pages) (VEA_ERANGE
 *               under VEA_CHECK; otherwise a row past the cache reads as 0).
 *   page_size   a power of two, 1 .. 65536.
 * Every other argument as vea_sparse_mqa_fwd (the same workspace size).  The
 * indices are put in canonical order by their LOGICAL position before the
 * table is applied, so the output is bitwise independent of both the index
 * order and the placement of the pages.
 */
int vea_sparse_mqa_paged_fwd(const void* q, const void* kv_cache, const int32_t* page_table, int page_size,
                             int num_pages, const int32_t* topk_idx, int num_rows, int num_heads, int n_kv,
                             int d_qk, int d_v, int k, float scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * vea_sparse_mqa_workspace_size — bytes of workspace vea_sparse_mqa_fwd uses
 * for these sizes on the current HIP device (0 when no split pays off, e.g.
 * when the units fill whole rounds of the CUs).  Validates like
 * vea_sparse_mqa_fwd; VEA_EHIP if the device cannot be queried.
 */
int vea_sparse_mqa_workspace_size(int num_rows, int num_heads, int d_qk, int d_v, int k, size_t* bytes);

/*
 * vea_topk_indices — deterministic top-k selection of the sparse indexer: for
 * each row, the positions of its k highest logits in rank order.
 * Sources: the indexer keeps the 2048 best positions of each [2590] row of
 * logits, and an unstable top-k let equal scores at the edge of the selection
 * fall either way, fixed by a stable sort [V32] sections 修改topk结果，输出后排序
 * and 用 torch.sort 替换 topk，输出对比; ties are resolved by id [MI250]
 * section 4.2.
 *
 * Rank order within a row's span: value descending; equal values by
 * ascending position; NaN after every number (NaNs by position); -0.0 ties
 * with +0.0.  The result is unique and independent of timing.
 *
 *   logits      fp32 [num_rows, row_stride] (4-byte aligned), columns [0, n).
 *   row_starts  device int32 [num_rows] or NULL (0); row_lens device int32
 *               [num_rows] or NULL (n - start).  Row r considers columns
 *               [start, start + len); spans outside [0, n) are clamped
 *               (VEA_ERANGE under VEA_CHECK).
 *   n           1 .. 4096 (VEA_EUNSUPPORTED above).
 *   k           >= 1.  out int32 [num_rows, k]: absolute column positions
 *               of ranks 0 .. min(k, len) - 1, then -1 (the padding value
 *               vea_sparse_mqa_fwd skips).
 */
int vea_topk_indices(const float* logits, int64_t row_stride, const int32_t* row_starts,
                     const int32_t* row_lens, int num_rows, int n, int k, int32_t* out,
                     void* stream);

/*
 * vea_quantize_fp8 — block quantisation of a bf16 tensor to OCP FP8 E4M3.
 * Sources: FP8 for matrix products, statistics kept in fp32 [MI250] section
 * 4.1; block-wise quantisation [MI250] section 5.3.
 *
 * x bf16 [num_tokens, num_heads, head_dim] (token stride x_tok_stride) is cut
 * into blocks: granularity 0 one per (token, head), scales float
 * [num_tokens, num_heads]; 1 one per head, scales [num_heads]; 2 one per
 * (head, channel), scales [num_heads, head_dim].  Per block:
 *     scale = fp32(amax / 448)   (1 when amax < 2^-64), inv = fp32(1 / scale)
 *     code  = nearest-even E4M3 of clamp(fp32(x * inv), -448, 448)
 * and x ~ code * scale.  out: uint8 codes [num_tokens, num_heads, head_dim],
 * contiguous.  head_dim 64 or 128.  Granularities 1 and 2 run two kernels (the
 * block maxima over all tokens, then the codes); there are no atomics and the
 * result is bitwise reproducible.  Non-finite inputs are not supported.
 */
int vea_quantize_fp8(const void* x, int64_t x_tok_stride, int num_tokens, int num_heads, int head_dim,
                     int granularity, void* out, float* scales, void* stream);

/*
 * vea_attn_fwd_fp8 — vea_attn_fwd with q, k and v as E4M3 codes
 * (vea_quantize_fp8): the attention of the dequantised
 *     q[t][h][:] * q_scale[t][h],  k[t][g][:] * k_scale[g],
 *     v[t][g][c] * v_scale[g][c]
 * (granularities 0, 1 and 2 of vea_quantize_fp8), written in bf16.
 * Sources: FP8 for the Q K^T and P V products with fp32 softmax statistics
 * and accumulation [MI250] section 4.1, block scales [MI250] section 5.3,
 * FP8 in the prefill attention kernel [SGLang] section 3.2.
 * The products run on the FP8 MFMA with fp32 accumulation; P is rounded to
 * E4M3 (nearest even) for the P V product, while l and lse use the fp32 P.
 * Every other argument as vea_attn_fwd (bf16 rules: head_dim 64 or 128;
 * strides of q, k, v in bytes = elements, multiples of 16; out bf16).  No
 * workspace, no paging.  k_tok_stride, v_tok_stride <= 2^24.
 */
int vea_attn_fwd_fp8(const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride, const void* v,
                     int64_t v_tok_stride, const float* q_scale, const float* k_scale, const float* v_scale,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int total_q, int total_k,
                     int max_seqlen_q, int max_seqlen_k, int num_heads_q, int num_heads_kv, int head_dim, int causal,
                     float scale, int piece_rows, void* out, int64_t out_tok_stride, float* lse, void* stream);

/*
 * vea_rope_cos_sin — per-token rotation table for vea_qkv_proj_rope: entry
 * [t][e] = (cos phi, sin phi) of pair e (features 2e, 2e + 1 of a head) of
 * token t, with the angle vea_qkv_rope uses for that pair (pos_dims 1: phi =
 * positions[t] * theta^(-2e/d); pos_dims 2: pairs e < d/4 turn with
 * positions[t][0] by theta^(-2e/(d/2)), the others with positions[t][1] by
 * theta^(-2(e - d/4)/(d/2))).  Angle, sine and cosine in fp64, stored as
 * fp32 (trigonometry in at least fp32 [MI250] section 4.1).  The positions of
 * an encoder's tokens are the same in every layer, so one table serves all
 * of its projections.
 *
 *   positions   device int32 [num_tokens] or [num_tokens, 2].
 *   head_dim    even (pos_dims 1) or a multiple of 4 (pos_dims 2), <= 256.
 *   theta       finite, > 0.
 *   cos_sin     float [num_tokens, head_dim / 2, 2], 8-byte aligned.
 */
int vea_rope_cos_sin(const int32_t* positions, int pos_dims, int num_tokens, int head_dim, float theta,
                     float* cos_sin, void* stream);

/*
 * vea_qkv_proj_rope — the fused QKV projection with the rotary embedding
 * applied in its epilogue: y = x w (+ bias), then q = rotate(y[:, Q]),
 * k = rotate(y[:, K]), v = y[:, V].
 * Sources: one fused weight holds Wq | Wk | Wv ([hidden, 3 * hidden] in
 * [SGLang] section 3.1); fusing the memory-bound work next to a projection
 * into it [MI250] section 5.2 (fourth point); the rotation as vea_qkv_rope.
 * The product runs on bf16 MFMA with fp32 accumulation; bias and rotation
 * are applied to the fp32 values, which are rounded to bf16 (nearest even)
 * once, when stored.
 *
 *   x           bf16 [num_tokens, x_tok_stride], columns [0, hidden).
 *   w           bf16 [hidden, w_row_stride], columns [Q heads | K heads |
 *               V heads] = (Hq + 2 Hkv) * head_dim, each head contiguous.
 *   bias        bf16 [(Hq + 2 Hkv) * head_dim] or NULL (no bias).
 *   cos_sin     the table of vea_rope_cos_sin for these tokens and head_dim,
 *               or NULL: no rotation (a plain projection and split).
 *   hidden      a multiple of 32.  head_dim: a multiple of 32, <= 256.
 *   rotate_half_span  0: adjacent pairs (2i, 2i + 1).  head_dim (1D tables)
 *               or head_dim / 2 (2D tables): rotate-half pairs (i, i + span/2)
 *               within each span, table entry e of pair i as vea_qkv_rope
 *               numbers it; head_dim 64 or 128.
 *   q, k, v     bf16 outputs [num_tokens, Hq, head_dim], [num_tokens, Hkv,
 *               head_dim] (both) contiguous; they must not overlap the inputs.
 * All pointers 16-byte aligned, strides multiples of 8 elements
 * (VEA_EINVAL).  num_tokens * x_tok_stride and hidden * w_row_stride must stay
 * below 2^30 elements (VEA_EUNSUPPORTED): buffer ranges are 32-bit.
 */
int vea_qkv_proj_rope(const void* x, int64_t x_tok_stride, const void* w, int64_t w_row_stride, const void* bias,
                      const float* cos_sin, int num_tokens, int hidden, int num_heads_q, int num_heads_kv,
                      int head_dim, int rotate_half_span, void* q, void* k, void* v, void* stream);

/*
 * vea_attn_probs_piece — debug export (not on the timed path) of the
 * probability matrix of one query piece of one head:
 *     P[r][j] = exp(scale * q_{q0+r} . k_j - lse_{q0+r}),  r < rows, j < len_k,
 * zero where the causal mask excludes the key.  The piece is written from the
 * START of p_out (row r at p_out + r * p_row_stride): the piece-local
 * addressing fix of [3090] section 三, and a buffer of rows x len_k floats is
 * always enough.  Row sums of P are 1 up to rounding; [3090] section 四 prints
 * 0.9997 .. 1.0003 for 1462 rows.
 *
 *   lse           the float [num_heads_q, lse_row_stride] output of vea_attn_fwd.
 *   seq_begin_q   global row of the sequence's first query; len_q its length.
 *   seq_begin_k   global row of the sequence's first key; len_k its length.
 *   q0, rows      the piece: local rows [q0, q0 + rows) of the sequence.
 */
int vea_attn_probs_piece(int dtype,
                         const void* q, int64_t q_tok_stride,
                         const void* k, int64_t k_tok_stride,
                         const float* lse, int64_t lse_row_stride,
                         int head, int num_heads_q, int num_heads_kv, int head_dim,
                         int seq_begin_q, int len_q, int seq_begin_k, int len_k,
                         int q0, int rows, int causal, float scale,
                         float* p_out, int64_t p_row_stride, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VEA_H */
