// C ABI of the tiled-attention library: argument validation, launch shape,
// dispatch to the kernel instances, and error reporting.  Declared in
// include/vea.h.
//
// Validation runs entirely on the host and before any HIP call, so a bad
// argument returns its status without touching the GPU.  Launch errors are
// read back with hipGetLastError and returned as VEA_EHIP; they are never
// swallowed (a swallowed error misled the debugging in
// 「DeepSeek V4.1 上 4×RTX 3090：视觉链路的两个坑和修复」 section 三, "误导报错").
#include "../../include/vea.h"
#include "vea_internal.h"

#include <dlfcn.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

using namespace vea;

namespace {

bool check_enabled() {
  const char* e = getenv("VEA_CHECK");
  return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? VEA_OK : VEA_EHIP; }

// VEA_ROCTX=1: every entry point is a named roctx range, so that a
// rocprofv3 --marker-trace timeline shows the library calls around their
// kernels.  The roctx library is opened on first use; without it (or without
// the variable) the ranges cost one load of a flag.
struct RoctxApi {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const RoctxApi& roctx_api() {
  static RoctxApi api;
  static std::once_flag once;
  std::call_once(once, [] {
    const char* e = getenv("VEA_ROCTX");
    if (e == nullptr || e[0] == '\0' || strcmp(e, "0") == 0) return;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (h == nullptr) h = dlopen("/opt/rocm/lib/librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (h == nullptr) return;
    auto push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    auto pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (push != nullptr && pop != nullptr) {
      api.push = push;
      api.pop = pop;
    }
  });
  return api;
}

class Range {
 public:
  explicit Range(const char* name) : api_(roctx_api()) {
    if (api_.push != nullptr) api_.push(name);
  }
  ~Range() {
    if (api_.pop != nullptr) api_.pop();
  }

 private:
  const RoctxApi& api_;
};

// VEA_CHECK: copy a device int32 array to the host after draining the stream.
int fetch_ints(const int32_t* dev, size_t n, hipStream_t s, std::vector<int32_t>& host) {
  host.resize(n);
  if (n == 0) return VEA_OK;
  if (hipStreamSynchronize(s) != hipSuccess) return VEA_EHIP;
  if (hipMemcpy(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return VEA_EHIP;
  return VEA_OK;
}

int check_cu(const int32_t* cu, int batch, int total, int max_len, hipStream_t s) {
  std::vector<int32_t> h;
  int st = fetch_ints(cu, (size_t)batch + 1, s, h);
  if (st != VEA_OK) return st;
  if (h[0] != 0 || h[batch] != total) return VEA_ERANGE;
  for (int b = 0; b < batch; ++b) {
    const int len = h[b + 1] - h[b];
    if (len < 0 || len > max_len) return VEA_ERANGE;
  }
  return VEA_OK;
}

int gcd_int(int a, int b) {
  while (b != 0) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

int finish(int st, hipStream_t s) {
  if (st != VEA_OK) return st;
  if (check_enabled()) {
    if (hipStreamSynchronize(s) != hipSuccess) return VEA_EHIP;
  }
  return VEA_OK;
}

}  // namespace

namespace vea {

int wg_order_perm(int grid) {
  const char* e = getenv("VEA_DEBUG_WG_ORDER");
  if (e == nullptr || grid < 2) return 0;
  if (strcmp(e, "reverse") == 0) return 1;
  if (strcmp(e, "stride") == 0) {
    if (grid < 4) return 1;
    // a multiplier near 0.618 grid, coprime to grid (a bijection of the slots)
    int a = std::max(2, (int)(grid * 0.618));
    while (gcd_int(a, grid) != 1) a = a + 1 < grid ? a + 1 : 2;
    return a;
  }
  return 0;
}

}  // namespace vea

extern "C" {

const char* vea_status_str(int status) {
  switch (status) {
    case VEA_OK: return "VEA_OK";
    case VEA_EINVAL: return "VEA_EINVAL: invalid argument (null pointer, non-finite scalar or misalignment)";
    case VEA_EDTYPE: return "VEA_EDTYPE: dtype not supported by this call";
    case VEA_ESHAPE: return "VEA_ESHAPE: inconsistent sizes";
    case VEA_EUNSUPPORTED: return "VEA_EUNSUPPORTED: shape outside the compiled kernel set";
    case VEA_ERANGE: return "VEA_ERANGE: index data out of range (VEA_CHECK)";
    case VEA_EWORKSPACE: return "VEA_EWORKSPACE: workspace too small";
    case VEA_EHIP: return "VEA_EHIP: HIP runtime error";
    case VEA_ESCRATCH:
      return "VEA_ESCRATCH: the call needs more scratch than vea_attn_fwd_noalloc's static array (36 MiB)";
    default: return "unknown vea status";
  }
}

const char* vea_version(void) { return "vea 0.1.0 gfx950"; }

namespace {

// Validation of the shape arguments shared by vea_attn_fwd and its workspace
// query.
int dense_shape_status(int dtype, int batch, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                       int num_heads_q, int num_heads_kv, int head_dim, int causal, int piece_rows) {
  if (dtype != VEA_BF16 && dtype != VEA_F32) return VEA_EDTYPE;
  if (batch < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || piece_rows < 0)
    return VEA_ESHAPE;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0) return VEA_ESHAPE;
  if (causal != 0 && causal != 1) return VEA_EINVAL;
  if (dtype == VEA_BF16 && head_dim != 64 && head_dim != 128) return VEA_EUNSUPPORTED;
  if (dtype == VEA_F32 && head_dim != 64) return VEA_EUNSUPPORTED;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return VEA_ESHAPE;
  return VEA_OK;
}

// Launch shape: (sequence, piece, tile, head) units.
int dense_layout(int batch, int max_seqlen_q, int num_heads_q, int piece_rows, int bm, DenseParams& p) {
  p.qb = (piece_rows > 0 && piece_rows < max_seqlen_q) ? piece_rows : max_seqlen_q;
  p.bm = bm;
  p.tiles_per_piece = (p.qb + bm - 1) / bm;
  const int64_t pieces = ((int64_t)max_seqlen_q + p.qb - 1) / p.qb;
  const int64_t tps = pieces * p.tiles_per_piece;
  const int64_t units = (int64_t)batch * tps * num_heads_q;
  if (units * 8 > 0x7fffffff) return VEA_EUNSUPPORTED;
  p.tiles_per_seq = (int)tps;
  p.units = (int)units;
  p.full_units = p.units;
  p.nsplit = 1;
  p.ws = nullptr;
  p.block_table = nullptr;
  p.page_shift = 0;
  p.max_pages = 0;
  p.q_scale = p.k_scale = p.v_scale = nullptr;
  p.dec_group = 0;
  p.ws_rows = bm;
  p.grid = 0;
  p.wg_perm = 0;
  return VEA_OK;
}

// Split of the last round (bf16, one non-causal sequence: there the host
// knows which units are empty without reading cu_seqlens).
int dense_split(int dtype, int batch, int total_q, int total_k, int num_heads_q, int head_dim, int causal,
                const DenseParams& p, DenseSplit& plan) {
  plan = DenseSplit{p.units, 1, 0};
  if (dtype != VEA_BF16 || batch != 1 || causal || total_q == 0) return VEA_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VEA_EHIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return VEA_EHIP;
  const int per_cu = dense_bf16_blocks_per_cu(head_dim);
  int64_t real_tiles = 0;                               // tiles with rows, per head
  for (int64_t r0 = 0; r0 < total_q; r0 += p.qb)
    real_tiles += (std::min<int64_t>(p.qb, total_q - r0) + p.bm - 1) / p.bm;
  const int empty = p.units - (int)(real_tiles * num_heads_q);
  plan = dense_split_plan(p.units, std::max(empty, 0), cus * per_cu, (total_k + 63) / 64);
  return VEA_OK;
}

}  // namespace

int vea_attn_fwd_workspace_size(int dtype, int batch, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                                int num_heads_q, int num_heads_kv, int head_dim, int causal, int piece_rows,
                                size_t* bytes) {
  if (bytes == nullptr) return VEA_EINVAL;
  *bytes = 0;
  int st = dense_shape_status(dtype, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q,
                              num_heads_kv, head_dim, causal, piece_rows);
  if (st != VEA_OK) return st;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return VEA_OK;
  DenseParams p;
  st = dense_layout(batch, max_seqlen_q, num_heads_q, piece_rows, dense_tile_rows(dtype == VEA_BF16, head_dim, causal), p);
  if (st != VEA_OK) return st;
  DenseSplit plan;
  st = dense_split(dtype, batch, total_q, total_k, num_heads_q, head_dim, causal, p, plan);
  if (st != VEA_OK) return st;
  *bytes = (size_t)plan.chunks * dense_chunk_bytes(p.bm, head_dim);
  return VEA_OK;
}

namespace {

int dense_fwd(int dtype, const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride, const void* v,
              int64_t v_tok_stride, const int32_t* block_table, int max_pages, int page_size, int num_pages,
              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int total_q, int total_k,
              int max_seqlen_q, int max_seqlen_k, int num_heads_q, int num_heads_kv, int head_dim, int causal,
              float scale, int piece_rows, void* out, int64_t out_tok_stride, float* lse, void* workspace,
              size_t workspace_bytes, void* stream) {
  // ---- validation (host only)
  int st = dense_shape_status(dtype, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q,
                              num_heads_kv, head_dim, causal, piece_rows);
  if (st != VEA_OK) return st;
  if (!isfinite(scale)) return VEA_EINVAL;
  int shift = 0;
  if (block_table != nullptr) {
    if (dtype != VEA_BF16) return VEA_EUNSUPPORTED;
    if (page_size < 64 || page_size > (1 << 16) || (page_size & (page_size - 1)) || num_pages < 0) return VEA_ESHAPE;
    while ((1 << shift) < page_size) ++shift;
    if (max_pages < (max_seqlen_k + page_size - 1) / page_size) return VEA_ESHAPE;
  }
  if (batch == 0 || total_q == 0) return VEA_OK;                 // nothing to compute
  if (!q || !out || !cu_seqlens_q || !cu_seqlens_k) return VEA_EINVAL;
  const bool has_keys = block_table != nullptr ? num_pages > 0 : total_k > 0;
  if (has_keys && (!k || !v)) return VEA_EINVAL;                  // no keys: k/v are never read
  const int64_t esz = dtype == VEA_BF16 ? 2 : 4;
  const int64_t qrow = (int64_t)num_heads_q * head_dim, krow = (int64_t)num_heads_kv * head_dim;
  if (q_tok_stride < qrow || out_tok_stride < qrow || k_tok_stride < krow || v_tok_stride < krow) return VEA_ESHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VEA_EINVAL;
  if ((q_tok_stride * esz) % 16 || (k_tok_stride * esz) % 16 || (v_tok_stride * esz) % 16 ||
      (out_tok_stride * esz) % 16)
    return VEA_EINVAL;
  if (workspace != nullptr && !aligned16(workspace)) return VEA_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;

  if (check_enabled()) {
    st = check_cu(cu_seqlens_q, batch, total_q, max_seqlen_q, s);
    if (st == VEA_OK) st = check_cu(cu_seqlens_k, batch, total_k, max_seqlen_k, s);
    if (st != VEA_OK) return st;
    if (block_table != nullptr) {
      std::vector<int32_t> cu, bt;
      st = fetch_ints(cu_seqlens_k, (size_t)batch + 1, s, cu);
      if (st == VEA_OK) st = fetch_ints(block_table, (size_t)batch * max_pages, s, bt);
      if (st != VEA_OK) return st;
      for (int b = 0; b < batch; ++b)
        for (int pg = 0; pg < (cu[b + 1] - cu[b] + page_size - 1) / page_size; ++pg) {
          const int32_t x = bt[(size_t)b * max_pages + pg];
          if (x < 0 || x >= num_pages) return VEA_ERANGE;
        }
    }
  }
  if (max_seqlen_q == 0) return finish(VEA_OK, s);

  DenseParams p;
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.q_stride = q_tok_stride; p.k_stride = k_tok_stride; p.v_stride = v_tok_stride; p.o_stride = out_tok_stride;
  p.batch = batch; p.total_q = total_q; p.total_k = total_k;
  p.hq = num_heads_q; p.hkv = num_heads_kv; p.group = num_heads_q / num_heads_kv;
  st = dense_layout(batch, max_seqlen_q, num_heads_q, piece_rows, dense_tile_rows(dtype == VEA_BF16, head_dim, causal),
                    p);
  if (st != VEA_OK) return st;
  p.xcd_map = (num_heads_kv % 8 == 0) ? 1 : 0;
  p.scale = scale;
  p.block_table = block_table;
  p.page_shift = shift;
  p.max_pages = max_pages;
  if (workspace != nullptr) {
    DenseSplit plan;
    st = dense_split(dtype, batch, total_q, total_k, num_heads_q, head_dim, causal, p, plan);
    if (st != VEA_OK) return st;
    if (plan.nsplit > 1) {
      if (workspace_bytes < (size_t)plan.chunks * dense_chunk_bytes(p.bm, head_dim)) return VEA_EWORKSPACE;
      p.full_units = plan.full_units;
      p.nsplit = plan.nsplit;
      p.ws = (float*)workspace;
    }
  }

  hipError_t e = dtype == VEA_BF16 ? launch_attn_fwd_bf16(p, head_dim, causal != 0, s)
                                   : launch_attn_fwd_f32(p, head_dim, causal != 0, s);
  return finish(hip_status(e), s);
}

}  // namespace

int vea_attn_fwd(int dtype, const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                 const void* v, int64_t v_tok_stride, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                 int batch, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int num_heads_q,
                 int num_heads_kv, int head_dim, int causal, float scale, int piece_rows, void* out,
                 int64_t out_tok_stride, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Range range("vea_attn_fwd");
  return dense_fwd(dtype, q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, nullptr, 0, 0, 0, cu_seqlens_q,
                   cu_seqlens_k, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                   head_dim, causal, scale, piece_rows, out, out_tok_stride, lse, workspace, workspace_bytes, stream);
}

int vea_attn_fwd_noalloc(int dtype, const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                         const void* v, int64_t v_tok_stride, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int batch, int total_q, int total_k, int max_seqlen_q,
                         int max_seqlen_k, int num_heads_q, int num_heads_kv, int head_dim, int causal, float scale,
                         int piece_rows, void* out, int64_t out_tok_stride, float* lse, void* stream) {
  Range range("vea_attn_fwd_noalloc");
  // the split plan of vea_attn_fwd for these sizes, served from the static scratch
  size_t need = 0;
  int st = vea_attn_fwd_workspace_size(dtype, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q,
                                       num_heads_kv, head_dim, causal, piece_rows, &need);
  if (st != VEA_OK) return st;
  if (need > VEA_ATTN_NOALLOC_SCRATCH_BYTES) return VEA_ESCRATCH;
  void* ws = nullptr;
  if (need > 0 && attn_noalloc_scratch(&ws) != hipSuccess) return VEA_EHIP;
  return dense_fwd(dtype, q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, nullptr, 0, 0, 0, cu_seqlens_q,
                   cu_seqlens_k, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                   head_dim, causal, scale, piece_rows, out, out_tok_stride, lse, ws, need, stream);
}

int vea_attn_fwd_paged(const void* q, int64_t q_tok_stride, const void* k_cache, int64_t k_tok_stride,
                       const void* v_cache, int64_t v_tok_stride, const int32_t* block_table, int max_pages_per_seq,
                       int page_size, int num_pages, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int batch, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int num_heads_q,
                       int num_heads_kv, int head_dim, int causal, float scale, int piece_rows, void* out,
                       int64_t out_tok_stride, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Range range("vea_attn_fwd_paged");
  if (block_table == nullptr && batch > 0 && total_q > 0) return VEA_EINVAL;
  return dense_fwd(VEA_BF16, q, q_tok_stride, k_cache, k_tok_stride, v_cache, v_tok_stride, block_table,
                   max_pages_per_seq, page_size, num_pages, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                   max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, causal, scale, piece_rows, out,
                   out_tok_stride, lse, workspace, workspace_bytes, stream);
}

namespace {

// Decode split: every (sequence, key/value head) unit is cut into key ranges
// so that about four rounds of workgroups fill the device (at most 8 ranges,
// at most one per key tile of the longest cache): the ranges of long caches
// are then short enough to even out unequal cache lengths.
int decode_split(int units, int max_seqlen_k, int head_dim, int* nsplit) {
  *nsplit = 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VEA_EHIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return VEA_EHIP;
  const int slots = cus * dense_bf16_blocks_per_cu(head_dim);
  if (slots > 0 && units > 0 && units < 4 * slots) *nsplit = std::min(8, (4 * slots + units - 1) / units);
  *nsplit = std::max(1, std::min(*nsplit, (max_seqlen_k + 63) / 64));
  return VEA_OK;
}

// Bytes of one decode split chunk: the group's rows (rounded up to 4, which
// keeps every chunk 16-byte aligned) x (d + 2) floats.
size_t decode_chunk_bytes(int group, int head_dim) {
  return (size_t)((group + 3) & ~3) * (head_dim + 2) * sizeof(float);
}

int decode_shape_status(int batch, int total_k, int max_seqlen_k, int num_heads_q, int num_heads_kv, int head_dim) {
  if (batch < 0 || total_k < 0 || max_seqlen_k < 0) return VEA_ESHAPE;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0) return VEA_ESHAPE;
  if (head_dim != 64 && head_dim != 128) return VEA_EUNSUPPORTED;
  if (num_heads_q / num_heads_kv > kDenseBM) return VEA_EUNSUPPORTED;   // a group's heads fill one tile
  if ((int64_t)batch * num_heads_kv * 8 * 8 > 0x7fffffff) return VEA_EUNSUPPORTED;
  return VEA_OK;
}

}  // namespace

int vea_attn_decode_workspace_size(int batch, int max_seqlen_k, int num_heads_q, int num_heads_kv, int head_dim,
                                   size_t* bytes) {
  if (bytes == nullptr) return VEA_EINVAL;
  *bytes = 0;
  int st = decode_shape_status(batch, max_seqlen_k, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  if (st != VEA_OK) return st;
  int nsplit = 1;
  st = decode_split(batch * num_heads_kv, max_seqlen_k, head_dim, &nsplit);
  if (st != VEA_OK) return st;
  if (nsplit > 1) *bytes = (size_t)batch * num_heads_kv * nsplit * decode_chunk_bytes(num_heads_q / num_heads_kv, head_dim);
  return VEA_OK;
}

int vea_attn_decode(const void* q, int64_t q_seq_stride, const void* k, int64_t k_tok_stride, const void* v,
                    int64_t v_tok_stride, const int32_t* block_table, int max_pages_per_seq, int page_size,
                    int num_pages, const int32_t* cu_seqlens_k, int batch, int total_k, int max_seqlen_k,
                    int num_heads_q, int num_heads_kv, int head_dim, float scale, void* out, int64_t out_seq_stride,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Range range("vea_attn_decode");
  int st = decode_shape_status(batch, total_k, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  if (st != VEA_OK) return st;
  if (!isfinite(scale)) return VEA_EINVAL;
  int shift = 0;
  if (block_table != nullptr) {
    if (page_size < 64 || page_size > (1 << 16) || (page_size & (page_size - 1)) || num_pages < 0) return VEA_ESHAPE;
    while ((1 << shift) < page_size) ++shift;
    if (max_pages_per_seq < (max_seqlen_k + page_size - 1) / page_size) return VEA_ESHAPE;
  } else if (max_seqlen_k > total_k) {
    return VEA_ESHAPE;
  }
  if (batch == 0) return VEA_OK;
  if (!q || !out || !cu_seqlens_k) return VEA_EINVAL;
  const bool has_keys = block_table != nullptr ? num_pages > 0 : total_k > 0;
  if (has_keys && (!k || !v)) return VEA_EINVAL;
  const int64_t qrow = (int64_t)num_heads_q * head_dim, krow = (int64_t)num_heads_kv * head_dim;
  if (q_seq_stride < qrow || out_seq_stride < qrow || k_tok_stride < krow || v_tok_stride < krow) return VEA_ESHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VEA_EINVAL;
  if ((q_seq_stride * 2) % 16 || (k_tok_stride * 2) % 16 || (v_tok_stride * 2) % 16 || (out_seq_stride * 2) % 16)
    return VEA_EINVAL;
  if (workspace != nullptr && !aligned16(workspace)) return VEA_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (check_enabled()) {
    std::vector<int32_t> cu;
    st = fetch_ints(cu_seqlens_k, (size_t)batch + 1, s, cu);
    if (st != VEA_OK) return st;
    if (cu[0] != 0) return VEA_ERANGE;
    for (int b = 0; b < batch; ++b)
      if (cu[b + 1] < cu[b] || cu[b + 1] - cu[b] > max_seqlen_k) return VEA_ERANGE;
    if (cu[batch] != total_k) return VEA_ERANGE;     // packed: the rows of k/v; paged: the key total
    if (block_table != nullptr) {
      std::vector<int32_t> bt;
      st = fetch_ints(block_table, (size_t)batch * max_pages_per_seq, s, bt);
      if (st != VEA_OK) return st;
      for (int b = 0; b < batch; ++b)
        for (int pg = 0; pg < (cu[b + 1] - cu[b] + page_size - 1) / page_size; ++pg) {
          const int32_t x = bt[(size_t)b * max_pages_per_seq + pg];
          if (x < 0 || x >= num_pages) return VEA_ERANGE;
        }
    }
  }
  DenseParams p;
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.cu_q = cu_seqlens_k; p.cu_k = cu_seqlens_k;
  p.q_stride = q_seq_stride; p.k_stride = k_tok_stride; p.v_stride = v_tok_stride; p.o_stride = out_seq_stride;
  p.batch = batch; p.total_q = batch; p.total_k = total_k;
  p.hq = num_heads_kv; p.hkv = num_heads_kv; p.group = 1;     // units are (sequence, key/value head)
  st = dense_layout(batch, num_heads_q / num_heads_kv, num_heads_kv, 0, kDenseBM, p);
  if (st != VEA_OK) return st;
  p.dec_group = num_heads_q / num_heads_kv;
  p.ws_rows = (p.dec_group + 3) & ~3;
  p.xcd_map = 0;
  p.scale = scale;
  p.block_table = block_table;
  p.page_shift = shift;
  p.max_pages = max_pages_per_seq;
  if (workspace != nullptr) {
    int nsplit = 1;
    st = decode_split(p.units, max_seqlen_k, head_dim, &nsplit);
    if (st != VEA_OK) return st;
    if (nsplit > 1) {
      if (workspace_bytes < (size_t)p.units * nsplit * decode_chunk_bytes(p.dec_group, head_dim))
        return VEA_EWORKSPACE;
      p.full_units = 0;
      p.nsplit = nsplit;
      p.ws = (float*)workspace;
    }
  }
  return finish(hip_status(launch_attn_fwd_bf16(p, head_dim, false, s)), s);
}

int vea_attn_fwd_fp8(const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride, const void* v,
                     int64_t v_tok_stride, const float* q_scale, const float* k_scale, const float* v_scale,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int total_q, int total_k,
                     int max_seqlen_q, int max_seqlen_k, int num_heads_q, int num_heads_kv, int head_dim, int causal,
                     float scale, int piece_rows, void* out, int64_t out_tok_stride, float* lse, void* stream) {
  Range range("vea_attn_fwd_fp8");
  // same shape rules as the bf16 path
  int st = dense_shape_status(VEA_BF16, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q,
                              num_heads_kv, head_dim, causal, piece_rows);
  if (st != VEA_OK) return st;
  if (!isfinite(scale)) return VEA_EINVAL;
  if (batch == 0 || total_q == 0) return VEA_OK;
  if (!q || !out || !cu_seqlens_q || !cu_seqlens_k || !q_scale) return VEA_EINVAL;
  if (total_k > 0 && (!k || !v || !k_scale || !v_scale)) return VEA_EINVAL;
  const int64_t qrow = (int64_t)num_heads_q * head_dim, krow = (int64_t)num_heads_kv * head_dim;
  if (q_tok_stride < qrow || out_tok_stride < qrow || k_tok_stride < krow || v_tok_stride < krow) return VEA_ESHAPE;
  // 16-byte loads; per-lane DMA offsets are 32-bit (64 rows of a tile)
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (v_scale && !aligned16(v_scale)))
    return VEA_EINVAL;
  if (q_tok_stride % 16 || k_tok_stride % 16 || v_tok_stride % 16 || (out_tok_stride * 2) % 16) return VEA_EINVAL;
  if (k_tok_stride > (1 << 24) || v_tok_stride > (1 << 24)) return VEA_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (check_enabled()) {
    st = check_cu(cu_seqlens_q, batch, total_q, max_seqlen_q, s);
    if (st == VEA_OK) st = check_cu(cu_seqlens_k, batch, total_k, max_seqlen_k, s);
    if (st != VEA_OK) return st;
  }
  if (max_seqlen_q == 0) return finish(VEA_OK, s);
  DenseParams p;
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.q_stride = q_tok_stride; p.k_stride = k_tok_stride; p.v_stride = v_tok_stride; p.o_stride = out_tok_stride;
  p.batch = batch; p.total_q = total_q; p.total_k = total_k;
  p.hq = num_heads_q; p.hkv = num_heads_kv; p.group = num_heads_q / num_heads_kv;
  st = dense_layout(batch, max_seqlen_q, num_heads_q, piece_rows, kDenseBM, p);
  if (st != VEA_OK) return st;
  p.xcd_map = (num_heads_kv % 8 == 0) ? 1 : 0;
  p.scale = scale;
  p.q_scale = q_scale; p.k_scale = k_scale; p.v_scale = v_scale;
  return finish(hip_status(launch_attn_fwd_fp8(p, head_dim, causal != 0, s)), s);
}

int vea_quantize_fp8(const void* x, int64_t x_tok_stride, int num_tokens, int num_heads, int head_dim,
                     int granularity, void* out, float* scales, void* stream) {
  Range range("vea_quantize_fp8");
  if (num_tokens < 0 || num_heads <= 0) return VEA_ESHAPE;
  if (granularity < 0 || granularity > 2) return VEA_EINVAL;
  if (head_dim != 64 && head_dim != 128) return VEA_EUNSUPPORTED;
  if (x_tok_stride < (int64_t)num_heads * head_dim) return VEA_ESHAPE;
  if (num_tokens == 0 && granularity == 0) return VEA_OK;
  if (!scales || (num_tokens > 0 && (!x || !out))) return VEA_EINVAL;
  if ((x && !aligned16(x)) || (out && !aligned16(out)) || !aligned16(scales) || (x_tok_stride * 2) % 16)
    return VEA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  QuantParams p;
  p.x = (const uint16_t*)x; p.x_stride = x_tok_stride; p.out = (uint8_t*)out; p.scales = scales;
  p.tokens = num_tokens; p.heads = num_heads; p.d = head_dim; p.granularity = granularity;
  return finish(hip_status(launch_quant_fp8(p, s)), s);
}

int vea_qkv_rope(const void* x_qkv, int64_t x_tok_stride, const int32_t* positions, int pos_dims, int num_tokens,
                 int num_heads_q, int num_heads_kv, int head_dim, float theta, int rotate_half, void* q, void* k,
                 void* stream) {
  Range range("vea_qkv_rope");
  if (num_tokens < 0 || num_heads_q <= 0 || num_heads_kv <= 0 || head_dim <= 0) return VEA_ESHAPE;
  if (pos_dims != 1 && pos_dims != 2) return VEA_EINVAL;
  if (!isfinite(theta) || !(theta > 0.f)) return VEA_EINVAL;
  if (head_dim % 8 != 0 || head_dim > 256 || (pos_dims == 2 && head_dim % 4 != 0)) return VEA_EUNSUPPORTED;
  if (rotate_half != 0 && rotate_half != 1) return VEA_EINVAL;
  if (rotate_half && head_dim % 32 != 0) return VEA_EUNSUPPORTED;   // whole 16-byte chunks per half span
  if (num_tokens == 0) return VEA_OK;
  if (!x_qkv || !positions || !q || !k) return VEA_EINVAL;
  if (x_tok_stride < (int64_t)(num_heads_q + 2 * num_heads_kv) * head_dim) return VEA_ESHAPE;
  if (!aligned16(x_qkv) || !aligned16(q) || !aligned16(k) || (x_tok_stride * 2) % 16) return VEA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  RopeParams p;
  p.x = (const uint16_t*)x_qkv; p.pos = positions; p.q = (uint16_t*)q; p.k = (uint16_t*)k;
  p.x_stride = x_tok_stride; p.tokens = num_tokens; p.hq = num_heads_q; p.hkv = num_heads_kv;
  p.d = head_dim; p.pos_dims = pos_dims; p.theta = (double)theta; p.rot_half = rotate_half;
  return finish(hip_status(launch_qkv_rope(p, s)), s);
}

namespace {

int sparse_shape_status(int num_rows, int num_heads, int d_qk, int d_v, int k) {
  if (num_rows < 0 || num_heads <= 0 || k <= 0) return VEA_ESHAPE;
  if (d_v <= 0 || d_qk <= 0 || d_v > d_qk) return VEA_ESHAPE;
  if (d_qk != 576 || d_v != 512 || k > 4096) return VEA_EUNSUPPORTED;
  const int64_t units = (int64_t)num_rows * ((num_heads + kSparseHeadsPerWG - 1) / kSparseHeadsPerWG);
  if (units * 8 > 0x7fffffff) return VEA_EUNSUPPORTED;
  return VEA_OK;
}

// CU count of the current device (the split plan's round size).
int current_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VEA_EHIP;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return VEA_EHIP;
  return VEA_OK;
}

}  // namespace

int vea_sparse_mqa_workspace_size(int num_rows, int num_heads, int d_qk, int d_v, int k, size_t* bytes) {
  if (bytes == nullptr) return VEA_EINVAL;
  *bytes = 0;
  int st = sparse_shape_status(num_rows, num_heads, d_qk, d_v, k);
  if (st != VEA_OK) return st;
  if (num_rows == 0) return VEA_OK;
  int cus = 0;
  st = current_cus(&cus);
  if (st != VEA_OK) return st;
  const int head_blocks = (num_heads + kSparseHeadsPerWG - 1) / kSparseHeadsPerWG;
  const SparseSplit plan = sparse_split_plan(num_rows * head_blocks, k, cus);
  *bytes = (size_t)plan.chunks * sparse_chunk_bytes(d_v);
  return VEA_OK;
}

namespace {

int sparse_fwd(const void* q, const void* kv, const int32_t* page_table, int page_size, int num_pages,
               const int32_t* topk_idx, int num_rows, int num_heads, int n_kv, int d_qk, int d_v, int k, float scale,
               void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_kv < 0) return VEA_ESHAPE;
  int st = sparse_shape_status(num_rows, num_heads, d_qk, d_v, k);
  if (st != VEA_OK) return st;
  if (!isfinite(scale)) return VEA_EINVAL;
  int shift = 0;
  int64_t n_phys = n_kv;
  if (page_table != nullptr) {
    if (page_size < 1 || page_size > (1 << 16) || (page_size & (page_size - 1)) || num_pages < 0) return VEA_ESHAPE;
    while ((1 << shift) < page_size) ++shift;
    n_phys = (int64_t)num_pages * page_size;
  }
  if (n_phys * 1152 >= ((int64_t)1 << 32) || n_kv >= (1 << 24)) return VEA_EUNSUPPORTED;   // 32-bit row offsets
  if (num_rows == 0) return VEA_OK;
  if (!q || !topk_idx || !out || (n_phys > 0 && !kv)) return VEA_EINVAL;
  if (!aligned16(q) || !aligned16(out) || (kv && !aligned16(kv))) return VEA_EINVAL;
  if (workspace != nullptr && !aligned16(workspace)) return VEA_EWORKSPACE;
  SparseParams p;
  p.q = (const uint16_t*)q; p.kv = (const uint16_t*)kv; p.idx = topk_idx; p.out = (uint16_t*)out;
  p.lse = lse; p.rows = num_rows; p.heads = num_heads; p.n_kv = n_kv; p.k = k;
  p.head_blocks = (num_heads + kSparseHeadsPerWG - 1) / kSparseHeadsPerWG;
  p.scale = scale;
  p.full_units = num_rows * p.head_blocks;
  p.nsplit = 1;
  p.ws = nullptr;
  p.page_table = page_table;
  p.page_shift = shift;
  p.n_phys = (int)n_phys;
  p.grid = 0;
  p.wg_perm = 0;
  if (workspace != nullptr) {
    int cus = 0;
    st = current_cus(&cus);
    if (st != VEA_OK) return st;
    const SparseSplit plan = sparse_split_plan(p.full_units, k, cus);
    if (plan.nsplit > 1) {
      if (workspace_bytes < (size_t)plan.chunks * sparse_chunk_bytes(d_v)) return VEA_EWORKSPACE;
      p.full_units = plan.full_units;
      p.nsplit = plan.nsplit;
      p.ws = (float*)workspace;
    }
  }
  hipStream_t s = (hipStream_t)stream;
  if (check_enabled()) {
    std::vector<int32_t> h;
    st = fetch_ints(topk_idx, (size_t)num_rows * k, s, h);
    if (st != VEA_OK) return st;
    for (int32_t x : h)
      if (x >= n_kv) return VEA_ERANGE;
    if (page_table != nullptr) {
      st = fetch_ints(page_table, (size_t)((n_kv + page_size - 1) / page_size), s, h);
      if (st != VEA_OK) return st;
      for (int32_t x : h)
        if (x < 0 || x >= num_pages) return VEA_ERANGE;
    }
  }
  return finish(hip_status(launch_sparse_mqa(p, d_qk, d_v, s)), s);
}

}  // namespace

int vea_sparse_mqa_fwd(const void* q, const void* kv_latent, const int32_t* topk_idx, int num_rows, int num_heads,
                       int n_kv, int d_qk, int d_v, int k, float scale, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Range range("vea_sparse_mqa_fwd");
  return sparse_fwd(q, kv_latent, nullptr, 0, 0, topk_idx, num_rows, num_heads, n_kv, d_qk, d_v, k, scale, out, lse,
                    workspace, workspace_bytes, stream);
}

int vea_sparse_mqa_paged_fwd(const void* q, const void* kv_cache, const int32_t* page_table, int page_size,
                             int num_pages, const int32_t* topk_idx, int num_rows, int num_heads, int n_kv, int d_qk,
                             int d_v, int k, float scale, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Range range("vea_sparse_mqa_paged_fwd");
  if (page_table == nullptr && num_rows > 0) return VEA_EINVAL;
  return sparse_fwd(q, kv_cache, page_table, page_size, num_pages, topk_idx, num_rows, num_heads, n_kv, d_qk, d_v, k,
                    scale, out, lse, workspace, workspace_bytes, stream);
}

int vea_topk_indices(const float* logits, int64_t row_stride, const int32_t* row_starts, const int32_t* row_lens,
                     int num_rows, int n, int k, int32_t* out, void* stream) {
  Range range("vea_topk_indices");
  if (num_rows < 0 || n < 1 || k < 1) return VEA_ESHAPE;
  if (row_stride < n) return VEA_ESHAPE;
  if (n > kTopkMaxN) return VEA_EUNSUPPORTED;
  if (num_rows == 0) return VEA_OK;
  if (!logits || !out) return VEA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u)) return VEA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (check_enabled()) {
    std::vector<int32_t> hs, hl;
    int st = VEA_OK;
    if (row_starts) st = fetch_ints(row_starts, (size_t)num_rows, s, hs);
    if (st == VEA_OK && row_lens) st = fetch_ints(row_lens, (size_t)num_rows, s, hl);
    if (st != VEA_OK) return st;
    for (int r = 0; r < num_rows; ++r) {
      const int64_t b = row_starts ? hs[r] : 0;
      const int64_t l = row_lens ? hl[r] : n - b;
      if (b < 0 || l < 0 || b + l > n) return VEA_ERANGE;
    }
  }
  TopkParams p;
  p.logits = logits; p.row_stride = row_stride; p.starts = row_starts; p.lens = row_lens; p.out = out;
  p.rows = num_rows; p.n = n; p.k = k;
  return finish(hip_status(launch_topk(p, s)), s);
}

int vea_rope_cos_sin(const int32_t* positions, int pos_dims, int num_tokens, int head_dim, float theta,
                     float* cos_sin, void* stream) {
  Range range("vea_rope_cos_sin");
  if (num_tokens < 0 || head_dim <= 0) return VEA_ESHAPE;
  if (pos_dims != 1 && pos_dims != 2) return VEA_EINVAL;
  if (!isfinite(theta) || !(theta > 0.f)) return VEA_EINVAL;
  if (head_dim % 2 != 0 || head_dim > 256 || (pos_dims == 2 && head_dim % 4 != 0)) return VEA_EUNSUPPORTED;
  if (num_tokens == 0) return VEA_OK;
  if (!positions || !cos_sin) return VEA_EINVAL;
  if (reinterpret_cast<uintptr_t>(cos_sin) & 7u) return VEA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  RopeTableParams p;
  p.pos = positions; p.out = cos_sin; p.tokens = num_tokens; p.d = head_dim; p.pos_dims = pos_dims;
  p.theta = (double)theta;
  return finish(hip_status(launch_rope_cos_sin(p, s)), s);
}

int vea_qkv_proj_rope(const void* x, int64_t x_tok_stride, const void* w, int64_t w_row_stride, const void* bias,
                      const float* cos_sin, int num_tokens, int hidden, int num_heads_q, int num_heads_kv,
                      int head_dim, int rotate_half_span, void* q, void* k, void* v, void* stream) {
  Range range("vea_qkv_proj_rope");
  if (num_tokens < 0 || hidden <= 0 || num_heads_q <= 0 || num_heads_kv <= 0 || head_dim <= 0) return VEA_ESHAPE;
  const int64_t n = (int64_t)(num_heads_q + 2 * (int64_t)num_heads_kv) * head_dim;
  if (x_tok_stride < hidden || w_row_stride < n) return VEA_ESHAPE;
  if (hidden % kProjStepK != 0 || head_dim % 32 != 0 || head_dim > 256) return VEA_EUNSUPPORTED;
  if (rotate_half_span != 0 && rotate_half_span != head_dim && rotate_half_span != head_dim / 2) return VEA_EINVAL;
  // rotate-half partners are found within a wave's 128 features
  if (rotate_half_span != 0 && head_dim != 64 && head_dim != 128) return VEA_EUNSUPPORTED;
  // Buffer ranges and per-lane offsets are 32-bit.
  if (n > 0x7fffffff / 2 || (int64_t)num_tokens * x_tok_stride * 2 > 0x7fffffff ||
      (int64_t)kProjTileT * x_tok_stride * 2 > 0x7fffffff || (int64_t)hidden * w_row_stride * 2 > 0x7fffffff)
    return VEA_EUNSUPPORTED;
  const int64_t ftiles = (n + kProjTileF - 1) / kProjTileF;
  if (ftiles * ((num_tokens + kProjTileT - 1) / kProjTileT) > 0x7fffffff) return VEA_EUNSUPPORTED;
  if (num_tokens == 0) return VEA_OK;
  if (!x || !w || !q || !k || !v) return VEA_EINVAL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return VEA_EINVAL;
  if ((bias && !aligned16(bias)) || (cos_sin && !aligned16(cos_sin))) return VEA_EINVAL;
  if ((x_tok_stride * 2) % 16 || (w_row_stride * 2) % 16) return VEA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  ProjParams p;
  p.x = (const uint16_t*)x; p.w = (const uint16_t*)w; p.bias = (const uint16_t*)bias; p.cs = cos_sin;
  p.q = (uint16_t*)q; p.k = (uint16_t*)k; p.v = (uint16_t*)v;
  p.x_stride = x_tok_stride; p.w_stride = w_row_stride;
  p.tokens = num_tokens; p.hidden = hidden; p.hq = num_heads_q; p.hkv = num_heads_kv; p.d = head_dim;
  p.n_feat = (int)n; p.ftiles = (int)ftiles; p.rot_span = rotate_half_span;
  return finish(hip_status(launch_qkv_proj(p, s)), s);
}

int vea_attn_probs_piece(int dtype, const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                         const float* lse, int64_t lse_row_stride, int head, int num_heads_q, int num_heads_kv,
                         int head_dim, int seq_begin_q, int len_q, int seq_begin_k, int len_k, int q0, int rows,
                         int causal, float scale, float* p_out, int64_t p_row_stride, void* stream) {
  Range range("vea_attn_probs_piece");
  if (dtype != VEA_BF16 && dtype != VEA_F32) return VEA_EDTYPE;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv) return VEA_ESHAPE;
  if (head < 0 || head >= num_heads_q || head_dim <= 0) return VEA_ESHAPE;
  if (seq_begin_q < 0 || seq_begin_k < 0 || len_q < 0 || len_k < 0 || q0 < 0 || rows < 0 || q0 + rows > len_q)
    return VEA_ESHAPE;
  if (p_row_stride < len_k || lse_row_stride < seq_begin_q + len_q) return VEA_ESHAPE;
  if (q_tok_stride < (int64_t)num_heads_q * head_dim || k_tok_stride < (int64_t)num_heads_kv * head_dim)
    return VEA_ESHAPE;
  if (!isfinite(scale) || (causal != 0 && causal != 1)) return VEA_EINVAL;
  if (rows == 0 || len_k == 0) return VEA_OK;
  if (!q || !k || !lse || !p_out) return VEA_EINVAL;
  ProbsParams p;
  p.q = q; p.k = k; p.lse = lse; p.p = p_out;
  p.q_stride = q_tok_stride; p.k_stride = k_tok_stride; p.lse_stride = lse_row_stride; p.p_stride = p_row_stride;
  p.head = head; p.kv_head = head / (num_heads_q / num_heads_kv); p.d = head_dim;
  p.seq_q = seq_begin_q; p.len_q = len_q; p.seq_k = seq_begin_k; p.len_k = len_k; p.q0 = q0; p.rows = rows;
  p.causal = causal; p.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  return finish(hip_status(launch_attn_probs(p, dtype == VEA_BF16, s)), s);
}

}  // extern "C"
