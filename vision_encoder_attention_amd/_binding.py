"""ctypes binding of libvea.so: argument marshalling only.

Every function here takes torch tensors that already live on the GPU, reads
their data pointers, element strides and the current HIP stream, and calls the
C ABI declared in include/vea.h.  All computation happens in the HIP kernels;
there is no Python or CPU fallback.  If the library is missing the first call
raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvea.so")

VEA_F32, VEA_BF16 = 0, 1
_lock = threading.Lock()
_lib = None


class VeaError(RuntimeError):
    """A vea_* call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


def lib_path() -> str:
    return LIB_PATH


def load_library():
    """Load libvea.so once (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libvea.so not found at %s; build it with "
                               "`python -m vision_encoder_attention_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.vea_status_str.argtypes = [i32]
        lib.vea_status_str.restype = ctypes.c_char_p
        lib.vea_version.argtypes = []
        lib.vea_version.restype = ctypes.c_char_p
        lib.vea_attn_fwd.argtypes = [i32, vp, i64, vp, i64, vp, i64, vp, vp, i32, i32, i32, i32, i32,
                                     i32, i32, i32, i32, f32, i32, vp, i64, vp, vp, ctypes.c_size_t, vp]
        lib.vea_attn_fwd.restype = i32
        lib.vea_attn_fwd_noalloc.argtypes = [i32, vp, i64, vp, i64, vp, i64, vp, vp, i32, i32, i32, i32, i32,
                                             i32, i32, i32, i32, f32, i32, vp, i64, vp, vp]
        lib.vea_attn_fwd_noalloc.restype = i32
        lib.vea_attn_fwd_paged.argtypes = [vp, i64, vp, i64, vp, i64, vp, i32, i32, i32, vp, vp, i32, i32, i32,
                                           i32, i32, i32, i32, i32, i32, f32, i32, vp, i64, vp, vp,
                                           ctypes.c_size_t, vp]
        lib.vea_attn_fwd_paged.restype = i32
        lib.vea_attn_decode.argtypes = [vp, i64, vp, i64, vp, i64, vp, i32, i32, i32, vp, i32, i32, i32, i32, i32,
                                        i32, f32, vp, i64, vp, vp, ctypes.c_size_t, vp]
        lib.vea_attn_decode.restype = i32
        lib.vea_attn_decode_workspace_size.argtypes = [i32] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
        lib.vea_attn_decode_workspace_size.restype = i32
        lib.vea_attn_fwd_workspace_size.argtypes = [i32] * 11 + [ctypes.POINTER(ctypes.c_size_t)]
        lib.vea_attn_fwd_workspace_size.restype = i32
        lib.vea_qkv_rope.argtypes = [vp, i64, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp]
        lib.vea_qkv_rope.restype = i32
        lib.vea_sparse_mqa_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                                           ctypes.c_size_t, vp]
        lib.vea_sparse_mqa_fwd.restype = i32
        lib.vea_sparse_mqa_paged_fwd.argtypes = [vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                                 vp, ctypes.c_size_t, vp]
        lib.vea_sparse_mqa_paged_fwd.restype = i32
        lib.vea_sparse_mqa_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
        lib.vea_sparse_mqa_workspace_size.restype = i32
        lib.vea_topk_indices.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp]
        lib.vea_topk_indices.restype = i32
        lib.vea_quantize_fp8.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp]
        lib.vea_quantize_fp8.restype = i32
        lib.vea_attn_fwd_fp8.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         i32, i32, i32, i32, f32, i32, vp, i64, vp, vp]
        lib.vea_attn_fwd_fp8.restype = i32
        lib.vea_rope_cos_sin.argtypes = [vp, i32, i32, i32, f32, vp, vp]
        lib.vea_rope_cos_sin.restype = i32
        lib.vea_qkv_proj_rope.argtypes = [vp, i64, vp, i64, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        lib.vea_qkv_proj_rope.restype = i32
        lib.vea_attn_probs_piece.argtypes = [i32, vp, i64, vp, i64, vp, i64, i32, i32, i32, i32, i32, i32,
                                             i32, i32, i32, i32, i32, f32, vp, i64, vp]
        lib.vea_attn_probs_piece.restype = i32
        _lib = lib
        return lib


def status_str(status: int) -> str:
    return load_library().vea_status_str(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise VeaError(status, status_str(status))


# ------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return VEA_BF16
    if t.dtype == torch.float32:
        return VEA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _token_major(t, name):
    """[tokens, heads, dim] view with contiguous heads and dims; returns token stride."""
    if t.dim() != 3:
        raise ValueError("%s must be [tokens, heads, dim]" % name)
    if t.numel() == 0:
        return t.shape[1] * t.shape[2]          # empty: strides are meaningless, nothing is read
    if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError("%s must have contiguous heads and head dims (token stride may differ)" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    return t.stride(0)


def _on_device(dev, *named):
    """Every given tensor, (name, tensor) pairs, None skipped, lives on dev:
    the call launches on q's device with raw pointers, so a tensor elsewhere
    would be read through an address that means nothing there."""
    for name, t in named:
        if t is not None and t.device != dev:
            raise ValueError("%s must be on %s (the device of the call), not %s" % (name, dev, t.device))


def _shape(t, want, name):
    if tuple(t.shape) != tuple(want):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(want), tuple(t.shape)))


def _dense_shapes(q, k, v, out, kname="k", vname="v"):
    """k and v of one shape [rows, Hkv, d] with q's d; out of q's shape."""
    _shape(v, k.shape, vname)
    if k.shape[2] != q.shape[2]:
        raise ValueError("%s must have q's head_dim %d, got %d" % (kname, q.shape[2], k.shape[2]))
    _shape(out, q.shape, "out")


def _int32_dev(t, name):
    torch = _torch()
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous int32 GPU tensor" % name)


def attn_fwd_workspace_size(dtype_code, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, heads_q, heads_kv,
                            head_dim, causal, piece_rows=0) -> int:
    """Workspace bytes vea_attn_fwd uses for these sizes on the current device
    (0: no split)."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.vea_attn_fwd_workspace_size(int(dtype_code), int(batch), int(total_q), int(total_k),
                                           int(max_seqlen_q), int(max_seqlen_k), int(heads_q), int(heads_kv),
                                           int(head_dim), 1 if causal else 0, int(piece_rows), ctypes.byref(n)))
    return int(n.value)


def attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, causal, scale, out, lse=None, *, piece_rows=0,
             max_seqlen_q=None, max_seqlen_k=None, workspace="auto"):
    """Blockwise attention forward (see vea_attn_fwd in include/vea.h).

    q [total_q, Hq, d], k/v [total_k, Hkv, d] (token strides free), out like q,
    lse float32 [Hq, total_q] or None.  max_seqlen_* default to the largest
    sequence length, read from cu_seqlens with one host copy (synchronising).
    workspace: "auto" allocates what the call asks for (a split of the last
    round of workgroups for one non-causal bf16 sequence), None never splits,
    or a contiguous uint8 GPU tensor to use.
    """
    lib = load_library()
    qs, ks, vs, os_ = (_token_major(q, "q"), _token_major(k, "k"), _token_major(v, "v"),
                       _token_major(out, "out"))
    _int32_dev(cu_seqlens_q, "cu_seqlens_q")
    _int32_dev(cu_seqlens_k, "cu_seqlens_k")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k, v and out must share a dtype")
    _dense_shapes(q, k, v, out)
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same number of entries")
    _on_device(q.device, ("k", k), ("v", v), ("out", out), ("cu_seqlens_q", cu_seqlens_q),
               ("cu_seqlens_k", cu_seqlens_k), ("lse", lse),
               ("workspace", None if isinstance(workspace, str) else workspace))
    if lse is not None:
        torch = _torch()
        if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (q.shape[1], q.shape[0]):
            raise ValueError("lse must be contiguous float32 [Hq, total_q]")
    batch = cu_seqlens_q.numel() - 1
    if max_seqlen_q is None or max_seqlen_k is None:
        lq = (cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item() if batch > 0 else 0
        lk = (cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item() if batch > 0 else 0
        max_seqlen_q = lq if max_seqlen_q is None else max_seqlen_q
        max_seqlen_k = lk if max_seqlen_k is None else max_seqlen_k
    torch = _torch()
    with torch.cuda.device(q.device):
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a uint8 GPU tensor')
            nbytes = attn_fwd_workspace_size(dt, batch, q.shape[0], k.shape[0], max_seqlen_q, max_seqlen_k,
                                             q.shape[1], k.shape[1], q.shape[2], causal, piece_rows)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
        if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()
                                      or workspace.device != q.device):
            raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
        st = lib.vea_attn_fwd(dt, _ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                              batch, q.shape[0], k.shape[0], int(max_seqlen_q), int(max_seqlen_k), q.shape[1],
                              k.shape[1], q.shape[2], 1 if causal else 0, float(scale), int(piece_rows),
                              _ptr(out), os_, _ptr(lse), _ptr(workspace),
                              0 if workspace is None else workspace.numel(), _stream(q))
    _check(st)
    return out, lse


def attn_fwd_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, causal, scale, out, lse=None, *, piece_rows=0,
                     max_seqlen_q, max_seqlen_k):
    """attn_fwd for callers that cannot allocate (see vea_attn_fwd_noalloc):
    the split of the last round uses the library's static scratch, so the
    call allocates nothing; max_seqlen_q / max_seqlen_k are required (no
    read-back of cu_seqlens).  Calls that overlap on one GPU race on that
    scratch."""
    lib = load_library()
    qs, ks, vs, os_ = (_token_major(q, "q"), _token_major(k, "k"), _token_major(v, "v"),
                       _token_major(out, "out"))
    _int32_dev(cu_seqlens_q, "cu_seqlens_q")
    _int32_dev(cu_seqlens_k, "cu_seqlens_k")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k, v and out must share a dtype")
    _dense_shapes(q, k, v, out)
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same number of entries")
    _on_device(q.device, ("k", k), ("v", v), ("out", out), ("cu_seqlens_q", cu_seqlens_q),
               ("cu_seqlens_k", cu_seqlens_k), ("lse", lse))
    if lse is not None:
        torch = _torch()
        if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (q.shape[1], q.shape[0]):
            raise ValueError("lse must be contiguous float32 [Hq, total_q]")
    torch = _torch()
    with torch.cuda.device(q.device):
        st = lib.vea_attn_fwd_noalloc(dt, _ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _ptr(cu_seqlens_q),
                                      _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1, q.shape[0], k.shape[0],
                                      int(max_seqlen_q), int(max_seqlen_k), q.shape[1], k.shape[1], q.shape[2],
                                      1 if causal else 0, float(scale), int(piece_rows), _ptr(out), os_, _ptr(lse),
                                      _stream(q))
    _check(st)
    return out, lse


def attn_fwd_paged(q, k_cache, v_cache, block_table, page_size, cu_seqlens_q, cu_seqlens_k, causal, scale, out,
                   lse=None, *, piece_rows=0, max_seqlen_q=None, max_seqlen_k=None, total_k=None,
                   workspace="auto"):
    """attn_fwd (bf16) over paged K/V caches (see vea_attn_fwd_paged):
    k_cache / v_cache [num_pages * page_size, Hkv, d] (token strides free),
    block_table int32 [batch, max_pages_per_seq]; cu_seqlens_k gives the key
    lengths.  max_seqlen_* and total_k (the sum of the key lengths) default
    to values read from cu_seqlens with a host copy (synchronising)."""
    lib = load_library()
    torch = _torch()
    qs, ks, vs, os_ = (_token_major(q, "q"), _token_major(k_cache, "k_cache"), _token_major(v_cache, "v_cache"),
                       _token_major(out, "out"))
    _int32_dev(cu_seqlens_q, "cu_seqlens_q")
    _int32_dev(cu_seqlens_k, "cu_seqlens_k")
    _int32_dev(block_table, "block_table")
    if q.dtype != torch.bfloat16 or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k_cache, v_cache and out must be bfloat16")
    if block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [batch, max_pages_per_seq]")
    page_size = int(page_size)
    if page_size < 1 or k_cache.shape[0] % page_size or v_cache.shape[0] != k_cache.shape[0]:
        raise ValueError("cache rows must be a multiple of page_size and equal for k and v")
    _dense_shapes(q, k_cache, v_cache, out, "k_cache", "v_cache")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same number of entries")
    _on_device(q.device, ("k_cache", k_cache), ("v_cache", v_cache), ("out", out), ("block_table", block_table),
               ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k), ("lse", lse),
               ("workspace", None if isinstance(workspace, str) else workspace))
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (q.shape[1], q.shape[0])):
        raise ValueError("lse must be contiguous float32 [Hq, total_q]")
    batch = cu_seqlens_q.numel() - 1
    if block_table.shape[0] != batch:
        raise ValueError("block_table needs one row per sequence")
    if max_seqlen_q is None or max_seqlen_k is None:
        lq = (cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item() if batch > 0 else 0
        lk = (cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item() if batch > 0 else 0
        max_seqlen_q = lq if max_seqlen_q is None else max_seqlen_q
        max_seqlen_k = lk if max_seqlen_k is None else max_seqlen_k
    if total_k is None:
        total_k = int(cu_seqlens_k[-1].item()) if batch > 0 else 0
    with torch.cuda.device(q.device):
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a uint8 GPU tensor')
            nbytes = attn_fwd_workspace_size(VEA_BF16, batch, q.shape[0], total_k, max_seqlen_q, max_seqlen_k,
                                             q.shape[1], k_cache.shape[1], q.shape[2], causal, piece_rows)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
        st = lib.vea_attn_fwd_paged(_ptr(q), qs, _ptr(k_cache), ks, _ptr(v_cache), vs, _ptr(block_table),
                                    block_table.shape[1], page_size, k_cache.shape[0] // page_size,
                                    _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, q.shape[0], total_k,
                                    int(max_seqlen_q), int(max_seqlen_k), q.shape[1], k_cache.shape[1], q.shape[2],
                                    1 if causal else 0, float(scale), int(piece_rows), _ptr(out), os_, _ptr(lse),
                                    _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q))
    _check(st)
    return out, lse


def packed_total_k(k_rows: int, v_rows: int, total_k=None) -> int:
    """total_k of a packed K/V pair: the kernel bounds every key row by it, so
    it must be the number of rows k and v really hold."""
    if v_rows != k_rows:
        raise ValueError("packed k and v need the same number of rows (%d, %d)" % (k_rows, v_rows))
    if total_k is not None and int(total_k) != k_rows:
        raise ValueError("packed K/V: total_k (%d) must equal k.shape[0] (%d)" % (int(total_k), k_rows))
    return int(k_rows)


def attn_decode_workspace_size(batch, max_seqlen_k, heads_q, heads_kv, head_dim) -> int:
    """Workspace bytes vea_attn_decode uses for these sizes on the current
    device (0: no split)."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.vea_attn_decode_workspace_size(int(batch), int(max_seqlen_k), int(heads_q), int(heads_kv),
                                              int(head_dim), ctypes.byref(n)))
    return n.value


def attn_decode(q, k, v, cu_seqlens_k, scale, out, lse=None, *, block_table=None, page_size=0, max_seqlen_k=None,
                total_k=None, workspace="auto"):
    """One query token per sequence over its cached keys (see vea_attn_decode):
    q / out [batch, Hq, d] bf16; k / v packed [total_k, Hkv, d] by
    cu_seqlens_k, or, with block_table int32 [batch, max_pages_per_seq],
    caches [num_pages * page_size, Hkv, d]; lse float32 [Hq, batch].
    max_seqlen_k defaults to the longest key length, read from cu_seqlens_k
    with a host copy (synchronising).  total_k: for packed K/V it is
    k.shape[0] (any other value is rejected); for paged caches it must be the
    sum of the key lengths (cu_seqlens_k[-1]), read back from the device when
    omitted."""
    lib = load_library()
    torch = _torch()
    qs, ks, vs, os_ = (_token_major(q, "q"), _token_major(k, "k"), _token_major(v, "v"), _token_major(out, "out"))
    _int32_dev(cu_seqlens_k, "cu_seqlens_k")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k, v and out must be bfloat16")
    batch = cu_seqlens_k.numel() - 1
    if q.shape[0] != batch or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out need one row per sequence")
    _dense_shapes(q, k, v, out)
    _on_device(q.device, ("k", k), ("v", v), ("out", out), ("cu_seqlens_k", cu_seqlens_k), ("lse", lse),
               ("block_table", block_table), ("workspace", None if isinstance(workspace, str) else workspace))
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (q.shape[1], batch)):
        raise ValueError("lse must be contiguous float32 [Hq, batch]")
    if max_seqlen_k is None:
        max_seqlen_k = (cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item() if batch > 0 else 0
    if block_table is None:
        total_k = packed_total_k(k.shape[0], v.shape[0], total_k)
    elif total_k is None:
        total_k = int(cu_seqlens_k[-1].item()) if batch > 0 else 0
    if block_table is not None:
        _int32_dev(block_table, "block_table")
        if block_table.dim() != 2 or not block_table.is_contiguous() or block_table.shape[0] != batch:
            raise ValueError("block_table must be contiguous int32 [batch, max_pages_per_seq]")
        page_size = int(page_size)
        if page_size < 1 or k.shape[0] % page_size or v.shape[0] != k.shape[0]:
            raise ValueError("cache rows must be a multiple of page_size and equal for k and v")
        mp, n_pages = block_table.shape[1], k.shape[0] // page_size
    else:
        page_size, mp, n_pages = 0, 0, 0
    with torch.cuda.device(q.device):
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a uint8 GPU tensor')
            nbytes = attn_decode_workspace_size(batch, max_seqlen_k, q.shape[1], k.shape[1], q.shape[2])
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
        st = lib.vea_attn_decode(_ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _ptr(block_table), mp, page_size, n_pages,
                                 _ptr(cu_seqlens_k), batch, total_k, int(max_seqlen_k), q.shape[1], k.shape[1],
                                 q.shape[2], float(scale), _ptr(out), os_, _ptr(lse), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream(q))
    _check(st)
    return out, lse


def qkv_rope(x_qkv, positions, theta, q, k, rotate_half=False):
    """Split the fused [T, (Hq+2Hkv) d] projection output into rotated q [T, Hq, d]
    and k [T, Hkv, d] (see vea_qkv_rope); V stays in x_qkv."""
    lib = load_library()
    torch = _torch()
    if x_qkv.dtype != torch.bfloat16 or q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise TypeError("qkv_rope works on bfloat16")
    if x_qkv.dim() != 2 or x_qkv.stride(1) != 1:
        raise ValueError("x_qkv must be [tokens, cols] with contiguous columns")
    if not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k outputs must be contiguous")
    _int32_dev(positions, "positions")
    t = x_qkv.shape[0]
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != t or k.shape[0] != t or k.shape[2] != q.shape[2]:
        raise ValueError("q [T, Hq, d] and k [T, Hkv, d] must have x_qkv's T tokens and one head_dim")
    if x_qkv.shape[1] < (q.shape[1] + k.shape[1]) * q.shape[2]:
        raise ValueError("x_qkv holds fewer columns than the Q and K heads")
    if positions.shape[0] != t or not (positions.dim() == 1 or (positions.dim() == 2 and positions.shape[1] == 2)):
        raise ValueError("positions must be int32 [T] or [T, 2]")
    _on_device(x_qkv.device, ("q", q), ("k", k), ("positions", positions))
    st = lib.vea_qkv_rope(_ptr(x_qkv), x_qkv.stride(0), _ptr(positions), positions.dim(), x_qkv.shape[0],
                          q.shape[1], k.shape[1], q.shape[2], float(theta), int(bool(rotate_half)), _ptr(q), _ptr(k),
                          _stream(x_qkv))
    _check(st)
    return q, k


def quantize_fp8(x, granularity, out=None, scales=None):
    """Block quantisation of bf16 x [T, H, d] to E4M3 codes (see
    vea_quantize_fp8).  granularity 0: scales [T, H]; 1: [H]; 2: [H, d].
    Returns (codes uint8 [T, H, d], scales float32)."""
    lib = load_library()
    torch = _torch()
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 3 or x.stride(2) != 1 or x.stride(1) != x.shape[2]:
        raise ValueError("x must be a bfloat16 GPU tensor [T, H, d] with contiguous heads")
    t, hh, d = x.shape
    shape = {0: (t, hh), 1: (hh,), 2: (hh, d)}[int(granularity)]
    if out is None:
        out = torch.empty((t, hh, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    if out.dtype != torch.uint8 or not out.is_contiguous() or tuple(out.shape) != (t, hh, d):
        raise ValueError("out must be a contiguous uint8 [T, H, d] tensor")
    if scales.dtype != torch.float32 or not scales.is_contiguous() or tuple(scales.shape) != shape:
        raise ValueError("scales must be a contiguous float32 tensor of shape %s" % (shape,))
    _check(lib.vea_quantize_fp8(_ptr(x), x.stride(0), t, hh, d, int(granularity), _ptr(out), _ptr(scales), _stream(x)))
    return out, scales


def attn_fwd_fp8(q, q_scale, k, k_scale, v, v_scale, cu_seqlens_q, cu_seqlens_k, causal, scale, out, lse=None, *,
                 piece_rows=0, max_seqlen_q=None, max_seqlen_k=None):
    """Attention on E4M3 codes (see vea_attn_fwd_fp8): q [Tq, Hq, d] uint8 with
    q_scale [Tq, Hq], k / v [Tk, Hkv, d] uint8 with k_scale [Hkv] and v_scale
    [Hkv, d]; out bf16 [Tq, Hq, d], lse float32 [Hq, Tq] or None."""
    lib = load_library()
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError("%s must be a uint8 GPU tensor [T, H, d] with contiguous heads" % n)
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous float32 GPU tensor" % n)
    if out.dtype != torch.bfloat16 or out.dim() != 3 or out.stride(2) != 1 or out.stride(1) != out.shape[2]:
        raise ValueError("out must be bfloat16 [Tq, Hq, d] with contiguous heads")
    _int32_dev(cu_seqlens_q, "cu_seqlens_q")
    _int32_dev(cu_seqlens_k, "cu_seqlens_k")
    _dense_shapes(q, k, v, out)
    _shape(q_scale, q.shape[:2], "q_scale")
    _shape(k_scale, (k.shape[1],), "k_scale")
    _shape(v_scale, (v.shape[1], v.shape[2]), "v_scale")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same number of entries")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (q.shape[1], q.shape[0])):
        raise ValueError("lse must be contiguous float32 [Hq, Tq]")
    _on_device(q.device, ("q_scale", q_scale), ("k", k), ("k_scale", k_scale), ("v", v), ("v_scale", v_scale),
               ("out", out), ("lse", lse), ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k))
    if max_seqlen_q is None or max_seqlen_k is None:
        cq = cu_seqlens_q.cpu()
        ck = cu_seqlens_k.cpu()
        max_seqlen_q = int((cq[1:] - cq[:-1]).max()) if cq.numel() > 1 else 0
        max_seqlen_k = int((ck[1:] - ck[:-1]).max()) if ck.numel() > 1 else 0
    st = lib.vea_attn_fwd_fp8(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(q_scale),
                              _ptr(k_scale), _ptr(v_scale), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                              cu_seqlens_q.numel() - 1, q.shape[0], k.shape[0], int(max_seqlen_q),
                              int(max_seqlen_k), q.shape[1], k.shape[1], q.shape[2], int(bool(causal)), float(scale),
                              int(piece_rows), _ptr(out), out.stride(0), _ptr(lse), _stream(q))
    _check(st)
    return out, lse


def rope_cos_sin(positions, head_dim, theta, out=None):
    """Per-token rotation table float32 [T, head_dim/2, 2] of (cos, sin) for
    qkv_proj_rope (see vea_rope_cos_sin); positions int32 [T] or [T, 2]."""
    lib = load_library()
    torch = _torch()
    _int32_dev(positions, "positions")
    t = positions.shape[0]
    if out is None:
        out = torch.empty((t, head_dim // 2, 2), dtype=torch.float32, device=positions.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (t, head_dim // 2, 2):
        raise ValueError("out must be a contiguous float32 [T, head_dim/2, 2] tensor")
    _check(lib.vea_rope_cos_sin(_ptr(positions), positions.dim(), t, int(head_dim), float(theta), _ptr(out),
                                _stream(positions)))
    return out


def qkv_proj_rope(x, w, bias, cos_sin, q, k, v, rotate_half_span=0):
    """q, k, v = split(x @ w (+ bias)) with Q and K rotated by the table
    cos_sin (None: not rotated); see vea_qkv_proj_rope.  x [T, hidden] and
    w [hidden, (Hq + 2 Hkv) d] bf16 with contiguous rows; q [T, Hq, d],
    k and v [T, Hkv, d] contiguous bf16 outputs."""
    lib = load_library()
    torch = _torch()
    for t, n in ((x, "x"), (w, "w"), (q, "q"), (k, "k"), (v, "v")) + (((bias, "bias"),) if bias is not None else ()):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("%s must be a bfloat16 GPU tensor" % n)
    if x.dim() != 2 or x.stride(1) != 1 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("x and w must be 2-D with contiguous rows")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k and v outputs must be contiguous")
    if bias is not None and not bias.is_contiguous():
        raise ValueError("bias must be contiguous")
    if cos_sin is not None and (cos_sin.dtype != torch.float32 or not cos_sin.is_contiguous()):
        raise ValueError("cos_sin must be a contiguous float32 table")
    t, hidden = x.shape
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be [T, heads, d]")
    d = q.shape[2]
    n = (q.shape[1] + 2 * k.shape[1]) * d
    _shape(q, (t, q.shape[1], d), "q")
    _shape(k, (t, k.shape[1], d), "k")
    _shape(v, k.shape, "v")
    _shape(w, (hidden, n), "w")
    if bias is not None:
        _shape(bias, (n,), "bias")
    if cos_sin is not None:
        _shape(cos_sin, (t, d // 2, 2), "cos_sin")
    _on_device(x.device, ("w", w), ("bias", bias), ("cos_sin", cos_sin), ("q", q), ("k", k), ("v", v))
    st = lib.vea_qkv_proj_rope(_ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(bias), _ptr(cos_sin), x.shape[0],
                               x.shape[1], q.shape[1], k.shape[1], q.shape[2], int(rotate_half_span), _ptr(q), _ptr(k),
                               _ptr(v), _stream(x))
    _check(st)
    return q, k, v


def _sparse_shapes(q, kv, out, kvname):
    """q [R, H, d_qk], kv [rows, d_qk], out [R, H, d_v]."""
    if q.dim() != 3 or kv.dim() != 2 or out.dim() != 3:
        raise ValueError("q and out must be [rows, heads, dim] and %s [rows, d_qk]" % kvname)
    if kv.shape[1] != q.shape[2]:
        raise ValueError("%s rows must hold q's d_qk = %d values" % (kvname, q.shape[2]))
    if out.shape[:2] != q.shape[:2]:
        raise ValueError("out must have q's rows and heads %s" % (tuple(q.shape[:2]),))


def sparse_mqa_workspace_size(rows, heads, d_qk, d_v, k) -> int:
    """Workspace bytes vea_sparse_mqa_fwd uses for these sizes on the current
    device (0: no split)."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.vea_sparse_mqa_workspace_size(int(rows), int(heads), int(d_qk), int(d_v), int(k), ctypes.byref(n)))
    return int(n.value)


def sparse_mqa_fwd(q, kv_latent, topk_idx, k, scale, out, lse=None, workspace="auto"):
    """Top-k sparse MQA (see vea_sparse_mqa_fwd): q [R, H, d_qk], kv_latent
    [n_kv, d_qk], topk_idx int32 [R, k], out [R, H, d_v], lse [H, R] or None.

    workspace: "auto" allocates the size the call asks for (split of the last
    round of workgroups), None runs every row alone (batch-invariant bits), or
    a contiguous uint8 GPU tensor to use."""
    lib = load_library()
    torch = _torch()
    for t, n in ((q, "q"), (kv_latent, "kv_latent"), (out, "out")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous bfloat16 GPU tensor" % n)
    _int32_dev(topk_idx, "topk_idx")
    _sparse_shapes(q, kv_latent, out, "kv_latent")
    _on_device(q.device, ("kv_latent", kv_latent), ("topk_idx", topk_idx), ("out", out), ("lse", lse),
               ("workspace", None if isinstance(workspace, str) else workspace))
    if topk_idx.shape != (q.shape[0], k):
        raise ValueError("topk_idx must be [rows, k]")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0])
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32 [heads, rows]")
    with torch.cuda.device(q.device):
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a uint8 GPU tensor')
            nbytes = sparse_mqa_workspace_size(q.shape[0], q.shape[1], q.shape[2], out.shape[2], k)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
        if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()
                                      or workspace.device != q.device):
            raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
        st = lib.vea_sparse_mqa_fwd(_ptr(q), _ptr(kv_latent), _ptr(topk_idx), q.shape[0], q.shape[1],
                                    kv_latent.shape[0], q.shape[2], out.shape[2], int(k), float(scale), _ptr(out),
                                    _ptr(lse), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                    _stream(q))
    _check(st)
    return out, lse


def sparse_mqa_paged_fwd(q, kv_cache, page_table, page_size, n_kv, topk_idx, k, scale, out, lse=None,
                         workspace="auto"):
    """Top-k sparse MQA over a paged latent cache (see vea_sparse_mqa_paged_fwd):
    kv_cache [num_pages * page_size, d_qk] bf16, page_table int32
    [ceil(n_kv / page_size)], topk_idx int32 [R, k] of logical positions."""
    lib = load_library()
    torch = _torch()
    for t, n in ((q, "q"), (kv_cache, "kv_cache"), (out, "out")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous bfloat16 GPU tensor" % n)
    _int32_dev(topk_idx, "topk_idx")
    _int32_dev(page_table, "page_table")
    _sparse_shapes(q, kv_cache, out, "kv_cache")
    _on_device(q.device, ("kv_cache", kv_cache), ("page_table", page_table), ("topk_idx", topk_idx), ("out", out),
               ("lse", lse), ("workspace", None if isinstance(workspace, str) else workspace))
    page_size = int(page_size)
    if page_size < 1 or kv_cache.shape[0] % page_size:
        raise ValueError("kv_cache rows must be a multiple of page_size")
    if page_table.numel() < -(-int(n_kv) // page_size):
        raise ValueError("page_table needs ceil(n_kv / page_size) entries")
    if topk_idx.shape != (q.shape[0], k):
        raise ValueError("topk_idx must be [rows, k]")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0])
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32 [heads, rows]")
    with torch.cuda.device(q.device):
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a uint8 GPU tensor')
            nbytes = sparse_mqa_workspace_size(q.shape[0], q.shape[1], q.shape[2], out.shape[2], k)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
        st = lib.vea_sparse_mqa_paged_fwd(_ptr(q), _ptr(kv_cache), _ptr(page_table), page_size,
                                          kv_cache.shape[0] // page_size, _ptr(topk_idx), q.shape[0], q.shape[1],
                                          int(n_kv), q.shape[2], out.shape[2], int(k), float(scale), _ptr(out),
                                          _ptr(lse), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                          _stream(q))
    _check(st)
    return out, lse


def topk_indices(logits, k, out, row_starts=None, row_lens=None):
    """Deterministic top-k positions per row (see vea_topk_indices): logits
    float32 [R, n] with contiguous columns, out int32 [R, k] contiguous,
    row_starts / row_lens int32 [R] or None."""
    lib = load_library()
    torch = _torch()
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
        raise ValueError("logits must be a float32 GPU tensor [rows, n] with contiguous columns")
    if out.dtype != torch.int32 or not out.is_contiguous() or tuple(out.shape) != (logits.shape[0], int(k)):
        raise ValueError("out must be contiguous int32 [rows, k]")
    for t, nm in ((row_starts, "row_starts"), (row_lens, "row_lens")):
        if t is not None:
            _int32_dev(t, nm)
            if t.numel() != logits.shape[0]:
                raise ValueError("%s must have one entry per row" % nm)
    _on_device(logits.device, ("out", out), ("row_starts", row_starts), ("row_lens", row_lens))
    st = lib.vea_topk_indices(_ptr(logits), logits.stride(0), _ptr(row_starts), _ptr(row_lens), logits.shape[0],
                              logits.shape[1], int(k), _ptr(out), _stream(logits))
    _check(st)
    return out


def attn_probs_piece(q, k, lse, head, seq_begin_q, len_q, seq_begin_k, len_k, q0, rows, causal, scale, p_out):
    """Debug export of P for one piece of one head into p_out [rows, >= len_k]
    (see vea_attn_probs_piece)."""
    lib = load_library()
    qs, ks = _token_major(q, "q"), _token_major(k, "k")
    if p_out.stride(1) != 1:
        raise ValueError("p_out rows must be contiguous")
    if int(seq_begin_q) + int(len_q) > q.shape[0] or int(seq_begin_k) + int(len_k) > k.shape[0]:
        raise ValueError("the piece's sequence lies past q's or k's rows")
    if p_out.dim() != 2 or p_out.shape[0] < int(rows) or p_out.shape[1] < int(len_k):
        raise ValueError("p_out must hold rows x len_k values")
    if lse.dim() != 2 or lse.shape[0] != q.shape[1] or lse.stride(1) != 1:
        raise ValueError("lse must be the float32 [Hq, total_q] output of attn_fwd")
    _on_device(q.device, ("k", k), ("lse", lse), ("p_out", p_out))
    st = lib.vea_attn_probs_piece(_dtype_code(q), _ptr(q), qs, _ptr(k), ks, _ptr(lse), lse.stride(0), int(head),
                                  q.shape[1], k.shape[1], q.shape[2], int(seq_begin_q), int(len_q),
                                  int(seq_begin_k), int(len_k), int(q0), int(rows), 1 if causal else 0,
                                  float(scale), _ptr(p_out), p_out.stride(0), _stream(q))
    _check(st)
    return p_out
