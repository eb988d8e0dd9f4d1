"""MI355X-native (gfx950) tiled attention forward.

The computation lives in hand-written HIP kernels inside ``libvea.so`` (C ABI
in ``include/vea.h``); this package is a thin binding over it:

* ``attn_fwd``        blockwise SDPA forward over a cu_seqlens-packed batch,
                      causal or not, GQA, query pieces, fp32 online softmax;
* ``qkv_rope``        fused QKV output split + 1D / 2D-grid RoPE;
* ``sparse_mqa_fwd``  top-k sparse MQA over a shared latent KV;
* ``topk_indices``    deterministic top-k positions per row (the sparse indexer);
* ``quantize_fp8`` / ``attn_fwd_fp8``  block quantisation to FP8 E4M3 and
                      attention on the quantised q, k, v (FP8 MFMA);
* ``qkv_proj_rope``   fused QKV projection GEMM with the RoPE rotation in its
                      epilogue; ``rope_cos_sin`` builds its per-token table;
* ``attn_probs_piece`` debug export of one piece's probabilities.

``workloads`` holds the seeded synthetic inputs; ``build`` compiles the library.
"""
from ._binding import (VeaError, attn_decode, attn_decode_workspace_size, attn_fwd, attn_fwd_noalloc, attn_fwd_paged, attn_fwd_workspace_size, attn_probs_piece, lib_path, load_library,  # noqa: F401
                       attn_fwd_fp8, quantize_fp8, qkv_proj_rope, qkv_rope, rope_cos_sin, sparse_mqa_fwd, sparse_mqa_paged_fwd,
                       sparse_mqa_workspace_size, status_str, topk_indices)

__all__ = ["attn_decode", "attn_decode_workspace_size", "attn_fwd", "attn_fwd_noalloc", "attn_fwd_paged", "attn_fwd_workspace_size", "qkv_rope", "sparse_mqa_fwd", "sparse_mqa_workspace_size", "attn_probs_piece",
           "sparse_mqa_paged_fwd", "topk_indices", "qkv_proj_rope", "rope_cos_sin", "quantize_fp8", "attn_fwd_fp8", "VeaError", "load_library",
           "lib_path", "status_str"]
