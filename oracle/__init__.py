"""CPU float64 oracle for the tiled-attention library — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP path never calls it, and it
imports nothing from the HIP path: the two share no code.  Inputs come from
``vision_encoder_attention_amd.workloads`` (random draws only) or from the
caller.

What it computes is the plain definition of each operation, in float64:

* ``attention``      softmax(scale * Q K^T + mask) V per sequence and head,
                     with the per-row log-sum-exp (two-pass softmax: row max,
                     then sum).  The pages compute this blockwise with an
                     online softmax, which reaches the same value in exact
                     arithmetic (merge identity of
                     「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」,
                     section 进一步探索, eq. (1)(2)).
* ``attention_paged`` the same over paged K/V caches (block tables).
* ``attn_probs``     the probability matrix P of one query piece.
* ``rope_*`` / ``qkv_rope``  rotary position embedding on the Q and K heads
                     of a fused QKV projection output (1D and 2D grid).
* ``qkv_proj`` / ``qkv_proj_rope``  the fused QKV projection (x w + b) and
                     its split into Q, K (rotated) and V; ``rope_cos_sin``
                     the per-token rotation table.
* ``e4m3_*`` / ``quantize_fp8`` / ``attention_fp8``  OCP FP8 E4M3 coding,
                     block quantisation and attention on quantised inputs.
* ``sparse_mqa``     multi-query attention over a per-row set of latent rows;
                     ``sparse_mqa_paged`` the same over a paged cache.
* ``topk_indices``   deterministic top-k selection of the sparse indexer
                     (ties go to the lower position).
* ``paged_rows``     logical position -> physical row of a paged cache.
* ``pieces``         query-piece arithmetic of the vision encoder.

Every function says which passage it follows.  Page titles used below:

* [3090]   「DeepSeek V4.1 上 4×RTX 3090：视觉链路的两个坑和修复」
* [MI250]  「AMD MI250部署DeepSeek-V4-Flash：先修正确性再谈性能」
* [SGLang] 「从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash - Prefill」
* [V32]    「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」

Parity pins (tests/test_oracle_*.py) tie each function to closed forms,
brute force, independent library implementations and invariants.
"""
from .attention import attention, attention_paged, attn_probs  # noqa: F401
from .rope import rope_1d, rope_2d, qkv_rope, rope_inv_freq  # noqa: F401
from .paging import paged_rows  # noqa: F401
from .sparse import sparse_mqa, sparse_mqa_paged  # noqa: F401
from .pieces import piece_ranges, piece_rows_for_capacity  # noqa: F401
from .topk import topk_indices  # noqa: F401
from .qkv_proj import qkv_proj, qkv_proj_rope, rope_cos_sin  # noqa: F401
from .fp8 import attention_fp8, e4m3_decode, e4m3_encode, e4m3_values, quantize_fp8  # noqa: F401
