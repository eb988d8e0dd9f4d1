"""Stage a seeded workload on the GPU and run the HIP path on it.

Glue only: allocates device tensors with torch (memory and streams are all
torch is used for), copies the generator's exact bf16 bit patterns over, and
calls the binding.  Used by the tests, ``bench.py`` and ``smoke()``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import _binding as B
from .workloads import DenseCase, ProjCase, SparseCase


def _torch():
    import torch
    return torch


def bits_to_tensor(bits: np.ndarray, device) -> "torch.Tensor":
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on ``device`` (exact)."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def tensor_to_bits(t) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 bit patterns on the host."""
    torch = _torch()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _dev_i32(a: np.ndarray, device):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


@dataclasses.dataclass
class DenseStaged:
    case: DenseCase
    q: "torch.Tensor"
    k: "torch.Tensor"
    v: "torch.Tensor"
    cu_q: "torch.Tensor"
    cu_k: "torch.Tensor"
    out: "torch.Tensor"
    lse: "torch.Tensor"
    x_qkv: Optional["torch.Tensor"] = None
    positions: Optional["torch.Tensor"] = None
    max_q: int = 0
    max_k: int = 0
    split: bool = True                 # let attn_fwd split the last round (workspace)
    ws: Optional["torch.Tensor"] = None


def stage_dense(case: DenseCase, device="cuda", split: bool = True) -> DenseStaged:
    """Copy a dense case to the device and allocate its outputs (and the
    attention workspace, when the call would use one and split is set).

    For cases with a fused QKV buffer, q/k are the (not yet computed) outputs
    of qkv_rope and v is a strided view into the fused buffer.
    """
    torch = _torch()
    hq, hkv, d = case.num_heads_q, case.num_heads_kv, case.head_dim
    x = pos = None
    if case.x_qkv is not None:
        x = bits_to_tensor(case.x_qkv, device)
        pos = _dev_i32(case.positions, device)
        t = x.shape[0]
        q = torch.empty((t, hq, d), dtype=torch.bfloat16, device=device)
        k = torch.empty((t, hkv, d), dtype=torch.bfloat16, device=device)
        v = x[:, (hq + hkv) * d:(hq + 2 * hkv) * d].view(t, hkv, d)
    elif case.dtype == "bf16":
        q, k, v = (bits_to_tensor(a, device) for a in (case.q, case.k, case.v))
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device) for a in (case.q, case.k, case.v))
    out = torch.empty((case.total_q, hq, d), dtype=q.dtype, device=device)
    lse = torch.empty((hq, case.total_q), dtype=torch.float32, device=device)
    lq = case.seqlens_q
    lk = case.seqlens_k
    st = DenseStaged(case, q, k, v, _dev_i32(case.cu_seqlens_q, device), _dev_i32(case.cu_seqlens_k, device),
                     out, lse, x, pos, int(lq.max()) if lq.size else 0, int(lk.max()) if lk.size else 0, split)
    if split:
        with torch.cuda.device(q.device):
            n = B.attn_fwd_workspace_size(B.VEA_BF16 if case.dtype == "bf16" else B.VEA_F32, len(lq),
                                          case.total_q, case.total_k, st.max_q, st.max_k, hq, hkv, d,
                                          case.causal, case.piece_rows)
        if n:
            st.ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    return st


def run_rope(st: DenseStaged):
    """qkv_rope step of a fused-QKV case (writes st.q, st.k)."""
    if st.x_qkv is not None:
        B.qkv_rope(st.x_qkv, st.positions, st.case.theta, st.q, st.k)


def run_attn(st: DenseStaged, piece_rows: Optional[int] = None, lse: bool = True):
    """attn_fwd step (writes st.out and st.lse)."""
    c = st.case
    if not st.split:
        ws = None
    elif piece_rows is None or piece_rows == c.piece_rows:
        ws = st.ws                                          # sized for the case's own pieces
    else:
        ws = "auto"
    B.attn_fwd(st.q, st.k, st.v, st.cu_q, st.cu_k, c.causal, c.scale, st.out, st.lse if lse else None,
               piece_rows=c.piece_rows if piece_rows is None else piece_rows,
               max_seqlen_q=st.max_q, max_seqlen_k=st.max_k, workspace=ws)


def run_dense(st: DenseStaged, piece_rows: Optional[int] = None):
    """One pass of the dense path: qkv_rope (if fused) then attn_fwd."""
    run_rope(st)
    run_attn(st, piece_rows)
    return st.out, st.lse


@dataclasses.dataclass
class SparseStaged:
    case: SparseCase
    q: "torch.Tensor"
    kv: "torch.Tensor"
    idx: "torch.Tensor"
    out: "torch.Tensor"
    lse: "torch.Tensor"
    ws: Optional["torch.Tensor"]       # split workspace, None: every row alone


def stage_sparse(case: SparseCase, device="cuda", idx: Optional[np.ndarray] = None,
                 split: bool = True) -> SparseStaged:
    torch = _torch()
    q = bits_to_tensor(case.q, device)
    kv = bits_to_tensor(case.kv_latent, device)
    ix = _dev_i32(case.topk_idx if idx is None else idx, device)
    out = torch.empty((case.num_rows, case.num_heads, case.d_v), dtype=torch.bfloat16, device=device)
    lse = torch.empty((case.num_heads, case.num_rows), dtype=torch.float32, device=device)
    ws = None
    if split:
        with torch.cuda.device(q.device):
            n = B.sparse_mqa_workspace_size(case.num_rows, case.num_heads, case.d_qk, case.d_v, ix.shape[1])
        if n:
            ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    return SparseStaged(case, q, kv, ix, out, lse, ws)


def run_sparse(st: SparseStaged):
    c = st.case
    B.sparse_mqa_fwd(st.q, st.kv, st.idx, st.idx.shape[1], c.scale, st.out, st.lse, workspace=st.ws)
    return st.out, st.lse


@dataclasses.dataclass
class ProjStaged:
    case: ProjCase
    x: "torch.Tensor"
    w: "torch.Tensor"
    bias: Optional["torch.Tensor"]
    positions: "torch.Tensor"
    cs: Optional["torch.Tensor"]       # rotation table, None: no rotation
    q: "torch.Tensor"
    k: "torch.Tensor"
    v: "torch.Tensor"


def stage_proj(case: ProjCase, device="cuda", rotate: bool = True) -> ProjStaged:
    torch = _torch()
    x = bits_to_tensor(case.x, device)
    w = bits_to_tensor(case.w, device)
    bias = None if case.bias is None else bits_to_tensor(case.bias, device)
    pos = _dev_i32(case.positions, device)
    t = x.shape[0]
    cs = torch.empty((t, case.d // 2, 2), dtype=torch.float32, device=device) if rotate else None
    q = torch.empty((t, case.hq, case.d), dtype=torch.bfloat16, device=device)
    k = torch.empty((t, case.hkv, case.d), dtype=torch.bfloat16, device=device)
    v = torch.empty((t, case.hkv, case.d), dtype=torch.bfloat16, device=device)
    return ProjStaged(case, x, w, bias, pos, cs, q, k, v)


def run_rope_table(st: ProjStaged):
    if st.cs is not None:
        B.rope_cos_sin(st.positions, st.case.d, st.case.theta, st.cs)
    return st.cs


def run_proj(st: ProjStaged):
    B.qkv_proj_rope(st.x, st.w, st.bias, st.cs, st.q, st.k, st.v)
    return st.q, st.k, st.v
