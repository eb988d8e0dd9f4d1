"""Seeded synthetic inputs for the tiled-attention library and its checks.

This module only draws random numbers and lays them out in the shapes of the
workloads the source pages describe.  It holds none of the attention, RoPE or
softmax arithmetic: both the HIP path (through the Python binding) and the CPU
oracle consume what it produces, and nothing here is shared with either
computation.

Workload shapes and where they come from:

* vision: one 1554x1078 image cut into 14-px patches gives a 111-column by
  77-row grid, 8547 tokens, attention run in query pieces of 1462 rows
  ("DeepSeek V4.1 上 4×RTX 3090：视觉链路的两个坑和修复", section 三).
* varlen prefill: a packed batch addressed by cu_seqlens
  ("从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash - Prefill", sections 2.2
  and 3.2).
* sparse MQA: 323 query rows selecting 2048 of 2590 positions (the top-k and
  logits shapes printed in "推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起",
  section 修改topk结果).

Random values are float32 N(0, 1) from ``numpy.random.default_rng(seed)``,
rounded to bfloat16 with round-to-nearest-even.  bfloat16 tensors are carried
as their raw uint16 bit patterns so that the exact same values reach both the
GPU and the float64 oracle (bf16 -> float32 -> float64 is exact).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

# ----------------------------------------------------------------------------
# bfloat16 bit handling (input preparation only)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs here are finite N(0,1) draws;
    NaN is kept quiet for completeness.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    return bf16_bits_to_f32(b).astype(np.float64)


def randn_bf16_bits(rng: np.random.Generator, shape, mul: float = 1.0) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16; ``mul`` (a power of two) is applied
    after rounding, which keeps it exact."""
    bits = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    if mul != 1.0:
        m, e = math.frexp(mul)
        if m != 0.5:
            raise ValueError("mul must be a power of two so scaling stays exact")
        bits = f32_to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(mul))
    return bits


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class DenseCase:
    """A dense attention call (optionally preceded by the fused QKV + RoPE step).

    Tensors are numpy arrays; bf16 ones are uint16 bit patterns.
    """
    name: str
    dtype: str                      # "bf16" or "f32"
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    causal: bool
    scale: float                    # passed to the kernel as float32
    piece_rows: int                 # query rows per piece; 0 = one piece per sequence
    cu_seqlens_q: np.ndarray        # int32 [B+1]
    cu_seqlens_k: np.ndarray        # int32 [B+1]
    q: Optional[np.ndarray] = None  # [total_q, Hq, d]
    k: Optional[np.ndarray] = None  # [total_k, Hkv, d]
    v: Optional[np.ndarray] = None  # [total_k, Hkv, d]
    # fused-projection form (qkv_rope prologue); when set, q/k/v come from it
    x_qkv: Optional[np.ndarray] = None      # [T, (Hq + 2 Hkv) d] bf16 bits
    positions: Optional[np.ndarray] = None  # int32 [T] or [T, 2]
    theta: float = 10000.0

    @property
    def batch(self) -> int:
        return len(self.cu_seqlens_q) - 1

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_seqlens_k[-1])

    @property
    def seqlens_q(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)

    @property
    def seqlens_k(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_k)

    def v_from_x(self) -> np.ndarray:
        """V heads read in place from the fused projection (columns after Q|K)."""
        assert self.x_qkv is not None
        hq, hkv, d = self.num_heads_q, self.num_heads_kv, self.head_dim
        t = self.x_qkv.shape[0]
        return self.x_qkv[:, (hq + hkv) * d:].reshape(t, hkv, d)


@dataclasses.dataclass
class SparseCase:
    name: str
    q: np.ndarray          # [R, H, d_qk] bf16 bits
    kv_latent: np.ndarray  # [n_kv, d_qk] bf16 bits
    topk_idx: np.ndarray   # int32 [R, k]
    d_v: int
    scale: float

    @property
    def num_rows(self) -> int:
        return self.q.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def d_qk(self) -> int:
        return self.q.shape[2]

    @property
    def n_kv(self) -> int:
        return self.kv_latent.shape[0]

    @property
    def k(self) -> int:
        return self.topk_idx.shape[1]


def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def grid_positions(rows: int, cols: int) -> np.ndarray:
    """(row, col) of each token of a row-major patch grid: int32 [rows*cols, 2]."""
    t = np.arange(rows * cols, dtype=np.int64)
    return np.stack([t // cols, t % cols], axis=1).astype(np.int32)


def seq_positions(lengths) -> np.ndarray:
    """Positions 0..L-1 restarting at each packed sequence: int32 [sum L]."""
    return np.concatenate([np.arange(int(n), dtype=np.int32) for n in lengths]) if len(lengths) else \
        np.zeros((0,), np.int32)


# ---------------------------------------------------------------- dense cases

def single_head_f32(n: int = 256, d: int = 64, piece_rows: int = 64, seed: int = 1) -> DenseCase:
    """Single-head, non-causal fp32 attention, q/k/v ~ N(0,1), scale 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, 1, d), dtype=np.float32)
    k = rng.standard_normal((n, 1, d), dtype=np.float32)
    v = rng.standard_normal((n, 1, d), dtype=np.float32)
    cu = _cu([n])
    return DenseCase("single_head_f32_n%d_d%d" % (n, d), "f32", 1, 1, d, False, 1.0 / math.sqrt(d),
                     piece_rows, cu, cu.copy(), q, k, v)


def vision(grid_rows: int = 77, grid_cols: int = 111, heads: int = 16, d: int = 64,
           piece_rows: int = 1462, seed: int = 2, theta: float = 10000.0) -> DenseCase:
    """One image as a patch grid; fused QKV output with 2D-grid RoPE, non-causal."""
    rng = np.random.default_rng(seed)
    t = grid_rows * grid_cols
    x = randn_bf16_bits(rng, (t, 3 * heads * d))
    cu = _cu([t])
    return DenseCase("vision_%dtok_h%d_d%d_qb%d" % (t, heads, d, piece_rows), "bf16", heads, heads, d,
                     False, 1.0 / math.sqrt(d), piece_rows, cu, cu.copy(),
                     x_qkv=x, positions=grid_positions(grid_rows, grid_cols), theta=theta)


def varlen_gqa(lengths=None, n_seqs: int = 8, lo: int = 512, hi: int = 8192, hq: int = 32, hkv: int = 8,
               d: int = 128, seed: int = 3, theta: float = 10000.0, piece_rows: int = 0) -> DenseCase:
    """Packed causal prefill batch; lengths uniform in [lo, hi] unless given; 1D RoPE."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(lo, hi, size=n_seqs, endpoint=True)
    lengths = [int(n) for n in lengths]
    t = sum(lengths)
    x = randn_bf16_bits(rng, (t, (hq + 2 * hkv) * d))
    cu = _cu(lengths)
    return DenseCase("varlen_gqa_b%d_tok%d_h%d-%d_d%d" % (len(lengths), t, hq, hkv, d), "bf16", hq, hkv, d,
                     True, 1.0 / math.sqrt(d), piece_rows, cu, cu.copy(),
                     x_qkv=x, positions=seq_positions(lengths), theta=theta)


def long_causal(n: int = 32768, heads: int = 16, d: int = 128, q_mul: float = 4.0, seed: int = 4,
                piece_rows: int = 0) -> DenseCase:
    """One long causal sequence; q is 4x N(0,1) so that logits are peaked."""
    rng = np.random.default_rng(seed)
    q = randn_bf16_bits(rng, (n, heads, d), mul=q_mul)
    k = randn_bf16_bits(rng, (n, heads, d))
    v = randn_bf16_bits(rng, (n, heads, d))
    cu = _cu([n])
    return DenseCase("long_causal_%d_h%d_d%d" % (n, heads, d), "bf16", heads, heads, d, True,
                     1.0 / math.sqrt(d), piece_rows, cu, cu.copy(), q, k, v)


def random_dense(lengths_q, lengths_k, hq: int, hkv: int, d: int, causal: bool, dtype: str = "bf16",
                 seed: int = 0, piece_rows: int = 0, scale: Optional[float] = None,
                 q_mul: float = 1.0) -> DenseCase:
    """General packed dense case with independent q/k/v (used for edge cases)."""
    rng = np.random.default_rng(seed)
    tq, tk = int(sum(lengths_q)), int(sum(lengths_k))
    if dtype == "bf16":
        q = randn_bf16_bits(rng, (tq, hq, d), mul=q_mul)
        k = randn_bf16_bits(rng, (tk, hkv, d))
        v = randn_bf16_bits(rng, (tk, hkv, d))
    else:
        q = rng.standard_normal((tq, hq, d), dtype=np.float32) * np.float32(q_mul)
        k = rng.standard_normal((tk, hkv, d), dtype=np.float32)
        v = rng.standard_normal((tk, hkv, d), dtype=np.float32)
    return DenseCase("random_dense_seed%d" % seed, dtype, hq, hkv, d, causal,
                     (1.0 / math.sqrt(d)) if scale is None else scale, piece_rows,
                     _cu(lengths_q), _cu(lengths_k), q, k, v)


# --------------------------------------------------------------- sparse case

def decode(batch: int = 64, lo: int = 512, hi: int = 8192, hq: int = 32, hkv: int = 8, d: int = 128,
           seed: int = 70) -> DenseCase:
    """Decode step: one new query token per sequence over cached keys of
    lengths drawn uniformly in [lo, hi] (GQA 32/8, d 128 as the varlen
    batch); causal with one query row = every cached key visible."""
    rng = np.random.default_rng(seed)
    lk = [int(x) for x in rng.integers(lo, hi + 1, batch)]
    c = random_dense([1] * batch, lk, hq, hkv, d, True, "bf16", seed=seed + 1)
    c.name = "decode_b%d_kv%d_h%d-%d_d%d" % (batch, sum(lk), hq, hkv, d)
    return c


def sparse_mqa(rows: int = 323, heads: int = 128, n_kv: int = 2590, d_qk: int = 576, d_v: int = 512,
               k: int = 2048, seed: int = 5, valid_offset: Optional[int] = None) -> SparseCase:
    """Top-k sparse MQA over a shared latent KV.

    Row r is the (n_kv - rows + r)-th position; it selects ``k`` distinct indices
    uniformly without replacement from its causally visible positions
    [0, n_kv - rows + r + 1) (at least ``k`` of them), in shuffled order.
    """
    rng = np.random.default_rng(seed)
    q = randn_bf16_bits(rng, (rows, heads, d_qk))
    kv = randn_bf16_bits(rng, (n_kv, d_qk))
    base = (n_kv - rows + 1) if valid_offset is None else valid_offset
    idx = np.empty((rows, k), dtype=np.int32)
    for r in range(rows):
        n_valid = min(n_kv, base + r)
        if n_valid < k:
            raise ValueError("row %d has only %d visible positions for k=%d" % (r, n_valid, k))
        idx[r] = rng.permutation(n_valid)[:k]
    return SparseCase("sparse_mqa_r%d_h%d_kv%d_k%d" % (rows, heads, n_kv, k), q, kv, idx, d_v,
                      1.0 / math.sqrt(d_qk))


def permute_rows(idx: np.ndarray, seed: int) -> np.ndarray:
    """Each row of an index matrix independently shuffled."""
    rng = np.random.default_rng(seed)
    out = idx.copy()
    for r in range(out.shape[0]):
        out[r] = out[r, rng.permutation(out.shape[1])]
    return out


# ------------------------------------------------------- named workloads

@dataclasses.dataclass
class IndexerCase:
    """Top-k selection over indexer logits."""
    name: str
    logits: np.ndarray              # [R, n] float32
    k: int
    row_starts: Optional[np.ndarray]  # [R] int32 or None
    row_lens: Optional[np.ndarray]    # [R] int32 or None


def indexer(rows: int = 323, n: int = 2590, k: int = 2048, grid: float = 1.0 / 16, seed: int = 6) -> IndexerCase:
    """Logits of the sparse indexer's top-k: rows [323, 2590] fp32, the
    last `rows` of n positions, row r seeing positions [0, n - rows + r + 1)
    (at least k of them).  Values are N(0,1) rounded to a grid of `grid`, so
    equal scores are common and fall at the edge of the selection, the case
    that made an unstable top-k disagree with itself."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n), dtype=np.float32)
    if grid:
        x = (np.round(x / grid) * grid).astype(np.float32)
    lens = np.minimum(n - rows + 1 + np.arange(rows), n).astype(np.int32)
    if lens.min() < k:
        raise ValueError("a row sees fewer than k positions")
    return IndexerCase("indexer_r%d_n%d_k%d" % (rows, n, k), x, k, None, lens)


@dataclasses.dataclass
class ProjCase:
    """Fused QKV projection + RoPE: x [T, hidden] and the fused weight
    [hidden, (Hq + 2 Hkv) d] as bf16 bits, optional bias [N] bf16 bits."""
    name: str
    x: np.ndarray                   # uint16 [T, hidden]
    w: np.ndarray                   # uint16 [hidden, N]
    bias: Optional[np.ndarray]      # uint16 [N] or None
    positions: np.ndarray           # int32 [T] or [T, 2]
    hq: int
    hkv: int
    d: int
    theta: float


def qkv_proj(tokens: int = 0, hidden: int = 1024, hq: int = 16, hkv: int = 16, d: int = 64, grid=(77, 111),
             lengths=None, bias: bool = False, seed: int = 7, theta: float = 10000.0) -> ProjCase:
    """x ~ N(0, 1), w ~ N(0, 1) / sqrt(hidden) (rounded to a power of two;
    outputs ~ N(0, 1)), bias ~
    N(0, 1) when asked.  Positions: the patch grid `grid` (2D) when given,
    else per-sequence positions of `lengths` (1D), else 0 .. tokens - 1."""
    rng = np.random.default_rng(seed)
    if grid is not None:
        positions = grid_positions(*grid)
    elif lengths is not None:
        positions = seq_positions(lengths)
    else:
        positions = np.arange(tokens, dtype=np.int32)
    t = positions.shape[0]
    n = (hq + 2 * hkv) * d
    x = randn_bf16_bits(rng, (t, hidden))
    w = randn_bf16_bits(rng, (hidden, n), mul=2.0 ** -round(math.log2(math.sqrt(hidden))))
    b = randn_bf16_bits(rng, (n,)) if bias else None
    return ProjCase("qkv_proj_tok%d_hid%d_h%d-%d_d%d" % (t, hidden, hq, hkv, d), x, w, b, positions, hq, hkv, d,
                    theta)


def vision_proj(seed: int = 7) -> ProjCase:
    """The vision encoder's projection before qkv_rope: 8547 grid tokens,
    hidden 1024 = 16 heads x 64, 2D positions."""
    return qkv_proj(hidden=1024, hq=16, hkv=16, d=64, grid=(77, 111), seed=seed)


def varlen_proj(seed: int = 8) -> ProjCase:
    """The varlen prefill batch's projection: the same 8 sequence lengths as
    varlen_gqa (32876 tokens), hidden 4096 = 32 heads x 128, GQA 32/8, 1D."""
    rng = np.random.default_rng(3)
    lengths = [int(n) for n in rng.integers(512, 8192, size=8, endpoint=True)]
    return qkv_proj(hidden=4096, hq=32, hkv=8, d=128, grid=None, lengths=lengths, seed=seed)


FULL_CASES = ("single_head_f32", "vision", "varlen_gqa", "long_causal", "sparse_mqa")


def full_case(name: str):
    """The five full-size workloads, by name."""
    return {
        "single_head_f32": single_head_f32,
        "vision": vision,
        "varlen_gqa": varlen_gqa,
        "long_causal": long_causal,
        "sparse_mqa": sparse_mqa,
    }[name]()


def small_cases() -> List:
    """Reduced versions the oracle finishes in seconds; each still spans
    several tiles, several pieces and a ragged tail."""
    return [
        single_head_f32(),
        vision(grid_rows=23, grid_cols=29, heads=4, d=64, piece_rows=150, seed=12),
        varlen_gqa(lengths=[130, 1, 257, 0, 700], hq=8, hkv=2, d=128, seed=13),
        long_causal(n=1500, heads=2, d=128, seed=14),
        sparse_mqa(rows=9, heads=128, n_kv=700, k=256, seed=15),
    ]
