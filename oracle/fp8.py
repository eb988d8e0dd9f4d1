"""FP8 (e4m3) quantisation and attention on quantised inputs (float64).
Test infrastructure only.

The pages allow FP8 for matrix products whose inputs have a safe dynamic
range, keeping softmax statistics and accumulation in fp32 ([MI250] section
4.1), recommend block-wise quantisation to make FP8 pay ([MI250] section 5.3),
and note that the prefill attention kernel they trace runs part of its work in
FP8 ([SGLang] section 3.2).  The format is OCP FP8 E4M3 ("e4m3fn"): 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity; the largest
finite value is 448.

Quantisation of a block B of real values (a block is one (token, head) row,
one head, or one (head, channel) column, depending on the granularity):

    amax  = max |x| over B                    (exact: the inputs are bf16)
    scale = fp32(amax / 448),  inv = fp32(1 / scale)
                                              (both 1 when amax < 2^-64,
                                               which counts as an empty block)
    code  = e4m3 nearest-even of clamp(fp32(x * inv), -448, 448)

inv is derived from the stored scale, and the product x * inv is rounded to
fp32 before the rounding to e4m3: the integer code is decided from the same
fp32 values a kernel has, also when the scales are computed by one pass and
the codes by another.
The dequantised value is decode(code) * scale.

``attention_fp8`` is attention (oracle.attention) on the dequantised q, k and
v: q with one scale per (token, head), k with one per head, v with one per
(head, channel).
"""
from __future__ import annotations

import numpy as np

from oracle.attention import attention

__all__ = ["e4m3_values", "e4m3_decode", "e4m3_encode", "quantize_fp8", "attention_fp8", "E4M3_MAX"]

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7f and 0xff)."""
    v = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 0xF and m == 7:
            v[c] = np.nan
        elif e == 0:
            v[c] = s * m * 2.0 ** -9
        else:
            v[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


_VALUES = e4m3_values()
_POS = _VALUES[:0x7F]                        # codes 0x00 .. 0x7e: 0 .. 448, increasing


def e4m3_decode(codes) -> np.ndarray:
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y) -> np.ndarray:
    """Nearest e4m3 code to each real y with |y| <= 448, ties to the even
    code (even mantissa); the sign is kept (-0.0 and negative values that
    round to zero give 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values in [-448, 448]")
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def quantize_fp8(x, granularity: int):
    """x: real [T, H, d] (bf16 values).  granularity 0: one scale per (token,
    head), scales [T, H]; 1: one per head, scales [H]; 2: one per (head,
    channel), scales [H, d].  Returns (codes uint8 [T, H, d], scales float32)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 3:
        raise ValueError("x must be [tokens, heads, head_dim]")
    ax = {0: (2,), 1: (0, 2), 2: (0,)}[granularity]
    amax = np.abs(x).max(axis=ax, keepdims=True) if x.size else np.zeros((1, 1, 1), np.float32)
    zero = amax < np.float32(2.0 ** -64)
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = (np.float32(1) / scale).astype(np.float32)
    y = np.clip((x * inv).astype(np.float32), -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(y)
    return codes, np.squeeze(scale, axis=ax).astype(np.float32)


def dequantize(codes, scales, granularity: int) -> np.ndarray:
    v = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    if granularity == 0:
        return v * s[:, :, None]
    if granularity == 1:
        return v * s[None, :, None]
    return v * s[None, :, :]


def attention_fp8(q8, q_scale, k8, k_scale, v8, v_scale, cu_seqlens_q, cu_seqlens_k, causal: bool, scale: float,
                  rows=None, heads=None):
    """Attention on dequantised inputs: q8 [Tq, Hq, d] with q_scale [Tq, Hq],
    k8 [Tk, Hkv, d] with k_scale [Hkv], v8 [Tk, Hkv, d] with v_scale
    [Hkv, d].  Returns (out [Tq, Hq, d], lse [Hq, Tq]) in float64."""
    q = dequantize(q8, q_scale, 0)
    k = dequantize(k8, k_scale, 1)
    v = dequantize(v8, v_scale, 2)
    return attention(q, k, v, cu_seqlens_q, cu_seqlens_k, causal, scale, rows=rows, heads=heads)
