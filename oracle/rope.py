"""Rotary position embedding oracle (float64).  Test infrastructure only.

The vision encoder applies RoPE to the Q and K parts of the fused QKV
projection output in its ``qkv_rope`` step ([3090] conclusion table and section
二); the decoder path applies ``rotary_emb`` in its attention prologue ([V32]
section 实验方法和结果); the fused projection stores Wq|Wk|Wv side by side so
the activation is [T, 3*hidden] ([SGLang] section 3.1).  The pages do not
define the rotation itself, so the oracle uses the standard rotary form:

    pair i of a rotated span of width d_r holds (x[2i], x[2i+1]) and is turned by
    phi = pos * theta^(-2i / d_r):
        x[2i]'   = x[2i] cos(phi) - x[2i+1] sin(phi)
        x[2i+1]' = x[2i] sin(phi) + x[2i+1] cos(phi)

* 1D: one span of width d over the whole head, pos = token position.
* 2D (patch grid): dims [0, d/2) rotate with the grid row, dims [d/2, d) with
  the grid column, each as a span of width d/2.

``rotate_half`` pairs x[i] with x[i + d_r/2] instead (i < d_r/2, same angles):
        x[i]'        = x[i] cos(phi_i) - x[i + d_r/2] sin(phi_i)
        x[i + d_r/2]' = x[i] sin(phi_i) + x[i + d_r/2] cos(phi_i)
the other common convention of the rotary form, offered as a flag.

Trigonometry is float64 here; the pages require at least float32 for it
([MI250] section 4.1, precision table).  V is not rotated.

Fused layout: columns of x_qkv are [Q heads | K heads | V heads], each head
``d`` contiguous values.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rope_inv_freq", "rope_1d", "rope_2d", "qkv_rope"]


def rope_inv_freq(span: int, theta: float) -> np.ndarray:
    """theta^(-2i/span) for the span's pairs i = 0 .. span/2 - 1 (float64)."""
    if span % 2:
        raise ValueError("rotated span must be even")
    i = np.arange(span // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / span)


def _rotate_span(x: np.ndarray, pos: np.ndarray, theta: float, rotate_half: bool = False) -> np.ndarray:
    """Rotate the last axis of x (width d_r) pairwise; pos broadcasts over the
    leading token axis.  x: [T, ..., d_r], pos: [T]."""
    d_r = x.shape[-1]
    phi = pos.astype(np.float64)[:, None] * rope_inv_freq(d_r, theta)[None, :]   # [T, d_r/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (d_r // 2,)
    c = np.cos(phi).reshape(shape)
    s = np.sin(phi).reshape(shape)
    first, second = (np.s_[..., :d_r // 2], np.s_[..., d_r // 2:]) if rotate_half else \
        (np.s_[..., 0::2], np.s_[..., 1::2])
    x0 = x[first]
    x1 = x[second]
    out = np.empty_like(x)
    out[first] = x0 * c - x1 * s
    out[second] = x0 * s + x1 * c
    return out


def rope_1d(x, positions, theta: float, rotate_half: bool = False) -> np.ndarray:
    """x: [T, H, d] real; positions: int [T].  Returns float64 [T, H, d]."""
    x = np.asarray(x, dtype=np.float64)
    return _rotate_span(x, np.asarray(positions), theta, rotate_half)


def rope_2d(x, positions, theta: float, rotate_half: bool = False) -> np.ndarray:
    """x: [T, H, d]; positions: int [T, 2] = (grid row, grid column).

    First half of each head rotates with the row, second half with the column.
    """
    x = np.asarray(x, dtype=np.float64)
    positions = np.asarray(positions)
    d = x.shape[-1]
    if d % 4:
        raise ValueError("2D RoPE needs head_dim divisible by 4")
    out = np.empty_like(x)
    out[..., : d // 2] = _rotate_span(x[..., : d // 2], positions[:, 0], theta, rotate_half)
    out[..., d // 2:] = _rotate_span(x[..., d // 2:], positions[:, 1], theta, rotate_half)
    return out


def qkv_rope(x_qkv, positions, theta: float, num_heads_q: int, num_heads_kv: int, head_dim: int,
             rotate_half: bool = False):
    """Split a fused [T, (Hq + 2 Hkv) d] projection output and rotate Q and K.

    positions: int [T] (1D) or [T, 2] (2D grid).  Returns (q [T, Hq, d],
    k [T, Hkv, d]) in float64.
    """
    x = np.asarray(x_qkv, dtype=np.float64)
    t = x.shape[0]
    hq, hkv, d = num_heads_q, num_heads_kv, head_dim
    if x.shape[1] < (hq + 2 * hkv) * d:
        raise ValueError("x_qkv has too few columns")
    q = x[:, : hq * d].reshape(t, hq, d)
    k = x[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d)
    positions = np.asarray(positions)
    rot = rope_1d if positions.ndim == 1 else rope_2d
    return rot(q, positions, theta, rotate_half), rot(k, positions, theta, rotate_half)
