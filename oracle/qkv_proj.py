"""Fused QKV projection with rotary embedding (float64).  Test infrastructure only.

The step before the vision encoder's ``qkv_rope``: the input tokens are
projected by one fused weight holding Wq | Wk | Wv side by side, shape
[hidden, (Hq + 2 Hkv) * d] ([SGLang] section 3.1, where it is
[hidden, 3 * hidden]), and the pages recommend fusing the memory-bound work
around a projection into it ([MI250] section 5.2, fourth point).  Here the
rotation of Q and K is applied to the projection result before it is stored:

    y = x @ w (+ bias)                          [T, (Hq + 2 Hkv) d]
    q, k = qkv_rope(y, positions, theta, ...)   rotation as in oracle.rope
    v = y[:, (Hq + Hkv) d : (Hq + 2 Hkv) d]     not rotated

The pages give no bias term; ``bias`` is optional and None means none.

``rope_cos_sin`` is the per-token table of the rotation: entry e of token t
holds (cos phi, sin phi) of pair e of the head (features 2e and 2e + 1), with
phi the angle ``oracle.rope`` uses for that pair (1D: span d; 2D: the first
d/4 pairs turn with the grid row, the rest with the grid column, spans of d/2).
"""
from __future__ import annotations

import numpy as np

from oracle.rope import qkv_rope, rope_inv_freq

__all__ = ["qkv_proj", "qkv_proj_rope", "rope_cos_sin"]


def qkv_proj(x, w, bias=None) -> np.ndarray:
    """x [T, hidden], w [hidden, N], bias [N] or None -> float64 [T, N]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[0]:
        raise ValueError("x [T, hidden] and w [hidden, N] do not match")
    y = x @ w
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def qkv_proj_rope(x, w, bias, positions, theta: float, num_heads_q: int, num_heads_kv: int, head_dim: int,
                  rotate: bool = True, rotate_half: bool = False):
    """Project and split; rotate Q and K unless rotate is False.

    Returns (q [T, Hq, d], k [T, Hkv, d], v [T, Hkv, d]) in float64.
    """
    hq, hkv, d = num_heads_q, num_heads_kv, head_dim
    n = (hq + 2 * hkv) * d
    w = np.asarray(w)
    if w.shape[1] != n:
        raise ValueError("w must have (Hq + 2 Hkv) * head_dim columns")
    y = qkv_proj(x, w, bias)
    t = y.shape[0]
    v = y[:, (hq + hkv) * d:].reshape(t, hkv, d)
    if not rotate:
        return y[:, :hq * d].reshape(t, hq, d), y[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d), v
    q, k = qkv_rope(y, positions, theta, hq, hkv, d, rotate_half)
    return q, k, v


def rope_cos_sin(positions, theta: float, head_dim: int) -> np.ndarray:
    """Per-token rotation table: float64 [T, head_dim / 2, 2] = (cos, sin)."""
    positions = np.asarray(positions)
    d = head_dim
    if positions.ndim == 1:
        phi = positions.astype(np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]
    else:
        if d % 4:
            raise ValueError("2D RoPE needs head_dim divisible by 4")
        f = rope_inv_freq(d // 2, theta)[None, :]
        phi = np.concatenate([positions[:, 0].astype(np.float64)[:, None] * f,
                              positions[:, 1].astype(np.float64)[:, None] * f], axis=1)
    return np.stack([np.cos(phi), np.sin(phi)], axis=-1)
