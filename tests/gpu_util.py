"""Shared helpers of the GPU parity tests: device staging goes through the
package runner; comparison metrics and tolerances live here."""
from __future__ import annotations

import math
import sys

import numpy as np

from oracle.pool import host_cores

# Tolerances (stated per output tensor):
#   fp32 path: normwise max relative error  max|g - r| / max|r|  <= 1e-5
#   bf16 path: max |g - r| <= 2e-2  and  cosine(g, r) >= 0.999
F32_NORMWISE = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MIN_COS = 0.999

# Host threads for the oracle on full-size workloads (the GPU host's CPU share
# is 16 cores).
ORACLE_WORKERS = max(1, min(16, host_cores()))


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(got, ref):
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    fin = np.isfinite(r)
    if not np.array_equal(fin, np.isfinite(g)):
        return dict(finite_match=False)
    g, r = g[fin], r[fin]
    if g.size == 0:
        return dict(finite_match=True, max_abs=0.0, cos=1.0, rmse=0.0, normwise=0.0, n=0)
    d = g - r
    ng, nr = np.linalg.norm(g), np.linalg.norm(r)
    cos = float(g @ r / (ng * nr)) if ng > 0 and nr > 0 else (1.0 if ng == nr else 0.0)
    mr = float(np.abs(r).max())
    return dict(finite_match=True, max_abs=float(np.abs(d).max()), cos=cos, rmse=float(math.sqrt((d * d).mean())),
                normwise=float(np.abs(d).max() / mr) if mr > 0 else float(np.abs(d).max()), n=int(g.size))


def assert_bf16_close(got, ref, name):
    m = metrics(got, ref)
    log("  %-28s %s" % (name, {k: (round(v, 7) if isinstance(v, float) else v) for k, v in m.items()}))
    assert m["finite_match"], "%s: -inf/NaN positions differ" % name
    assert m["max_abs"] <= BF16_MAX_ABS, "%s: max abs %.3g > %.3g" % (name, m["max_abs"], BF16_MAX_ABS)
    assert m["cos"] >= BF16_MIN_COS, "%s: cosine %.6f < %.3f" % (name, m["cos"], BF16_MIN_COS)
    return m


def assert_f32_close(got, ref, name):
    m = metrics(got, ref)
    log("  %-28s %s" % (name, {k: (round(v, 10) if isinstance(v, float) else v) for k, v in m.items()}))
    assert m["finite_match"], "%s: -inf/NaN positions differ" % name
    assert m["normwise"] <= F32_NORMWISE, "%s: normwise rel %.3g > %.1g" % (name, m["normwise"], F32_NORMWISE)
    return m


def first_split_tiles(head_dim, heads=16):
    """Smallest number of 128-row query tiles per head of one non-causal bf16
    image (one piece) for which attn_fwd splits the last round of workgroups
    on this device (the round size depends on the CU count and the kernel's
    occupancy, so tests ask the library instead of assuming it)."""
    import vision_encoder_attention_amd as vea
    for t in range(1, 4096):
        n = 128 * t
        if vea.attn_fwd_workspace_size(1, 1, n, n, n, n, heads, heads, head_dim, False, 0) > 0:
            return t
    raise RuntimeError("no split found")
