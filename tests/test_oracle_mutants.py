"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Every mutant is the oracle's own source file with ONE plausible mistake
substituted in (a dropped term, a wrong sign or index, a swapped operand or
axis).  The mutated module is executed in isolation and the pins of its family
are run against it; the test passes when some pin rejects the mutant.  The
snippet being replaced must exist verbatim, so the list stays in step with the
oracle.
"""
import importlib
import inspect
import json
import os
import types

import pytest

import oracle
from tests import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")

MUTANTS = [
    # (oracle module, original snippet, planted mistake, description)
    ("attention", "return h // (num_heads_q // num_heads_kv)", "return h % num_heads_kv",
     "query heads interleaved over key/value heads"),
    ("attention", "np.clip(i_local + (len_k - len_q) + 1, 0, len_k)", "np.clip(i_local + 1, 0, len_k)",
     "causal mask aligned top-left"),
    ("attention", "np.clip(i_local + (len_k - len_q) + 1, 0, len_k)",
     "np.clip(i_local + (len_k - len_q), 0, len_k)", "causal mask excludes the diagonal"),
    ("attention", "return (e @ vv) / l_sum[:, None], m + np.log(l_sum)",
     "return (e @ vv) / l_sum[:, None], np.log(l_sum)", "lse drops the row max"),
    ("attention", "return (e @ vv) / l_sum[:, None], m + np.log(l_sum)",
     "return (e @ vv), m + np.log(l_sum)", "output not normalised"),
    ("attention", "logits = scale * (q[r[has], h, :] @ kk.T)", "logits = scale * scale * (q[r[has], h, :] @ kk.T)",
     "scale applied twice"),
    ("attention", "kk = k[k0:k0 + nk, g, :]", "kk = k[q0:q0 + nk, g, :]",
     "keys addressed with the query prefix offset"),
    ("attention", "vv = v[k0:k0 + nk, g, :]", "vv = v[k0:k0 + nk, h % v.shape[1], :]",
     "values from the wrong head"),
    ("attention", "nk = int(n_allowed.max()) if n_allowed.size else 0",
     "nk = int(n_allowed.min()) if n_allowed.size else 0", "a causal block's keys cut to its first row's"),
    ("attention", "e = np.where(mask, np.exp(lg - m[:, None]), 0.0)",
     "e = np.exp(np.where(mask, logits, 0.0) - m[:, None])", "masked keys given logit 0 instead of excluded"),
    ("attention", "m = lg.max(axis=1)                                   # pass 1: row max",
     "m = lg.max(axis=1) * 0.5", "row max halved"),
    ("rope", "-2.0 * i / span", "-1.0 * i / span", "frequency exponent -i/d"),
    ("rope", "out[first] = x0 * c - x1 * s", "out[first] = x0 * c + x1 * s", "rotation sign flipped"),
    ("rope", "(np.s_[..., 0::2], np.s_[..., 1::2])", "(np.s_[..., :d_r // 2], np.s_[..., d_r // 2:])",
     "rotate-half pairing for the adjacent form"),
    ("rope", "(np.s_[..., :d_r // 2], np.s_[..., d_r // 2:]) if rotate_half", "(np.s_[..., 0::2], np.s_[..., 1::2]) if rotate_half",
     "adjacent pairing for the rotate-half form"),
    ("rope", "return rot(q, positions, theta, rotate_half), rot(k, positions, theta, rotate_half)",
     "return rot(q, positions, theta, rotate_half), rot(k, positions, theta)", "flag not passed on to K"),
    ("rope", "_rotate_span(x[..., : d // 2], positions[:, 0], theta, rotate_half)",
     "_rotate_span(x[..., : d // 2], positions[:, 1], theta, rotate_half)", "2D first half turned by the column"),
    ("rope", "k = x[:, hq * d:(hq + hkv) * d]", "k = x[:, (hq + hkv) * d:(hq + 2 * hkv) * d]",
     "K read from the V columns"),
    ("sparse", "sel = idx[r][idx[r] >= 0]", "sel = idx[r]", "padding entries not skipped"),
    ("sparse", "kr[:, :d_v]", "kr[:, d_qk - d_v:]", "V taken from the last latent columns"),
    ("sparse", "sel = idx[r][idx[r] >= 0]", "sel = np.unique(idx[r][idx[r] >= 0])", "repeated indices collapsed"),
    ("sparse", "lse[:, r] = m + np.log(l_sum)", "lse[:, r] = np.log(l_sum)", "lse drops the row max"),
    ("paging", "return pt[j // page_size] * page_size + j % page_size",
     "return pt[j % page_size] * page_size + j // page_size", "page index and offset swapped"),
    ("paging", "return pt[j // page_size] * page_size + j % page_size", "return pt[j // page_size] + j % page_size",
     "physical page not scaled by the page size"),
    ("attention", "idx = [paged_rows(bt[b], page_size, int(ck[b + 1] - ck[b])) for b in range(len(ck) - 1)]",
     "idx = [paged_rows(bt[0], page_size, int(ck[b + 1] - ck[b])) for b in range(len(ck) - 1)]",
     "every sequence read through the first block table row"),
    ("pieces", "return min(n, cap_floats // n)", "return min(n, -(-cap_floats // n))", "piece rows rounded up"),
    ("topk", "order = np.lexsort((np.arange(ln), key, nan))", "order = np.lexsort((-np.arange(ln), key, nan))",
     "ties go to the higher position"),
    ("topk", "order = np.lexsort((np.arange(ln), key, nan))", "order = np.argsort(key)",
     "unstable sort for ties (and NaN not ranked last)"),
    ("topk", "key = np.where(nan, 0.0, -seg)", "key = np.where(nan, 0.0, seg)", "lowest values selected"),
    ("topk", "order = np.lexsort((np.arange(ln), key, nan))", "order = np.lexsort((np.arange(ln), key, ~nan))",
     "NaN ranked first"),
    ("topk", "out[r, :m] = (order[:m] + s).astype(np.int32)", "out[r, :m] = order[:m].astype(np.int32)",
     "positions relative to the span start"),
    ("topk", "m = min(k, ln)", "m = min(k, ln - 1)", "one selection short"),
    ("qkv_proj", "y = y + np.asarray(bias, dtype=np.float64)[None, :]", "y = y", "bias dropped"),
    ("qkv_proj", "y = x @ w\n    if bias", "y = x @ w[::-1]\n    if bias", "weight rows reversed (input features misaligned)"),
    ("qkv_proj", "v = y[:, (hq + hkv) * d:].reshape(t, hkv, d)", "v = y[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d)",
     "V taken from the K columns"),
    ("qkv_proj", "q, k = qkv_rope(y, positions, theta, hq, hkv, d, rotate_half)\n    return q, k, v",
     "q, k = qkv_rope(y, positions, theta, hq, hkv, d, rotate_half)\n    return k, q, v", "Q and K swapped"),
    ("qkv_proj", "return y[:, :hq * d].reshape(t, hq, d), y[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d), v",
     "return y[:, :hq * d].reshape(t, hq, d), y[:, (hq + hkv) * d:].reshape(t, hkv, d), v",
     "unrotated K taken from the V columns"),
    ("qkv_proj", "phi = np.concatenate([positions[:, 0].astype(np.float64)[:, None] * f,\n"
                 "                              positions[:, 1].astype(np.float64)[:, None] * f], axis=1)",
     "phi = np.concatenate([positions[:, 1].astype(np.float64)[:, None] * f,\n"
     "                              positions[:, 0].astype(np.float64)[:, None] * f], axis=1)",
     "2D table halves swapped"),
    ("qkv_proj", "return np.stack([np.cos(phi), np.sin(phi)], axis=-1)",
     "return np.stack([np.cos(phi), -np.sin(phi)], axis=-1)", "table turns clockwise"),
    ("qkv_proj", "phi = positions.astype(np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]",
     "phi = positions.astype(np.float64)[:, None] * rope_inv_freq(d // 2, theta)[None, :].repeat(2, 1)",
     "1D table built with half-span frequencies"),
    ("fp8", "v[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)", "v[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 8)",
     "e4m3 exponent bias 8 (the FNUZ variant)"),
    ("fp8", "v[c] = s * m * 2.0 ** -9", "v[c] = s * m * 2.0 ** -10", "subnormal step halved"),
    ("fp8", "pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))", "pick_hi = (dhi <= dlo)",
     "ties rounded up instead of to even"),
    ("fp8", "return np.where(neg, code | 0x80, code).astype(np.uint8)", "return code.astype(np.uint8)",
     "sign dropped"),
    ("fp8", "ax = {0: (2,), 1: (0, 2), 2: (0,)}[granularity]", "ax = {0: (1,), 1: (0, 2), 2: (0,)}[granularity]",
     "per-token blocks taken over heads instead of channels"),
    ("fp8", "ax = {0: (2,), 1: (0, 2), 2: (0,)}[granularity]", "ax = {0: (2,), 1: (0, 2), 2: (2,)}[granularity]",
     "per-channel scales taken over channels"),
    ("fp8", "scale = np.where(zero, np.float32(1), safe / np.float32(E4M3_MAX)).astype(np.float32)",
     "scale = np.where(zero, np.float32(1), safe / np.float32(240.0)).astype(np.float32)",
     "dequantisation scale for a 240 maximum"),
    ("fp8", "return v * s[None, :, :]", "return v * s[None, :, 0:1]", "v scaled by its first channel's scale"),
    ("fp8", "k = dequantize(k8, k_scale, 1)", "k = e4m3_decode(k8)", "k scale ignored"),
]

FAMILY = {"attention": P.DENSE_PINS, "rope": P.ROPE_PINS, "sparse": P.SPARSE_PINS, "pieces": ["pieces"],
          "topk": P.TOPK_PINS, "paging": P.SPARSE_PINS + P.DENSE_PINS, "qkv_proj": P.PROJ_PINS, "fp8": P.FP8_PINS}


def _mutated_oracle(modname, old, new):
    mod = importlib.import_module("oracle." + modname)
    src = inspect.getsource(mod)
    assert src.count(old) >= 1, "snippet not found in oracle/%s.py: %r" % (modname, old)
    mut = types.ModuleType("oracle_mutant_" + modname)
    exec(compile(src.replace(old, new, 1), "<mutant %s>" % modname, "exec"), mut.__dict__)
    ns = types.SimpleNamespace(**{n: getattr(oracle, n) for n in dir(oracle) if not n.startswith("_")})
    for name in getattr(mod, "__all__", []):
        setattr(ns, name, getattr(mut, name))
    return ns


@pytest.mark.parametrize("modname,old,new,desc", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_mutant_is_caught(modname, old, new, desc):
    orc = _mutated_oracle(modname, old, new)
    caught = []
    for pin in FAMILY[modname]:
        try:
            if pin == "pieces":
                with open(GOLDEN) as f:
                    P.pin_pieces(orc, json.load(f))
            else:
                pin(orc)
        except Exception as e:  # a failed assertion or a crash both reject the mutant
            caught.append((getattr(pin, "__name__", pin), type(e).__name__))
    assert caught, "planted mistake '%s' passed every pin" % desc


def test_unmutated_source_passes_through_the_same_harness():
    orc = _mutated_oracle("attention", "return h // (num_heads_q // num_heads_kv)",
                          "return h // (num_heads_q // num_heads_kv)")
    for pin in P.DENSE_PINS:
        pin(orc)
