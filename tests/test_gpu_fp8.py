"""GPU parity of the FP8 path: block quantisation (vea_quantize_fp8) bit-exact
against the oracle, and attention on E4M3 codes (vea_attn_fwd_fp8) against
oracle.attention_fp8 on the oracle's own codes and scales.

Tolerance of the FP8 attention, derived from its arithmetic.
  * Logits: the products of E4M3 values are exact, but the FP8 MFMA sums its
    64 products in groups of 8 aligned to the group's largest, dropping what
    lies more than 2^13 below it (measured on the instruction: one product
    2^14 above 63 equal ones loses the 7 of its group), then adds the group
    sums in fp32.  A logit (natural units) is therefore off by at most
    e_s = (7 2^-13 + (D + 10) 2^-24) L, L = |scale| max_k sum_d |q_d k_d|
    over the row's keys (per group error < 7 2^-13 of its largest product).
  * P is rounded to E4M3 for the P V product: |P^ - P| <= 2^-4 P + 2^-10 in
    the kernel's units, where P = 2^(s c - m) with m at most the row max, so
    the sum l of the fp32 P is at least l_n = sum_k exp(s_k - s_max) =
    1 / max_k p_k.
With p the exact softmax probabilities and V8 the value codes,

    |out - ref|[c] <= v_scale[c] ((2^-4 + 2 e_s) sum_k p_k |V8_k[c]|
                                  + 2^-10 sum_k |V8_k[c]| / l_n)
                      + 2^-8 |ref| (bf16 output rounding) + 1e-5,
    |lse - ref|    <= e_s + 1e-5 |ref| + 1e-4.

Beyond the per-element bound the outputs must also meet cosine >= 0.999."""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import log
from vision_encoder_attention_amd import runner as R
from vision_encoder_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("no GPU visible")
    import vision_encoder_attention_amd as vea
    vea.load_library()
    return t


def _bf16(torch, bits):
    return R.bits_to_tensor(bits, "cuda")


# ----------------------------------------------------------------- quantiser

@pytest.mark.parametrize("d,t", [(64, 333), (128, 333), (64, 2500), (128, 2500)])
def test_quantiser_bit_exact(torch, d, t):
    """333 tokens: one pass per head; 2500: the chunked maximum (ragged last
    chunk) staged in the code buffer."""
    import vision_encoder_attention_amd as vea
    rng = np.random.default_rng(900 + d + t)
    h = 3
    x = W.randn_bf16_bits(rng, (t, h, d))
    xf = W.bf16_bits_to_f32(x)
    # magnitudes spread over heads, a zero row, negative zeros, a tiny row
    xf = xf * np.array([1.0, 64.0, 1.0 / 1024], np.float32)[None, :, None]
    xf[5, 0, :] = 0.0
    xf[6, 1, :] = -0.0
    xf[7, 2, :] = 3e-30
    x = W.f32_to_bf16_bits(xf)
    xg = _bf16(torch, x)
    for g in (0, 1, 2):
        log("quantise d=%d granularity=%d" % (d, g))
        codes, scales = vea.quantize_fp8(xg, g)
        torch.cuda.synchronize()
        rc, rs = oracle.quantize_fp8(W.bf16_bits_to_f32(x), g)
        gc = codes.cpu().numpy()
        gs = scales.cpu().numpy()
        bad = np.argwhere(gc != rc)
        assert bad.size == 0, "codes differ at %s: got %#x want %#x" % (bad[0], gc[tuple(bad[0])], rc[tuple(bad[0])])
        assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), "scales differ"
    # strided input (a view into a wider buffer) and a second run: same bits
    wide = torch.zeros((t, h * d + 64), dtype=torch.bfloat16, device="cuda")
    wide[:, :h * d] = xg.reshape(t, h * d)
    c2, s2 = vea.quantize_fp8(wide.as_strided((t, h, d), (h * d + 64, d, 1)), 0)
    c1, s1 = vea.quantize_fp8(xg, 0)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


# ------------------------------------------------------------- attention

def _case(lengths, hq, hkv, d, seed, q_mul=1.0):
    c = W.random_dense(lengths, lengths, hq, hkv, d, True, "bf16", seed=seed)
    q = W.bf16_bits_to_f32(c.q) * np.float32(q_mul)
    k = W.bf16_bits_to_f32(c.k)
    v = W.bf16_bits_to_f32(c.v)
    q8, qs = oracle.quantize_fp8(q, 0)
    k8, ks = oracle.quantize_fp8(k, 1)
    v8, vs = oracle.quantize_fp8(v, 2)
    return c.cu_seqlens_q, q8, qs, k8, ks, v8, vs


def _run(torch, cu, q8, qs, k8, ks, v8, vs, causal, scale, piece_rows=0):
    import vision_encoder_attention_amd as vea
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cuq = dev(np.asarray(cu, np.int32))
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((q8.shape[1], q8.shape[0]), dtype=torch.float32, device="cuda")
    vea.attn_fwd_fp8(dev(q8), dev(qs), dev(k8), dev(ks), dev(v8), dev(vs), cuq, cuq, causal, scale, out, lse,
                     piece_rows=piece_rows)
    torch.cuda.synchronize()
    return W.bf16_bits_to_f64(R.tensor_to_bits(out)), lse.cpu().numpy().astype(np.float64)


def _bound_and_check(cu, q8, qs, k8, ks, v8, vs, causal, scale, got_o, got_l, rows):
    """Oracle on the sampled rows, and the per-element bound of the module
    docstring computed from exact softmax probabilities."""
    o_ref, l_ref = oracle.attention_fp8(q8, qs, k8, ks, v8, vs, cu, cu, causal, scale, rows=rows)
    q = oracle.fp8.dequantize(q8, qs, 0)
    k = oracle.fp8.dequantize(k8, ks, 1)
    v8a = np.abs(oracle.e4m3_decode(v8))
    hq, hkv = q8.shape[1], k8.shape[1]
    cu = np.asarray(cu)
    worst = worst_l = 0.0
    for r in rows:
        b = int(np.searchsorted(cu, r, side="right") - 1)
        s0, n = int(cu[b]), int(cu[b + 1] - cu[b])
        i = r - s0
        nk = min(n, i + 1) if causal else n
        for h in range(hq):
            g = h // (hq // hkv)
            ref = o_ref[r, h]
            if nk == 0:
                assert np.all(got_o[r, h] == 0) and got_l[h, r] == -np.inf
                continue
            s = scale * (k[s0:s0 + nk, g, :] @ q[r, h, :])
            l1 = float((np.abs(k[s0:s0 + nk, g, :]) @ np.abs(q[r, h, :])).max())
            e_s = (7 * 2.0 ** -13 + (q8.shape[2] + 10) * 2.0 ** -24) * abs(scale) * l1
            e = np.exp(s - s.max())
            p = e / e.sum()
            vv = v8a[s0:s0 + nk, g, :]
            bound = vs[g] * ((2.0 ** -4 + 2 * e_s) * (p @ vv) + 2.0 ** -10 * vv.sum(0) * p.max()) \
                + 2.0 ** -8 * np.abs(ref) + 1e-5
            err = np.abs(got_o[r, h] - ref)
            worst = max(worst, float((err / bound).max()))
            assert np.all(err <= bound), "row %d head %d: error %.3g over bound %.3g" % (
                r, h, float(err.max()), float(bound[np.argmax(err)]))
            lb = e_s + 1e-4 + 1e-5 * abs(l_ref[h, r])
            worst_l = max(worst_l, abs(got_l[h, r] - l_ref[h, r]) / lb)
            assert abs(got_l[h, r] - l_ref[h, r]) <= lb, (r, h, got_l[h, r], l_ref[h, r], e_s)
    g = got_o[rows].ravel()
    rf = o_ref[rows].ravel()
    fin = np.isfinite(rf)
    cos = float(g[fin] @ rf[fin] / (np.linalg.norm(g[fin]) * np.linalg.norm(rf[fin]) + 1e-300))
    log("  worst error / bound %.3f (out), %.3f (lse), cosine %.6f" % (worst, worst_l, cos))
    assert cos >= 0.999


@pytest.mark.parametrize("d,causal,hq,hkv", [(64, False, 4, 4), (64, True, 8, 2), (128, True, 8, 2),
                                             (128, False, 4, 1)])
def test_fp8_attention_against_the_oracle(torch, d, causal, hq, hkv):
    """Several tiles, ragged tails, an empty and a one-token sequence, GQA."""
    cu, q8, qs, k8, ks, v8, vs = _case([300, 0, 1, 197, 513], hq, hkv, d, seed=910 + d + causal)
    scale = 1.0 / math.sqrt(d)
    log("fp8 attention d=%d causal=%s h=%d/%d" % (d, causal, hq, hkv))
    o, l = _run(torch, cu, q8, qs, k8, ks, v8, vs, causal, scale)
    _bound_and_check(cu, q8, qs, k8, ks, v8, vs, causal, scale, o, l, rows=np.arange(q8.shape[0]))


def test_fp8_peaked_logits_and_negative_scale(torch):
    """Peaked rows (q 8x larger: the reference max moves and the rare path
    runs) and a negative scale."""
    cu, q8, qs, k8, ks, v8, vs = _case([700, 260], 4, 2, 64, seed=921, q_mul=8.0)
    for scale in (0.125, -0.125):
        log("fp8 attention peaked scale=%g" % scale)
        o, l = _run(torch, cu, q8, qs, k8, ks, v8, vs, True, scale)
        _bound_and_check(cu, q8, qs, k8, ks, v8, vs, True, scale, o, l, rows=np.arange(0, q8.shape[0], 3))


def test_fp8_pieces_do_not_change_bits_and_repeat_is_bitwise(torch):
    cu, q8, qs, k8, ks, v8, vs = _case([900], 4, 4, 64, seed=922)
    o1, l1 = _run(torch, cu, q8, qs, k8, ks, v8, vs, False, 0.125, piece_rows=0)
    o2, l2 = _run(torch, cu, q8, qs, k8, ks, v8, vs, False, 0.125, piece_rows=250)
    o3, l3 = _run(torch, cu, q8, qs, k8, ks, v8, vs, False, 0.125, piece_rows=0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def _bound_and_check_whole(q8, qs, k8, ks, v8, vs, scale, got_o, got_l):
    """Every element of one non-causal sequence against the oracle, within the
    per-element bound of the module docstring (the same formula as
    _bound_and_check, evaluated a head at a time as whole matrices)."""
    o_ref, l_ref = oracle.attention_fp8(q8, qs, k8, ks, v8, vs, [0, q8.shape[0]], [0, k8.shape[0]], False, scale)
    q = oracle.fp8.dequantize(q8, qs, 0)
    k = oracle.fp8.dequantize(k8, ks, 1)
    v8a = np.abs(oracle.e4m3_decode(v8))
    hq, hkv, d = q8.shape[1], k8.shape[1], q8.shape[2]
    worst = worst_l = 0.0
    for h in range(hq):
        g = h // (hq // hkv)
        kg, qh, vv = k[:, g, :], q[:, h, :], v8a[:, g, :]
        s = scale * (qh @ kg.T)                                   # [rows, keys]
        l1 = (np.abs(qh) @ np.abs(kg).T).max(axis=1)
        e_s = (7 * 2.0 ** -13 + (d + 10) * 2.0 ** -24) * abs(scale) * l1
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ref = o_ref[:, h, :]
        bound = vs[g][None, :] * ((2.0 ** -4 + 2 * e_s[:, None]) * (p @ vv)
                                  + 2.0 ** -10 * vv.sum(0)[None, :] * p.max(axis=1)[:, None]) \
            + 2.0 ** -8 * np.abs(ref) + 1e-5
        del s, p
        err = np.abs(got_o[:, h, :] - ref)
        worst = max(worst, float((err / bound).max()))
        assert np.all(err <= bound), "head %d: %d elements over the bound" % (h, int((err > bound).sum()))
        lb = e_s + 1e-4 + 1e-5 * np.abs(l_ref[h])
        dl = np.abs(got_l[h] - l_ref[h])
        worst_l = max(worst_l, float((dl / lb).max()))
        assert np.all(dl <= lb), "head %d: lse over the bound" % h
    g_, r_ = got_o.ravel(), o_ref.ravel()
    cos = float(g_ @ r_ / (np.linalg.norm(g_) * np.linalg.norm(r_) + 1e-300))
    log("  whole tensors: worst error / bound %.3f (out), %.3f (lse), cosine %.6f, max abs %.3g" % (
        worst, worst_l, cos, float(np.abs(g_ - r_).max())))
    assert cos >= 0.999


def test_fp8_full_size_vision_whole_tensors(torch):
    """The vision image (8547 tokens, 16 heads of 64, pieces of 1462) in FP8:
    every element of out and lse against the oracle within the derived bound."""
    rng = np.random.default_rng(923)
    t, h, d = 8547, 16, 64
    x = [W.bf16_bits_to_f32(W.randn_bf16_bits(rng, (t, h, d))) for _ in range(3)]
    q8, qs = oracle.quantize_fp8(x[0], 0)
    k8, ks = oracle.quantize_fp8(x[1], 1)
    v8, vs = oracle.quantize_fp8(x[2], 2)
    cu = np.array([0, t], np.int32)
    log("fp8 attention vision full size")
    o, l = _run(torch, cu, q8, qs, k8, ks, v8, vs, False, 0.125, piece_rows=1462)
    _bound_and_check_whole(q8, qs, k8, ks, v8, vs, 0.125, o, l)


def test_fp8_mfma_accumulation_measured_through_lse(torch):
    """The accumulation property the logit bound above rests on, measured
    through the public entry point: with one key the lse is the logit itself,
    so a head whose 64 products are one large product 2^(2a) and 63 products
    of 1 shows what the FP8 MFMA's sum drops.  From 2^14 on, exactly the 7
    small products that share the large one's group of 8 vanish; below that
    the sum loses fewer; equal products are summed exactly; and every case
    stays inside e_s of the module docstring."""
    d = 64
    cases = [(a, p) for a in range(9) for p in (0, 37)] + [(None, None)]   # (log2 of the large factor, its position)
    h = len(cases)
    one = 0x38                                          # E4M3 1.0
    q8 = np.full((1, h, d), one, np.uint8)
    exact = np.empty(h)
    for i, (a, p) in enumerate(cases):
        if a is None:
            exact[i] = d                                # 64 products of 1
        else:
            q8[0, i, p] = (a + 7) << 3                  # E4M3 2^a (bias 7, mantissa 0)
            exact[i] = 2.0 ** (2 * a) + (d - 1)
    k8 = q8.copy()                                      # products q_j k_j = q_j^2
    v8 = np.full((1, h, d), one, np.uint8)
    qs = np.ones((1, h), np.float32)
    ks = np.ones(h, np.float32)
    vs = np.ones((h, d), np.float32)
    scale = 2.0 ** -10
    o, l = _run(torch, [0, 1], q8, qs, k8, ks, v8, vs, False, scale)
    got = l[:, 0] / scale                               # the kernel's sum of products
    drop = exact - got
    log("fp8 MFMA sum of one large product 2^(2a) and 63 ones: drop per (a, position) %s" %
        {c: round(float(x), 3) for c, x in zip(cases, drop)})
    e_s = (7 * 2.0 ** -13 + (d + 10) * 2.0 ** -24) * exact                   # in product units
    tol = e_s + (1e-5 * np.abs(exact * scale) + 1e-4) / scale
    assert np.all(np.abs(drop) <= tol)
    assert np.all(np.abs(drop - np.round(drop)) < 0.05)  # whole products of 1 are dropped, nothing else
    drop = np.round(drop)
    for (a, p), x in zip(cases, drop):
        if a is None:
            assert x == 0
        elif a >= 7:
            assert x == 7, (a, p, x)
        else:
            assert 0 <= x <= 7, (a, p, x)
    assert np.all(o == 1.0)                             # one key: the output is its value row
