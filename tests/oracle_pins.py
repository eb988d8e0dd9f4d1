"""Pins that tie the float64 oracle to facts other than itself.

Each pin is a function taking the oracle module (or a mutated stand-in) and
raising AssertionError when the oracle disagrees with:

* a closed form (zero query -> mean of visible V rows; one-hot logits select
  one V row; RoPE of position 0 is the identity; pair norms are kept),
* brute force with pure-Python loops and ``math.fsum`` on tiny inputs,
* an independent library implementation (torch CPU float64
  ``scaled_dot_product_attention``, scipy ``logsumexp``, complex128 rotation),
* an algebraic identity (the blockwise online-softmax merge of
  「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」 section 进一步探索, eq. (1)(2)),
* invariants (permutation of a sparse index row, packing of sequences,
  grouped-query = repeated heads, relative-position property of RoPE).

``tests/test_oracle_pins.py`` runs every pin on the oracle;
``tests/test_oracle_mutants.py`` plants plausible mistakes in the oracle and
checks that some pin fails for each.
"""
from __future__ import annotations

import math

import numpy as np

from vision_encoder_attention_amd import workloads as W


def _rng(seed):
    return np.random.default_rng(seed)


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _visible(i, lq, lk, causal):
    """Keys row i (local) may see — restated here from the causal reading
    (bottom-right alignment), independently of the oracle's helper."""
    if not causal:
        return lk
    return max(0, min(lk, i + lk - lq + 1))


# =========================================================== dense attention

def pin_zero_query_mean(orc):
    """q = 0: every visible key has the same logit, so o_i is the mean of the
    visible V rows and lse_i = ln(#visible); scale = 0 gives the same."""
    rng = _rng(101)
    lq, lk = [5, 1, 9, 4], [5, 3, 12, 0]
    hq, hkv, d = 4, 2, 8
    tq, tk = sum(lq), sum(lk)
    k = rng.standard_normal((tk, hkv, d))
    v = rng.standard_normal((tk, hkv, d))
    for causal in (False, True):
        for q, scale in ((np.zeros((tq, hq, d)), 0.7), (rng.standard_normal((tq, hq, d)), 0.0)):
            out, lse = orc.attention(q, k, v, _cu(lq), _cu(lk), causal, scale)
            cq, ck = _cu(lq), _cu(lk)
            for b in range(len(lq)):
                for i in range(lq[b]):
                    n = _visible(i, lq[b], lk[b], causal)
                    for h in range(hq):
                        g = h // (hq // hkv)
                        row = cq[b] + i
                        if n == 0:
                            assert np.all(out[row, h] == 0) and lse[h, row] == -np.inf
                        else:
                            want = v[ck[b]:ck[b] + n, g].mean(axis=0)
                            assert np.allclose(out[row, h], want, rtol=0, atol=1e-14)
                            assert abs(lse[h, row] - math.log(n)) < 1e-14


def pin_one_hot_select(orc):
    """k_j = e_j and q_i = c e_{pi_g(i)} with c*scale = 100: s_ij is 100 at
    j = pi_g(i) and 0 elsewhere, so o_i = v_{pi_g(i)} up to (n-1) e^-100 and
    lse_i = 100 + ln(1 + (n-1) e^-100).  A different permutation per key/value
    head pins the head mapping, the q-vs-k roles and the V row index."""
    rng = _rng(102)
    lq, lk = [6, 7], [6, 7]
    hq, hkv, d = 4, 2, 8
    cq, ck = _cu(lq), _cu(lk)
    scale = 0.25
    c = 100.0 / scale
    q = np.zeros((sum(lq), hq, d))
    k = np.zeros((sum(lk), hkv, d))
    v = rng.standard_normal((sum(lk), hkv, d))
    perms = {}
    for b in range(2):
        for j in range(lk[b]):
            k[ck[b] + j, :, j] = 1.0
        for h in range(hq):
            g = h // (hq // hkv)
            p = perms.setdefault((b, g), rng.permutation(lk[b]))
            for i in range(lq[b]):
                q[cq[b] + i, h, p[i]] = c
    out, lse = orc.attention(q, k, v, cq, ck, False, scale)
    for b in range(2):
        n = lk[b]
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(lq[b]):
                row = cq[b] + i
                want = v[ck[b] + perms[(b, g)][i], g]
                assert np.allclose(out[row, h], want, rtol=0, atol=1e-35 + 1e-40)
                assert abs(lse[h, row] - (100.0 + math.log1p((n - 1) * math.exp(-100.0)))) < 1e-12


def _brute(q, k, v, lq, lk, causal, scale):
    """Pure-Python loops, math.exp and math.fsum; no numpy arithmetic."""
    cq, ck = _cu(lq), _cu(lk)
    hq, hkv = q.shape[1], k.shape[1]
    d, dv = q.shape[2], v.shape[2]
    out = [[[0.0] * dv for _ in range(hq)] for _ in range(sum(lq))]
    lse = [[0.0] * sum(lq) for _ in range(hq)]
    for b in range(len(lq)):
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(lq[b]):
                row = int(cq[b]) + i
                n = _visible(i, lq[b], lk[b], causal)
                if n == 0:
                    lse[h][row] = -math.inf
                    continue
                s = [scale * math.fsum(float(q[row, h, c]) * float(k[ck[b] + j, g, c]) for c in range(d))
                     for j in range(n)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for c in range(dv):
                    out[row][h][c] = math.fsum(e[j] * float(v[ck[b] + j, g, c]) for j in range(n)) / tot
                lse[h][row] = m + math.log(tot)
    return np.array(out), np.array(lse)


def pin_brute_force(orc):
    """Tiny packed batches (L_q != L_k, empty sequences, GQA, both masks)
    against pure-Python loops."""
    for seed, (lq, lk, hq, hkv) in enumerate([([3, 0, 5], [4, 2, 5], 4, 2), ([1, 6], [7, 3], 2, 1),
                                              ([4], [4], 3, 3)]):
        rng = _rng(200 + seed)
        d, dv = 4, 3
        q = rng.standard_normal((sum(lq), hq, d))
        k = rng.standard_normal((sum(lk), hkv, d))
        v = rng.standard_normal((sum(lk), hkv, dv))
        for causal in (False, True):
            o1, l1 = orc.attention(q, k, v, _cu(lq), _cu(lk), causal, 0.6)
            o2, l2 = _brute(q, k, v, lq, lk, causal, 0.6)
            assert np.allclose(o1, o2, rtol=0, atol=1e-14)
            fin = np.isfinite(l2)
            assert np.array_equal(fin, np.isfinite(l1))
            assert np.allclose(l1[fin], l2[fin], rtol=0, atol=1e-14)


def pin_blocks_and_workers(orc):
    """Row blocks of 1..3 rows (each causal block bounds its own key range)
    evaluated on several threads give the pure-Python result, and the same
    bits as one block per sequence on one thread."""
    lq, lk, hq, hkv = [7, 0, 5, 9], [9, 2, 5, 6], 4, 2
    rng = _rng(230)
    d, dv = 4, 3
    q = rng.standard_normal((sum(lq), hq, d))
    k = rng.standard_normal((sum(lk), hkv, d))
    v = rng.standard_normal((sum(lk), hkv, dv))
    for causal in (False, True):
        o2, l2 = _brute(q, k, v, lq, lk, causal, 0.45)
        fin = np.isfinite(l2)
        ref = None
        for blk, workers in ((1, 3), (2, 2), (3, 4), (512, 1)):
            o1, l1 = orc.attention(q, k, v, _cu(lq), _cu(lk), causal, 0.45, row_block=blk, workers=workers)
            assert np.allclose(o1, o2, rtol=0, atol=1e-14)
            assert np.array_equal(fin, np.isfinite(l1))
            assert np.allclose(l1[fin], l2[fin], rtol=0, atol=1e-14)
            if blk == 1:
                ref = (o1, l1)
        o3, l3 = orc.attention(q, k, v, _cu(lq), _cu(lk), causal, 0.45, row_block=1, workers=1)
        assert np.array_equal(o3, ref[0]) and np.array_equal(l3, ref[1])


def pin_torch_sdpa(orc):
    """torch CPU float64 scaled_dot_product_attention with an explicit boolean
    mask (an independent implementation of the same definition), GQA via
    repeated heads, rows that all see at least one key."""
    import torch
    rng = _rng(103)
    lq, lk = [37, 64, 5], [37, 80, 9]
    hq, hkv, d = 6, 2, 16
    q = rng.standard_normal((sum(lq), hq, d))
    k = rng.standard_normal((sum(lk), hkv, d))
    v = rng.standard_normal((sum(lk), hkv, d))
    cq, ck = _cu(lq), _cu(lk)
    for causal in (False, True):
        out, lse = orc.attention(q, k, v, cq, ck, causal, 0.3)
        for b in range(3):
            qt = torch.from_numpy(q[cq[b]:cq[b + 1]]).permute(1, 0, 2)             # [H, Lq, d]
            kt = torch.from_numpy(k[ck[b]:ck[b + 1]]).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
            vt = torch.from_numpy(v[ck[b]:ck[b + 1]]).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
            mask = torch.ones(lq[b], lk[b], dtype=torch.bool)
            if causal:
                mask = torch.tril(mask, diagonal=lk[b] - lq[b])
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.3)
            assert np.allclose(out[cq[b]:cq[b + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-13)
            # lse against scipy's logsumexp of the masked logits
            from scipy.special import logsumexp
            s = 0.3 * torch.einsum("hid,hjd->hij", qt, kt).numpy()
            s = np.where(mask.numpy()[None], s, -np.inf)
            assert np.allclose(lse[:, cq[b]:cq[b + 1]], logsumexp(s, axis=2), rtol=0, atol=1e-12)


def pin_online_merge(orc):
    """Blockwise online softmax with the merge of eq. (1)(2) (and the matching
    O merge) over random key blocks equals the oracle's two-pass result."""
    rng = _rng(104)
    lq = lk = 50
    d = 8
    q = rng.standard_normal((lq, 1, d)) * 3
    k = rng.standard_normal((lk, 1, d))
    v = rng.standard_normal((lk, 1, d))
    out, lse = orc.attention(q, k, v, _cu([lq]), _cu([lk]), False, 0.5)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, lk), size=rng.integers(1, 8), replace=False))
        bounds = [0] + list(cuts) + [lk]
        for i in range(lq):
            m, s, o = -np.inf, 0.0, np.zeros(d)
            for a, z in zip(bounds[:-1], bounds[1:]):
                sb = 0.5 * (k[a:z, 0] @ q[i, 0])
                mb = sb.max()
                eb = np.exp(sb - mb)
                m_new = max(m, mb)                                     # eq. (1)
                wa, wb = math.exp(m - m_new), math.exp(mb - m_new)
                s_new = wa * s + wb * eb.sum()                         # eq. (2)
                o = (wa * s * o + wb * (eb @ v[a:z, 0])) / s_new      # same weights on O
                m, s = m_new, s_new
            assert np.allclose(out[i, 0], o, rtol=0, atol=1e-13)
            assert abs(lse[0, i] - (m + math.log(s))) < 1e-13


def pin_single_key_and_causal_edges(orc):
    """One key: lse = s_00 and o = v_0.  Causal row 0 (L_q = L_k) sees only
    key 0.  Causal with L_q = L_k = 1 equals non-causal.  A causal row with
    L_q > L_k near the top sees nothing (o = 0, lse = -inf)."""
    rng = _rng(105)
    d = 5
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    v = rng.standard_normal((1, 1, d))
    for causal in (False, True):
        out, lse = orc.attention(q, k, v, _cu([1]), _cu([1]), causal, 0.9)
        assert np.allclose(out[0, 0], v[0, 0], rtol=0, atol=1e-15)
        assert abs(lse[0, 0] - 0.9 * float(q[0, 0] @ k[0, 0])) < 1e-14
    q = rng.standard_normal((6, 1, d))
    k = rng.standard_normal((6, 1, d))
    v = rng.standard_normal((6, 1, d))
    out, lse = orc.attention(q, k, v, _cu([6]), _cu([6]), True, 0.9)
    assert np.allclose(out[0, 0], v[0, 0], rtol=0, atol=1e-15)
    q = rng.standard_normal((5, 1, d))
    k = rng.standard_normal((2, 1, d))
    v = rng.standard_normal((2, 1, d))
    out, lse = orc.attention(q, k, v, _cu([5]), _cu([2]), True, 0.9)
    assert np.all(out[:3] == 0) and np.all(lse[0, :3] == -np.inf)
    assert np.allclose(out[3, 0], v[0, 0], rtol=0, atol=1e-15)


def pin_packing_and_gqa(orc):
    """A packed batch equals separate single-sequence calls (exactly), and
    grouped-query attention equals multi-head attention with each key/value
    head repeated for its group (exactly)."""
    rng = _rng(106)
    lq, lk = [7, 3, 11], [9, 3, 11]
    hq, hkv, d = 6, 3, 8
    q = rng.standard_normal((sum(lq), hq, d))
    k = rng.standard_normal((sum(lk), hkv, d))
    v = rng.standard_normal((sum(lk), hkv, d))
    cq, ck = _cu(lq), _cu(lk)
    for causal in (False, True):
        out, lse = orc.attention(q, k, v, cq, ck, causal, 0.4)
        for b in range(3):
            o1, l1 = orc.attention(q[cq[b]:cq[b + 1]], k[ck[b]:ck[b + 1]], v[ck[b]:ck[b + 1]],
                                   _cu([lq[b]]), _cu([lk[b]]), causal, 0.4)
            assert np.array_equal(o1, out[cq[b]:cq[b + 1]])
            assert np.array_equal(l1, lse[:, cq[b]:cq[b + 1]])
        k_rep = np.repeat(k, hq // hkv, axis=1)
        v_rep = np.repeat(v, hq // hkv, axis=1)
        o2, l2 = orc.attention(q, k_rep, v_rep, cq, ck, causal, 0.4)
        assert np.array_equal(o2, out) and np.array_equal(l2, lse)


def pin_probs(orc):
    """Debug probabilities of a piece: every row sums to 1 (to 1e-14), P V of
    the piece equals the attention output of its rows, and the piece returned
    starts at its own first row."""
    rng = _rng(107)
    lq = lk = 40
    hq, hkv, d = 2, 1, 8
    q = rng.standard_normal((lq, hq, d))
    k = rng.standard_normal((lk, hkv, d))
    v = rng.standard_normal((lk, hkv, d))
    for causal in (False, True):
        out, _ = orc.attention(q, k, v, _cu([lq]), _cu([lk]), causal, 0.5)
        for q0, rows in ((0, 13), (13, 13), (26, 14)):
            p = orc.attn_probs(q, k, _cu([lq]), _cu([lk]), causal, 0.5, head=1, seq=0, q0=q0, rows=rows)
            assert p.shape == (rows, lk)
            assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
            assert np.allclose(p @ v[:, 0], out[q0:q0 + rows, 1], rtol=0, atol=1e-14)
            if causal:
                beyond = np.arange(lk)[None, :] > (q0 + np.arange(rows))[:, None]
                assert np.all(p[beyond] == 0) and np.all(p[~beyond] > 0)


def pin_row_subset(orc):
    """Evaluating a subset of rows/heads gives the same values as the full call."""
    rng = _rng(108)
    lq, lk = [20, 30], [25, 30]
    q = rng.standard_normal((50, 4, 8))
    k = rng.standard_normal((55, 2, 8))
    v = rng.standard_normal((55, 2, 8))
    for causal in (False, True):
        out, lse = orc.attention(q, k, v, _cu(lq), _cu(lk), causal, 0.3)
        rows = np.array([0, 7, 19, 20, 33, 49])
        o2, l2 = orc.attention(q, k, v, _cu(lq), _cu(lk), causal, 0.3, rows=rows, heads=[1, 3])
        assert np.array_equal(o2[rows][:, [1, 3]], out[rows][:, [1, 3]])
        assert np.array_equal(l2[[1, 3]][:, rows], lse[[1, 3]][:, rows])


def pin_attention_paged_roundtrip(orc):
    """A packed varlen batch (GQA, causal) scattered into shuffled pages of a
    shared cache, one block table row per sequence, unused pages holding
    garbage: the paged view gives the unpaged result bitwise."""
    rng = _rng(230)
    lens = [5, 17, 1, 12]
    hq, hkv, d, ps = 4, 2, 6, 4
    cu = _cu(lens)
    q = rng.standard_normal((cu[-1], hq, d))
    k = rng.standard_normal((cu[-1], hkv, d))
    v = rng.standard_normal((cu[-1], hkv, d))
    want_o, want_l = orc.attention(q, k, v, cu, cu, True, 0.4)
    max_pages = max(-(-n // ps) for n in lens)
    n_pages = sum(-(-n // ps) for n in lens) + 3
    order = rng.permutation(n_pages)
    bt = np.full((len(lens), max_pages), -7, np.int64)
    kc = rng.standard_normal((n_pages * ps, hkv, d))
    vc = rng.standard_normal((n_pages * ps, hkv, d))
    nxt = 0
    for b, n in enumerate(lens):
        for pg in range(-(-n // ps)):
            bt[b, pg] = order[nxt]
            nxt += 1
        for j in range(n):
            row = bt[b, j // ps] * ps + j % ps
            kc[row] = k[cu[b] + j]
            vc[row] = v[cu[b] + j]
    o, l = orc.attention_paged(q, kc, vc, bt, ps, cu, cu, True, 0.4)
    assert np.array_equal(o, want_o) and np.array_equal(l, want_l)


DENSE_PINS = [pin_blocks_and_workers, pin_attention_paged_roundtrip, pin_zero_query_mean, pin_one_hot_select, pin_brute_force, pin_torch_sdpa, pin_online_merge,
              pin_single_key_and_causal_edges, pin_packing_and_gqa, pin_probs, pin_row_subset]


# ====================================================================== RoPE

def pin_rope_identity_and_norm(orc):
    """Position 0 is the identity; every rotated pair keeps its length."""
    rng = _rng(301)
    x = rng.standard_normal((9, 3, 16))
    assert np.array_equal(orc.rope_1d(x, np.zeros(9, np.int64), 1e4), x)
    assert np.array_equal(orc.rope_2d(x, np.zeros((9, 2), np.int64), 1e4), x)
    pos = rng.integers(0, 5000, 9)
    y = orc.rope_1d(x, pos, 1e4)
    assert np.allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]),
                       rtol=1e-14, atol=0)


def pin_rope_complex(orc):
    """Adjacent pairs as complex numbers z = x[2i] + i x[2i+1]: RoPE multiplies
    z by e^{i phi} with phi = pos * theta^(-2i/d) (complex128), i.e. a
    counter-clockwise turn by an angle whose per-pair frequency starts at 1
    and falls geometrically by theta^(-2/d) per pair."""
    rng = _rng(302)
    d, theta = 12, 500.0
    x = rng.standard_normal((7, 2, d))
    pos = np.array([0, 1, 2, 3, 10, 100, 977])
    y = orc.rope_1d(x, pos, theta)
    freq = theta ** (-np.arange(0, d, 2) / d)                 # 1, theta^-2/d, theta^-4/d, ...
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    assert np.allclose(y[..., 0::2], z.real, rtol=0, atol=1e-12)
    assert np.allclose(y[..., 1::2], z.imag, rtol=0, atol=1e-12)
    # recovered angle of a unit vector, pair by pair
    e = np.zeros((1, 1, d))
    e[..., 0::2] = 1.0
    ang = orc.rope_1d(e, np.array([1]), theta)
    got = np.arctan2(ang[0, 0, 1::2], ang[0, 0, 0::2])
    assert abs(got[0] - 1.0) < 1e-15
    assert np.allclose(got[1:] / got[:-1], theta ** (-2.0 / d), rtol=1e-12, atol=0)


def pin_rope_relative(orc):
    """<R(p) q, R(p') k> depends only on p - p'."""
    rng = _rng(303)
    d = 16
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    vals = []
    for p in (5, 40, 1234):
        rq = orc.rope_1d(q, np.array([p]), 1e4)
        rk = orc.rope_1d(k, np.array([p - 3]), 1e4)
        vals.append(float((rq * rk).sum()))
    assert np.allclose(vals, vals[0], rtol=0, atol=1e-12)


def pin_rope_2d_halves(orc):
    """2D with column 0 leaves the second half untouched and turns the first
    half like a 1D rotation of width d/2 by the row; with row 0 the mirror
    holds for the column."""
    rng = _rng(304)
    d = 16
    x = rng.standard_normal((6, 2, d))
    rows = np.array([0, 1, 5, 9, 76, 33])
    pos = np.stack([rows, np.zeros(6, np.int64)], 1)
    y = orc.rope_2d(x, pos, 1e4)
    assert np.array_equal(y[..., d // 2:], x[..., d // 2:])
    assert np.allclose(y[..., :d // 2], orc.rope_1d(x[..., :d // 2], rows, 1e4), rtol=0, atol=1e-15)
    pos = np.stack([np.zeros(6, np.int64), rows], 1)
    y = orc.rope_2d(x, pos, 1e4)
    assert np.array_equal(y[..., :d // 2], x[..., :d // 2])
    assert np.allclose(y[..., d // 2:], orc.rope_1d(x[..., d // 2:], rows, 1e4), rtol=0, atol=1e-15)


def pin_qkv_split(orc):
    """Column layout [Q heads | K heads | V heads]: at position 0 q[t,h,c] is
    column h*d + c and k[t,g,c] is column (Hq + g)*d + c."""
    hq, hkv, d, t = 3, 2, 4, 5
    x = np.tile(np.arange((hq + 2 * hkv) * d, dtype=np.float64), (t, 1)) + 1000 * np.arange(t)[:, None]
    q, k = orc.qkv_rope(x, np.zeros(t, np.int64), 1e4, hq, hkv, d)
    for h in range(hq):
        assert np.array_equal(q[:, h, :], x[:, h * d:(h + 1) * d])
    for g in range(hkv):
        assert np.array_equal(k[:, g, :], x[:, (hq + g) * d:(hq + g + 1) * d])
    # 1D vs 2D chosen by the positions' rank
    rng = _rng(305)
    x = rng.standard_normal((t, (hq + 2 * hkv) * d))
    p1 = np.arange(t)
    q1, _ = orc.qkv_rope(x, p1, 1e4, hq, hkv, d)
    assert np.allclose(q1, orc.rope_1d(x[:, :hq * d].reshape(t, hq, d), p1, 1e4), rtol=0, atol=0)


def pin_rope_rotate_half(orc):
    """Rotate-half pairing is the adjacent-pair rotation of the same vector
    with its features reordered (halves interleaved): R_half(x) = P^T
    R_adj(P x) with (P x)[2i] = x[i], (P x)[2i+1] = x[i + d_r/2], per span;
    and pair i of the halves keeps its length."""
    rng = _rng(306)
    d, t = 16, 7
    x = rng.standard_normal((t, 3, d))
    pos = rng.integers(0, 4000, t)
    perm = np.empty(d, np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    y = orc.rope_1d(x, pos, 1e4, rotate_half=True)
    ref = np.empty_like(x)
    ref[..., perm] = orc.rope_1d(x[..., perm], pos, 1e4)
    assert np.allclose(y, ref, rtol=0, atol=1e-13)
    assert np.allclose(np.hypot(y[..., :d // 2], y[..., d // 2:]), np.hypot(x[..., :d // 2], x[..., d // 2:]),
                       rtol=1e-13, atol=0)
    pos2 = rng.integers(0, 90, (t, 2))
    y2 = orc.rope_2d(x, pos2, 1e4, rotate_half=True)
    q = d // 2
    perm2 = np.empty(q, np.int64)
    perm2[0::2] = np.arange(q // 2)
    perm2[1::2] = np.arange(q // 2) + q // 2
    for sp in range(2):
        seg = x[..., sp * q:(sp + 1) * q]
        want = np.empty_like(seg)
        want[..., perm2] = orc.rope_1d(seg[..., perm2], pos2[:, sp], 1e4)
        assert np.allclose(y2[..., sp * q:(sp + 1) * q], want, rtol=0, atol=1e-13)
    xq = np.concatenate([x.reshape(t, -1), x.reshape(t, -1)[:, :d]], 1)       # Q: 2 heads, K: 1, V: 1
    a, b = orc.qkv_rope(xq, pos, 1e4, 2, 1, d, rotate_half=True)
    assert np.allclose(a, orc.rope_1d(x[:, :2, :], pos, 1e4, rotate_half=True), rtol=0, atol=0)
    assert np.allclose(b, orc.rope_1d(x[:, 2:3, :], pos, 1e4, rotate_half=True), rtol=0, atol=0)


ROPE_PINS = [pin_rope_identity_and_norm, pin_rope_complex, pin_rope_relative, pin_rope_2d_halves, pin_qkv_split, pin_rope_rotate_half]


# ============================================== fused QKV projection + RoPE

def pin_qkv_proj_brute(orc):
    """Each output is the exactly rounded dot product of a row of x with a
    column of w, plus the bias (math.fsum over the terms, tiny sizes)."""
    rng = _rng(311)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((7, 9))
    b = rng.standard_normal(9)
    y = orc.qkv_proj(x, w, b)
    y0 = orc.qkv_proj(x, w)
    for t in range(5):
        for n in range(9):
            terms = [x[t, i] * w[i, n] for i in range(7)]
            assert abs(y[t, n] - math.fsum(terms + [b[n]])) < 1e-13
            assert abs(y0[t, n] - math.fsum(terms)) < 1e-13


def pin_qkv_proj_rope_identity_weight(orc):
    """With the identity as weight (hidden = N) the fused step is the
    already-pinned qkv_rope of x, and V is x's last Hkv heads unrotated."""
    rng = _rng(312)
    hq, hkv, d, t = 3, 1, 8, 6
    n = (hq + 2 * hkv) * d
    x = rng.standard_normal((t, n))
    for pos in (rng.integers(0, 3000, t), rng.integers(0, 90, (t, 2))):
        q, k, v = orc.qkv_proj_rope(x, np.eye(n), None, pos, 1e4, hq, hkv, d)
        q0, k0 = orc.qkv_rope(x, pos, 1e4, hq, hkv, d)
        assert np.array_equal(q, q0) and np.array_equal(k, k0)
        assert np.array_equal(v, x[:, (hq + hkv) * d:].reshape(t, hkv, d))


def pin_qkv_proj_rope_structure(orc):
    """Position 0 (or rotate=False) gives the plain column split of x w + b,
    column by column; the rotation keeps each pair's length; a token's output
    depends only on its own row and position; the map is linear in (x, b)."""
    rng = _rng(313)
    hq, hkv, d, t, hid = 2, 2, 8, 5, 11
    n = (hq + 2 * hkv) * d
    x = rng.standard_normal((t, hid))
    w = rng.standard_normal((hid, n))
    b = rng.standard_normal(n)
    q, k, v = orc.qkv_proj_rope(x, w, b, np.zeros(t, np.int64), 1e4, hq, hkv, d)
    pos = rng.integers(1, 5000, t)
    qa, ka, va = orc.qkv_proj_rope(x, w, b, pos, 1e4, hq, hkv, d, rotate=False)
    for tt in range(t):
        for c in range(n):
            ref = math.fsum([x[tt, i] * w[i, c] for i in range(hid)] + [b[c]])
            h, e = divmod(c, d)
            if h < hq:
                got = (q[tt, h, e], qa[tt, h, e])
            elif h < hq + hkv:
                got = (k[tt, h - hq, e], ka[tt, h - hq, e])
            else:
                got = (v[tt, h - hq - hkv, e], va[tt, h - hq - hkv, e])
            assert abs(got[0] - ref) < 1e-12 and abs(got[1] - ref) < 1e-12
    qr, kr, vr = orc.qkv_proj_rope(x, w, b, pos, 1e4, hq, hkv, d)
    assert np.array_equal(vr, v)
    assert np.allclose(np.hypot(qr[..., 0::2], qr[..., 1::2]), np.hypot(q[..., 0::2], q[..., 1::2]), rtol=1e-13, atol=0)
    assert np.allclose(np.hypot(kr[..., 0::2], kr[..., 1::2]), np.hypot(k[..., 0::2], k[..., 1::2]), rtol=1e-13, atol=0)
    qs, ks_, _ = orc.qkv_proj_rope(x[2:3], w, b, pos[2:3], 1e4, hq, hkv, d)
    assert np.allclose(qs[0], qr[2], rtol=0, atol=1e-12) and np.allclose(ks_[0], kr[2], rtol=0, atol=1e-12)
    x2 = rng.standard_normal((t, hid))
    b2 = rng.standard_normal(n)
    s1 = orc.qkv_proj_rope(x, w, b, pos, 1e4, hq, hkv, d)
    s2 = orc.qkv_proj_rope(x2, w, b2, pos, 1e4, hq, hkv, d)
    s12 = orc.qkv_proj_rope(x + x2, w, b + b2, pos, 1e4, hq, hkv, d)
    for a1, a2, a12 in zip(s1, s2, s12):
        assert np.allclose(a1 + a2, a12, rtol=0, atol=1e-11)


def pin_rope_cos_sin(orc):
    """Table entry e of a token is (cos, sin) of pair e's angle: 1D pos *
    theta^(-2e/d); 2D the first d/4 pairs by the grid row with span d/2, the
    rest by the column.  Turning pairs by the table (as complex numbers)
    reproduces the pinned rope_1d / rope_2d."""
    rng = _rng(314)
    d, theta, t = 16, 777.0, 7
    p1 = rng.integers(0, 9000, t)
    cs = orc.rope_cos_sin(p1, theta, d)
    assert cs.shape == (t, d // 2, 2)
    for tt in range(t):
        for e in range(d // 2):
            phi = p1[tt] * theta ** (-2.0 * e / d)
            assert abs(cs[tt, e, 0] - math.cos(phi)) < 1e-12 and abs(cs[tt, e, 1] - math.sin(phi)) < 1e-12
    p2 = rng.integers(0, 120, (t, 2))
    cs2 = orc.rope_cos_sin(p2, theta, d)
    for tt in range(t):
        for e in range(d // 2):
            axis, i = divmod(e, d // 4)
            phi = p2[tt, axis] * theta ** (-2.0 * i / (d // 2))
            assert abs(cs2[tt, e, 0] - math.cos(phi)) < 1e-12 and abs(cs2[tt, e, 1] - math.sin(phi)) < 1e-12
    assert np.array_equal(orc.rope_cos_sin(np.zeros(3, np.int64), theta, d)[..., 0], np.ones((3, d // 2)))
    x = rng.standard_normal((t, 3, d))
    for pos, table, rot in ((p1, cs, orc.rope_1d), (p2, cs2, orc.rope_2d)):
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * (table[:, None, :, 0] + 1j * table[:, None, :, 1])
        y = rot(x, pos, theta)
        assert np.allclose(y[..., 0::2], z.real, rtol=0, atol=1e-12)
        assert np.allclose(y[..., 1::2], z.imag, rtol=0, atol=1e-12)


PROJ_PINS = [pin_qkv_proj_brute, pin_qkv_proj_rope_identity_weight, pin_qkv_proj_rope_structure, pin_rope_cos_sin]


# ========================================================== FP8 (OCP e4m3)

def _e4m3_by_fields(c):
    """Value of code c from its bit fields, written out: (-1)^s 2^(e-7) (1 + m/8),
    subnormals (e = 0) m 2^-9, S.1111.111 NaN."""
    c = int(c)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -mag if s else mag


def pin_e4m3_table(orc):
    """Every code decodes as its bit fields say; 254 non-NaN codes; 1.0 is
    0x38, the largest value 448 is 0x7e, the smallest normal 2^-6 is 0x08,
    the smallest subnormal 2^-9 is 0x01; codes 0x00..0x7e increase."""
    v = orc.e4m3_values()
    for c in range(256):
        f = _e4m3_by_fields(c)
        assert (math.isnan(f) and math.isnan(v[c])) or v[c] == f, c
    assert int(np.sum(~np.isnan(v))) == 254
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert np.all(np.diff(v[:0x7F]) > 0) and np.array_equal(v[0x80:0xFF], -v[:0x7F])


def pin_e4m3_rounding(orc):
    """Encoding returns every finite value's own code; a value strictly
    between two neighbours goes to the nearer; a midpoint goes to the even
    code (the even mantissa); the sign survives rounding to zero.  Worked
    cases: 1.0625 (midpoint of 1 and 1.125) -> 0x38, 1.1875 -> 0x3a (1.25),
    2^-10 (midpoint of 0 and 2^-9) -> 0x00, 1.5 * 2^-10 -> 0x01, 240 -> 0x77,
    3 -> 0x44, -0.0 -> 0x80."""
    v = orc.e4m3_values()
    fin = [c for c in range(256) if not math.isnan(v[c])]
    got = orc.e4m3_encode(v[fin])
    for c, g in zip(fin, got):
        assert int(g) == c or (v[c] == 0 and v[int(g)] == 0 and (c >> 7) == (int(g) >> 7)), (c, int(g))
    pos = v[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2
    enc = orc.e4m3_encode(mid)
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(enc, even.astype(np.uint8))
    eps = (pos[1:] - pos[:-1]) * 1e-3
    assert np.array_equal(orc.e4m3_encode(mid - eps), np.arange(0x7E, dtype=np.uint8))
    assert np.array_equal(orc.e4m3_encode(mid + eps), np.arange(1, 0x7F, dtype=np.uint8))
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (240.0, 0x77),
             (3.0, 0x44), (-0.0, 0x80), (-2.0 ** -11, 0x80), (-448.0, 0xFE)]
    got = orc.e4m3_encode(np.array([a for a, _ in cases]))
    assert [int(g) for g in got] == [b for _, b in cases]


def pin_quantize_fp8(orc):
    """Each block's largest magnitude becomes +-448 exactly (code 0x7e /
    0xfe) and its scale is amax / 448; the dequantised values are within half
    an e4m3 step of the inputs; an all-zero block gets scale 1 and zero
    codes; the block axes are (token, head), head, (head, channel) -- checked
    by brute force over each block."""
    rng = _rng(321)
    x = (rng.standard_normal((7, 3, 16)) * np.array([1.0, 30.0, 0.01])[None, :, None]).astype(np.float32)
    x[2, 1, :] = 0.0
    v = orc.e4m3_values()
    for g in (0, 1, 2):
        codes, sc = orc.quantize_fp8(x, g)
        blocks = {0: [(t, h, slice(None)) for t in range(7) for h in range(3)],
                  1: [(slice(None), h, slice(None)) for h in range(3)],
                  2: [(slice(None), h, c) for h in range(3) for c in range(16)]}[g]
        for blk in blocks:
            xb = x[blk].astype(np.float64)
            cb = codes[blk]
            s = float({0: sc[blk[0], blk[1]] if g == 0 else 0, 1: sc[blk[1]] if g == 1 else 0,
                       2: sc[blk[1], blk[2]] if g == 2 else 0}[g])
            amax = float(np.abs(xb).max())
            if amax == 0:
                assert s == 1.0 and not np.any(v[cb]) 
                continue
            assert s == float(np.float32(np.float32(amax) / np.float32(448.0)))
            i = np.unravel_index(np.argmax(np.abs(xb)), xb.shape)
            assert abs(v[cb[i]]) == 448.0
            deq = v[cb] * s
            step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(v[cb]), 2.0 ** -6))) - 3), 2.0 ** -9)
            assert np.all(np.abs(deq - xb) <= step * s * 0.5 * (1 + 1e-6) + 448 * s * 2.0 ** -24)


def pin_attention_fp8(orc):
    """Attention on fp8 inputs is attention on the inputs decoded from their
    bit fields and scaled (per (token, head), head, (head, channel)); and for
    inputs that are exact e4m3 values with power-of-two block maxima the whole
    quantise -> attention_fp8 chain returns attention on the inputs."""
    rng = _rng(322)
    cu = _cu([5, 0, 9])
    tq, hq, hkv, d = 14, 4, 2, 8
    q8 = rng.integers(0, 256, (tq, hq, d)).astype(np.uint8)
    k8 = rng.integers(0, 256, (tq, hkv, d)).astype(np.uint8)
    v8 = rng.integers(0, 256, (tq, hkv, d)).astype(np.uint8)
    for a in (q8, k8, v8):
        a[(a & 0x7F) == 0x7F] = 0x38                     # no NaN codes
    qs = rng.uniform(0.01, 0.1, (tq, hq)).astype(np.float32)
    ks = rng.uniform(0.01, 0.1, hkv).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, (hkv, d)).astype(np.float32)
    dec = np.vectorize(_e4m3_by_fields)
    q = dec(q8) * qs[:, :, None]
    k = dec(k8) * ks[None, :, None]
    v = dec(v8) * vs[None, :, :]
    for causal in (False, True):
        o1, l1 = orc.attention_fp8(q8, qs, k8, ks, v8, vs, cu, cu, causal, 0.3)
        o2, l2 = orc.attention(q, k, v, cu, cu, causal, 0.3)
        assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)
    vals = orc.e4m3_values()[[0x30, 0x38, 0x3C, 0x44, 0x7E, 0xB8, 0xC4, 0x00]]
    xq = rng.choice(vals, (tq, hq, d))
    xq[:, :, 0] = 448.0                                  # every block's max is 448: scale 1
    xk = rng.choice(vals, (tq, hkv, d))
    xk[0, :, 0] = 448.0
    xv = rng.choice(vals, (tq, hkv, d))
    xv[0, :, :] = 448.0
    cq, sq = orc.quantize_fp8(xq, 0)
    ck, sk = orc.quantize_fp8(xk, 1)
    cv, sv = orc.quantize_fp8(xv, 2)
    assert np.all(sq == 1) and np.all(sk == 1) and np.all(sv == 1)
    o1, l1 = orc.attention_fp8(cq, sq, ck, sk, cv, sv, cu, cu, True, 0.01)
    o2, l2 = orc.attention(xq, xk, xv, cu, cu, True, 0.01)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


FP8_PINS = [pin_e4m3_table, pin_e4m3_rounding, pin_quantize_fp8, pin_attention_fp8]


# ================================================================ sparse MQA

def _sparse_small(seed, rows=4, heads=5, n_kv=30, d_qk=12, k=9):
    rng = _rng(seed)
    q = rng.standard_normal((rows, heads, d_qk))
    kv = rng.standard_normal((n_kv, d_qk))
    idx = np.stack([rng.permutation(n_kv)[:k] for _ in range(rows)]).astype(np.int64)
    return q, kv, idx


def pin_sparse_permutation(orc):
    """Result depends on the index set only: permuting each row changes the
    output by rounding at most."""
    q, kv, idx = _sparse_small(401)
    o1, l1 = orc.sparse_mqa(q, kv, idx, 8, 0.3)
    o2, l2 = orc.sparse_mqa(q, kv, W.permute_rows(idx.astype(np.int32), 9), 8, 0.3)
    assert np.allclose(o1, o2, rtol=0, atol=1e-14) and np.allclose(l1, l2, rtol=0, atol=1e-14)
    # rows on several threads: the same bits
    o3, l3 = orc.sparse_mqa(q, kv, idx, 8, 0.3, workers=3)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def pin_sparse_brute(orc):
    """Pure-Python loops over the selected rows (V = first d_v columns)."""
    q, kv, idx = _sparse_small(402, rows=3, heads=2, n_kv=10, d_qk=5, k=4)
    idx[1, 2] = -1                                  # one padding entry
    dv = 3
    out, lse = orc.sparse_mqa(q, kv, idx, dv, 0.7)
    for r in range(3):
        sel = [int(j) for j in idx[r] if j >= 0]
        for h in range(2):
            s = [0.7 * math.fsum(q[r, h, c] * kv[j, c] for c in range(5)) for j in sel]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            for c in range(dv):
                want = math.fsum(e[t] * kv[sel[t], c] for t in range(len(sel))) / tot
                assert abs(out[r, h, c] - want) < 1e-14
            assert abs(lse[h, r] - (m + math.log(tot))) < 1e-14


def pin_sparse_reductions(orc):
    """k = n_kv in order equals dense non-causal attention of each row's heads
    over the whole latent (torch CPU float64 SDPA); k = 1 gives o = v_idx and
    lse = s; padding entries are skipped; a repeated index counts twice;
    an all-padding row gives o = 0, lse = -inf."""
    import torch
    rng = _rng(403)
    rows, heads, n_kv, d_qk, dv = 3, 4, 11, 10, 6
    q = rng.standard_normal((rows, heads, d_qk))
    kv = rng.standard_normal((n_kv, d_qk))
    idx = np.tile(np.arange(n_kv), (rows, 1))
    out, lse = orc.sparse_mqa(q, kv, idx, dv, 0.4)
    kt = torch.from_numpy(kv)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, kt[..., :dv], scale=0.4)
    assert np.allclose(out, ref.numpy(), rtol=0, atol=1e-13)
    one = rng.integers(0, n_kv, (rows, 1))
    o1, l1 = orc.sparse_mqa(q, kv, one, dv, 0.4)
    for r in range(rows):
        assert np.allclose(o1[r], np.broadcast_to(kv[one[r, 0], :dv], (heads, dv)), rtol=0, atol=1e-15)
        assert np.allclose(l1[:, r], 0.4 * (q[r] @ kv[one[r, 0]]), rtol=0, atol=1e-14)
    pad = np.array([[3, -1, 5, -7], [-1, -1, -1, -1], [2, 2, 9, -1]])
    o2, l2 = orc.sparse_mqa(q, kv, pad, dv, 0.4)
    o3, l3 = orc.sparse_mqa(q[:1], kv, np.array([[3, 5]]), dv, 0.4)
    assert np.allclose(o2[0], o3[0], rtol=0, atol=1e-15)
    assert np.all(o2[1] == 0) and np.all(l2[:, 1] == -np.inf)
    # duplicate: rows {2, 2, 9} = dense attention over keys [kv2, kv2, kv9]
    k3 = torch.from_numpy(kv[[2, 2, 9]])[None]
    ref3 = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q[2:3]), k3, k3[..., :dv], scale=0.4)
    assert np.allclose(o2[2], ref3.numpy()[0], rtol=0, atol=1e-14)


def pin_paged_rows_brute(orc):
    """Each logical position looked up by hand: page j // ps of the table,
    offset j % ps inside that physical page."""
    pt = [5, 0, 3, 7, 1]
    for ps in (1, 2, 4):
        n = len(pt) * ps - 1
        rows = orc.paged_rows(pt, ps, n)
        for j in range(n):
            page, off = divmod(j, ps)
            assert rows[j] == pt[page] * ps + off, (ps, j)


def pin_paged_scatter_roundtrip(orc):
    """A logical cache scattered into shuffled physical pages (plus unused
    ones) through a table gives the unpaged result bitwise; the identity
    table gives it too."""
    rng = _rng(404)
    rows, heads, n_kv, d_qk, dv, ps = 3, 4, 37, 10, 6, 4
    q = rng.standard_normal((rows, heads, d_qk))
    kv = rng.standard_normal((n_kv, d_qk))
    idx = np.stack([rng.permutation(n_kv)[:11] for _ in range(rows)])
    want_o, want_l = orc.sparse_mqa(q, kv, idx, dv, 0.3)
    n_pages = -(-n_kv // ps)
    phys = rng.permutation(n_pages + 3)[:n_pages]            # 3 physical pages left unused
    cache = rng.standard_normal(((n_pages + 3) * ps, d_qk))  # garbage everywhere else
    for j in range(n_kv):
        cache[phys[j // ps] * ps + j % ps] = kv[j]
    o, l = orc.sparse_mqa_paged(q, cache, phys, ps, n_kv, idx, dv, 0.3)
    assert np.array_equal(o, want_o) and np.array_equal(l, want_l)
    ident = np.zeros(((n_pages) * ps, d_qk))
    ident[:n_kv] = kv
    o2, l2 = orc.sparse_mqa_paged(q, ident, np.arange(n_pages), ps, n_kv, idx, dv, 0.3)
    assert np.array_equal(o2, want_o) and np.array_equal(l2, want_l)


SPARSE_PINS = [pin_sparse_permutation, pin_sparse_brute, pin_sparse_reductions, pin_paged_rows_brute,
               pin_paged_scatter_roundtrip]


# ====================================================================== top-k

def _ranks_before(x, i, j):
    """Pairwise rank rule written out: does position i rank before position j?"""
    xi, xj = float(x[i]), float(x[j])
    ni, nj = math.isnan(xi), math.isnan(xj)
    if ni or nj:
        return (not ni and nj) or (ni and nj and i < j)
    if xi != xj:                      # -0.0 == +0.0 falls through to the tie rule
        return xi > xj
    return i < j


def _topk_by_counting(x, k, start, ln):
    """Brute force without sorting: the rank of position j is the number of
    valid positions that rank before it; slot t holds the position of rank t."""
    out = [-1] * k
    for j in range(start, start + ln):
        rank = sum(1 for i in range(start, start + ln) if i != j and _ranks_before(x, i, j))
        if rank < k:
            out[rank] = j
    return out


def pin_topk_brute_force(orc):
    """Tiny rows with many ties (values from a 4-level alphabet), spans, k
    above and below the span length, against the pairwise-count brute force."""
    rng = _rng(501)
    for trial in range(40):
        n = int(rng.integers(1, 13))
        rows = 3
        x = rng.choice(np.array([-1.5, 0.0, 0.25, 2.0], np.float32), size=(rows, n))
        k = int(rng.integers(1, n + 3))
        starts = rng.integers(0, n, rows)
        lens = np.array([int(rng.integers(0, n - s + 1)) for s in starts])
        got = orc.topk_indices(x, k, starts, lens)
        for r in range(rows):
            assert got[r].tolist() == _topk_by_counting(x[r], k, int(starts[r]), int(lens[r])), (trial, r)


def pin_topk_special_values(orc):
    """NaN ranks after every number (NaNs by position), +inf first, -inf last
    among numbers, and -0.0 ties with +0.0 (lower index first)."""
    x = np.array([[0.0, np.nan, -np.inf, 1.0, -0.0, np.inf, np.nan, 0.0]], np.float32)
    x[0, 4] = np.float32(-0.0)
    got = orc.topk_indices(x, 8)[0].tolist()
    assert got == [5, 3, 0, 4, 7, 2, 1, 6], got
    assert got == _topk_by_counting(x[0], 8, 0, 8)


def pin_topk_closed_forms(orc):
    """All-equal row: the first k positions in order.  Strictly decreasing:
    0..k-1.  Strictly increasing: n-1 down to n-k.  A span shorter than k is
    padded with -1.  k = n returns a permutation of the span."""
    n, k = 2590, 2048
    eq = np.full((1, n), 0.5, np.float32)
    assert orc.topk_indices(eq, k)[0].tolist() == list(range(k))
    dec = -np.arange(n, dtype=np.float32)[None]
    assert orc.topk_indices(dec, k)[0].tolist() == list(range(k))
    inc = np.arange(n, dtype=np.float32)[None]
    assert orc.topk_indices(inc, k)[0].tolist() == list(range(n - 1, n - 1 - k, -1))
    short = orc.topk_indices(inc, k, row_starts=[100], row_lens=[1000])[0]
    assert short[:1000].tolist() == list(range(1099, 99, -1)) and np.all(short[1000:] == -1)
    rng = _rng(502)
    x = rng.standard_normal((2, 300)).astype(np.float32)
    full = orc.topk_indices(x, 300)
    for r in range(2):
        assert sorted(full[r].tolist()) == list(range(300))
        assert np.all(np.diff(x[r, full[r]]) <= 0)


def pin_topk_selection_property(orc):
    """On a full-size row with ties planted at the edge of the selection: every
    selected value is >= every unselected one, and among values equal to the
    k-th largest the lowest positions are the ones selected."""
    rng = _rng(503)
    n, k = 2590, 2048
    x = np.round(rng.standard_normal(n) * 8).astype(np.float32)     # many exact ties
    got = orc.topk_indices(x[None], k)[0]
    sel = np.zeros(n, bool)
    sel[got] = True
    assert sel.sum() == k
    kth = x[got[-1]]
    assert x[sel].min() == kth and x[~sel].max() <= kth
    tied = np.flatnonzero(x == kth)
    n_in = int(sel[tied].sum())
    assert 0 < n_in < tied.size                     # the edge does split a tie class
    assert np.all(sel[tied[:n_in]]) and not np.any(sel[tied[n_in:]])


TOPK_PINS = [pin_topk_brute_force, pin_topk_special_values, pin_topk_closed_forms, pin_topk_selection_property]


# =================================================================== pieces

def pin_pieces(orc, figures):
    """Piece arithmetic against the figures printed for the 8547-token image:
    any buffer that fits N = 3535 in one piece but not 3536 gives qb = 1462
    and 6 pieces; the buggy last piece wrote up to N*N floats (7300万, 292 MB)."""
    f = figures["vision_pieces"]
    n = f["tokens"]
    assert f["grid_cols_rows"][0] * f["grid_cols_rows"][1] == n
    assert (f["image_px"][0] // 14, f["image_px"][1] // 14) == tuple(f["grid_cols_rows"])
    safe = f["safe_n_max_single_piece"]
    for cap in (safe * safe, (safe + 1) ** 2 - 1, int(f["buffer_capacity_wan_floats"] * 1e4)):
        assert orc.piece_rows_for_capacity(cap, safe) == safe
        assert orc.piece_rows_for_capacity(cap, n) == f["qb"]
    pieces = orc.piece_ranges(n, f["qb"])
    assert len(pieces) == f["pieces"]
    assert pieces[0] == (0, f["qb"]) and pieces[-1][1] == n
    assert all(b == c for (_, b), (c, _) in zip(pieces[:-1], pieces[1:]))
    assert round(n * n / 1e4, -2) == f["overrun_end_wan_floats"]
    assert round(n * n * 4 / 1e6) == f["overrun_end_mb_approx"]
    assert orc.piece_ranges(n, 0) == [(0, n)] and orc.piece_ranges(0, 5) == []
