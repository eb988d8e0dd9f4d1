"""GPU parity of the dense path (qkv_rope + attn_fwd) against the float64 oracle.

All inputs are seeded.  bf16 tensors reach the oracle as the exact same
values (bf16 -> float64 is exact).  Tolerances: see tests/gpu_util.py.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests.gpu_util import ORACLE_WORKERS, assert_bf16_close, assert_f32_close, log, metrics
from vision_encoder_attention_amd import runner as R
from vision_encoder_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("no GPU visible")
    import vision_encoder_attention_amd as vea
    vea.load_library()
    return t


def _f64(t, dtype):
    if dtype == "bf16":
        return W.bf16_bits_to_f64(R.tensor_to_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def _inputs64(case, st):
    """q, k, v as the attention kernel saw them (float64)."""
    if case.x_qkv is not None:
        q = W.bf16_bits_to_f64(R.tensor_to_bits(st.q))
        k = W.bf16_bits_to_f64(R.tensor_to_bits(st.k))
        v = W.bf16_bits_to_f64(case.v_from_x())
    elif case.dtype == "bf16":
        q, k, v = (W.bf16_bits_to_f64(a) for a in (case.q, case.k, case.v))
    else:
        q, k, v = (np.asarray(a, np.float64) for a in (case.q, case.k, case.v))
    return q, k, v


def _check_case(torch, case, piece_rows=None, rows=None):
    log("case %s (piece_rows=%s)" % (case.name, case.piece_rows if piece_rows is None else piece_rows))
    st = R.stage_dense(case)
    R.run_dense(st, piece_rows)
    torch.cuda.synchronize()
    out = _f64(st.out, case.dtype)
    lse = st.lse.cpu().numpy().astype(np.float64)
    if case.x_qkv is not None:
        q_ref, k_ref = oracle.qkv_rope(W.bf16_bits_to_f64(case.x_qkv), case.positions, case.theta,
                                       case.num_heads_q, case.num_heads_kv, case.head_dim)
        assert_bf16_close(_f64(st.q, "bf16"), q_ref, "rope q")
        assert_bf16_close(_f64(st.k, "bf16"), k_ref, "rope k")
    q, k, v = _inputs64(case, st)
    o_ref, l_ref = oracle.attention(q, k, v, case.cu_seqlens_q, case.cu_seqlens_k, case.causal,
                                    float(np.float32(case.scale)), rows=rows, workers=ORACLE_WORKERS)
    sel = slice(None) if rows is None else np.asarray(rows)
    check = assert_f32_close if case.dtype == "f32" else assert_bf16_close
    check(out[sel], o_ref[sel], "out")
    check(lse[:, sel], l_ref[:, sel], "lse")
    if case.x_qkv is not None:
        # end to end from the fused projection, unrounded q/k (reported and gated alike)
        v64 = W.bf16_bits_to_f64(case.v_from_x())
        o_e2e, l_e2e = oracle.attention(q_ref, k_ref, v64, case.cu_seqlens_q, case.cu_seqlens_k, case.causal,
                                        float(np.float32(case.scale)), rows=rows, workers=ORACLE_WORKERS)
        assert_bf16_close(out[sel], o_e2e[sel], "out (end to end)")
        assert_bf16_close(lse[:, sel], l_e2e[:, sel], "lse (end to end)")
    return st


# ----------------------------------------------------------- small configs

@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_small_workloads(torch, idx):
    """Reduced versions of the four dense workloads (several tiles, several
    pieces, ragged tails, empty and one-token sequences)."""
    _check_case(torch, W.small_cases()[idx])


def test_single_head_f32_full(torch):
    """The fp32 workload at full size: N = 256, d = 64, 4 pieces of 64."""
    _check_case(torch, W.single_head_f32())


EDGE = [
    # (lengths_q, lengths_k, hq, hkv, d, causal, dtype, piece_rows, scale, q_mul)
    ([5, 300, 77], [9, 300, 200], 4, 4, 64, False, "bf16", 0, None, 1.0),      # L_q != L_k, non-causal
    ([300, 64, 40], [200, 64, 100], 4, 2, 128, True, "bf16", 0, None, 1.0),    # L_q > L_k: fully masked rows
    ([1], [1], 2, 1, 64, True, "bf16", 0, None, 1.0),                           # single key
    ([0, 129, 0], [0, 129, 0], 8, 8, 128, True, "bf16", 0, None, 1.0),          # empty sequences around one
    ([200], [0], 2, 2, 64, False, "bf16", 0, None, 1.0),                         # no keys at all
    ([257], [257], 8, 1, 128, True, "bf16", 37, None, 1.0),                      # MQA, odd pieces
    ([333], [333], 2, 2, 64, False, "bf16", 0, 0.0, 1.0),                        # scale 0: mean of V
    ([190], [190], 2, 2, 128, True, "bf16", 64, -0.3, 1.0),                      # negative scale
    ([1000], [1000], 2, 2, 128, True, "bf16", 0, None, 8.0),                     # very peaked logits
    ([129, 63], [129, 63], 1, 1, 64, True, "f32", 0, None, 1.0),                 # fp32 causal
    ([100, 3], [40, 3], 1, 1, 64, False, "f32", 7, None, 1.0),                   # fp32 pieces, L_q != L_k
]


@pytest.mark.parametrize("i", range(len(EDGE)))
def test_edge_cases(torch, i):
    lq, lk, hq, hkv, d, causal, dt, qb, scale, qm = EDGE[i]
    case = W.random_dense(lq, lk, hq, hkv, d, causal, dt, seed=500 + i, piece_rows=qb, scale=scale, q_mul=qm)
    _check_case(torch, case)


def _extreme_logit_case(seed, n, heads, mode):
    """Non-causal head_dim 64 images whose logits leave the range of a fixed
    exponent reference: 'over' has rows with q x 64 (2^(s c) would overflow
    fp32), 'under' has every key nearly opposite to every query (all logits
    near -700 in log2 units), 'mixed' scales only the first 100 rows of the
    first head (one workgroup of 256 rows where some rows need the careful
    path and the rest do not)."""
    rng = np.random.default_rng(seed)
    q = W.randn_bf16_bits(rng, (n, heads, 64))
    k = W.randn_bf16_bits(rng, (n, heads, 64))
    v = W.randn_bf16_bits(rng, (n, heads, 64))
    if mode in ("over", "mixed"):
        big = W.randn_bf16_bits(rng, (n, heads, 64), mul=64.0)
        if mode == "over":
            q = big
        else:
            q[:100, 0] = big[:100, 0]
    if mode == "under":
        q = np.full((n, heads, 64), 0x4100, np.uint16)                     # 8.0
        k = W.f32_to_bf16_bits(-8.0 + rng.standard_normal((n, heads, 64), dtype=np.float32))
    cu = np.array([0, n], np.int32)
    return W.DenseCase("extreme_%s" % mode, "bf16", heads, heads, 64, False, 0.125, 300, cu, cu.copy(), q, k, v)


@pytest.mark.parametrize("mode", ["over", "under", "mixed"])
def test_image_kernel_fallback_paths(torch, mode):
    """The head_dim 64 image kernel's fast path uses no per-row reference and
    hands a workgroup to the careful per-step path when a P overflowed or a
    row's sum underflowed: both extremes (and a workgroup where only some
    rows need it) against the oracle, with the key-range split (96 units
    fill less than one round, so every unit splits; bitwise repeatable) and
    without it."""
    case = _extreme_logit_case(750 + len(mode), 1337, 16, mode)
    st = _check_case(torch, case)
    o0, l0 = st.out.clone(), st.lse.clone()
    R.run_attn(st)
    torch.cuda.synchronize()
    assert torch.equal(st.out, o0) and torch.equal(st.lse, l0)
    whole = R.stage_dense(case, split=False)
    R.run_attn(whole)
    torch.cuda.synchronize()
    q, k, v = _inputs64(case, whole)
    o_ref, l_ref = oracle.attention(q, k, v, case.cu_seqlens_q, case.cu_seqlens_k, False,
                                    float(np.float32(case.scale)), workers=ORACLE_WORKERS)
    assert_bf16_close(_f64(whole.out, "bf16"), o_ref, "out (no split)")
    assert_bf16_close(whole.lse.cpu().numpy().astype(np.float64), l_ref, "lse (no split)")


# --------------------------------------------- invariances and determinism

def test_piece_rows_do_not_change_results(torch):
    """Without a workspace O and lse are bitwise identical for every piece
    size (the piece is a scheduling unit only).  With one, small pieces make
    enough workgroups for the last round to be split, and those rows differ
    only by the merge's rounding."""
    case = W.small_cases()[1]            # 667-token vision case
    st = R.stage_dense(case, split=False)
    R.run_dense(st, piece_rows=0)
    torch.cuda.synchronize()
    ref_o, ref_l = st.out.clone(), st.lse.clone()
    for qb in (1, 7, 64, 127, 128, 129, 150, 300, 666, 667, 5000):
        R.run_attn(st, piece_rows=qb)
        torch.cuda.synchronize()
        assert torch.equal(st.out, ref_o), qb
        assert torch.equal(st.lse, ref_l), qb
    sp = R.stage_dense(case)
    R.run_rope(sp)
    for qb in (1, 7):
        R.run_attn(sp, piece_rows=qb)
        torch.cuda.synchronize()
        assert_bf16_close(_f64(sp.out, "bf16"), _f64(ref_o, "bf16"), "split, piece_rows=%d" % qb)
        assert_bf16_close(sp.lse.cpu().numpy().astype(np.float64), ref_l.cpu().numpy().astype(np.float64),
                          "lse split, piece_rows=%d" % qb)


def test_packing_does_not_change_results(torch):
    """A packed batch gives bitwise the same rows as each sequence alone."""
    lens = [70, 129, 1, 260]
    big = W.random_dense(lens, lens, 4, 2, 128, True, "bf16", seed=601)
    st = R.stage_dense(big)
    R.run_attn(st)
    torch.cuda.synchronize()
    cq = big.cu_seqlens_q
    for b, n in enumerate(lens):
        one = W.DenseCase("one", "bf16", 4, 2, 128, True, big.scale, 0, np.array([0, n], np.int32),
                          np.array([0, n], np.int32), big.q[cq[b]:cq[b + 1]], big.k[cq[b]:cq[b + 1]],
                          big.v[cq[b]:cq[b + 1]])
        s1 = R.stage_dense(one)
        R.run_attn(s1)
        torch.cuda.synchronize()
        assert torch.equal(s1.out, st.out[cq[b]:cq[b + 1]])
        assert torch.equal(s1.lse, st.lse[:, cq[b]:cq[b + 1]])


def test_repeated_runs_are_bitwise_identical(torch):
    case = W.small_cases()[2]
    st = R.stage_dense(case)
    R.run_dense(st)
    torch.cuda.synchronize()
    o0, l0, q0 = st.out.clone(), st.lse.clone(), st.q.clone()
    for _ in range(5):
        st.out.fill_(0)
        st.lse.fill_(0)
        R.run_dense(st)
        torch.cuda.synchronize()
        assert torch.equal(st.q, q0) and torch.equal(st.out, o0) and torch.equal(st.lse, l0)


_SHA_SCRIPT = r"""
import hashlib, sys
sys.path.insert(0, %r)
import torch
import vision_encoder_attention_amd as vea
from vision_encoder_attention_amd import runner as R, workloads as W
vea.load_library()
st = R.stage_dense(W.full_case(sys.argv[1]))
R.run_dense(st)
torch.cuda.synchronize()
h = hashlib.sha256()
h.update(R.tensor_to_bits(st.out).tobytes())
h.update(st.lse.cpu().numpy().tobytes())
print("SHA", h.hexdigest())
"""


def _sha(torch, st):
    import hashlib
    h = hashlib.sha256()
    h.update(R.tensor_to_bits(st.out).tobytes())
    h.update(st.lse.cpu().numpy().tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name", ["vision", "varlen_gqa"])
def test_full_size_bitwise_across_runs_and_processes(torch, name):
    """Run-to-run determinism at full size in the benchmark's launch
    configuration (the image with the split of its last round): six runs in
    this process and one in a fresh process give the same SHA-256 of out and
    lse."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    st = R.stage_dense(W.full_case(name))
    digests = set()
    for _ in range(6):
        st.out.fill_(0)
        st.lse.fill_(0)
        R.run_dense(st)
        torch.cuda.synchronize()
        digests.add(_sha(torch, st))
    assert len(digests) == 1, digests
    res = subprocess.run([sys.executable, "-c", _SHA_SCRIPT % root, name], capture_output=True, text=True,
                         timeout=300)
    line = [ln for ln in res.stdout.splitlines() if ln.startswith("SHA ")]
    assert res.returncode == 0 and line, res.stderr[-2000:]
    log("  %s: sha %s in both processes" % (name, line[0][4:20]))
    assert line[0][4:] == digests.pop()


def test_outputs_stay_inside_their_buffers(torch):
    """Guard canaries of 64 KiB around out and lse stay untouched (the bug
    class of an S/P buffer written past its end)."""
    case = W.random_dense([300, 77], [300, 77], 4, 4, 64, False, "bf16", seed=602, piece_rows=100)
    st = R.stage_dense(case)
    guard = 32768
    n_out = st.out.numel()
    big = torch.full((guard + n_out + guard,), -7.0, dtype=torch.bfloat16, device="cuda")
    out = big[guard:guard + n_out].view_as(st.out)
    big_l = torch.full((guard + st.lse.numel() + guard,), 1234.5, dtype=torch.float32, device="cuda")
    lse = big_l[guard:guard + st.lse.numel()].view_as(st.lse)
    st.out, st.lse = out, lse
    R.run_attn(st)
    torch.cuda.synchronize()
    assert bool((big[:guard] == -7.0).all()) and bool((big[guard + n_out:] == -7.0).all())
    assert bool((big_l[:guard] == 1234.5).all()) and bool((big_l[guard + lse.numel():] == 1234.5).all())


def test_probability_piece_export(torch):
    """P of a non-first piece, exported from the start of a piece-sized
    buffer: rows sum to 1 within the band printed for the fixed encoder
    (0.9997 .. 1.0003) and match the oracle's P."""
    import vision_encoder_attention_amd as vea
    with open(GOLDEN) as f:
        band = json.load(f)["row_sums_after_fix"]
    case = W.vision(grid_rows=23, grid_cols=29, heads=4, d=64, piece_rows=150, seed=12)
    st = R.stage_dense(case)
    R.run_dense(st)
    n = case.total_q
    for causal in (False,):
        for q0 in (150, 600):
            rows = min(150, n - q0)
            guard = 4096
            buf = torch.full((guard + rows * n + guard,), -3.0, dtype=torch.float32, device="cuda")
            p = buf[guard:guard + rows * n].view(rows, n)
            vea.attn_probs_piece(st.q, st.k, st.lse, 2, 0, n, 0, n, q0, rows, causal, case.scale, p)
            torch.cuda.synchronize()
            assert bool((buf[:guard] == -3.0).all()) and bool((buf[guard + rows * n:] == -3.0).all())
            pg = p.cpu().numpy().astype(np.float64)
            sums = pg.sum(axis=1)
            log("  piece q0=%d row sums in [%.6f, %.6f]" % (q0, sums.min(), sums.max()))
            assert sums.min() >= band["lo"] and sums.max() <= band["hi"]
            assert np.abs(sums - 1).max() < 1e-4
            q64 = W.bf16_bits_to_f64(R.tensor_to_bits(st.q))
            k64 = W.bf16_bits_to_f64(R.tensor_to_bits(st.k))
            p_ref = oracle.attn_probs(q64, k64, case.cu_seqlens_q, case.cu_seqlens_k, causal,
                                      float(np.float32(case.scale)), head=2, seq=0, q0=q0, rows=rows)
            assert np.abs(pg - p_ref).max() < 1e-4


# ------------------------------------ full-size workloads, whole tensors

@pytest.fixture(scope="module")
def full_run(torch):
    """One GPU pass of a full-size workload in the benchmark's launch
    configuration (qkv_rope, then attn_fwd with the workspace the call asks
    for), kept on the host as float64, plus a second pass compared bitwise.
    Shared by the tests below so that each oracle slice is its own test."""
    cache = {}

    def get(name):
        if name not in cache:
            case = W.full_case(name)
            log("full-size GPU run: %s" % case.name)
            st = R.stage_dense(case)
            R.run_dense(st)
            torch.cuda.synchronize()
            o0, l0 = st.out.clone(), st.lse.clone()
            R.run_dense(st)
            torch.cuda.synchronize()
            run = dict(case=case, repeat_bitwise=bool(torch.equal(st.out, o0) and torch.equal(st.lse, l0)),
                       finite=bool(torch.isfinite(st.out.float()).all()),
                       out=_f64(st.out, "bf16"), lse=st.lse.cpu().numpy().astype(np.float64),
                       q=_f64(st.q, "bf16") if case.x_qkv is not None else None,
                       k=_f64(st.k, "bf16") if case.x_qkv is not None else None,
                       split=st.ws is not None, ref={})
            del st, o0, l0
            torch.cuda.empty_cache()
            cache[name] = run
        return cache[name]
    return get


def _attn_inputs(run):
    """q, k, v as attn_fwd saw them (GPU-produced q and k for fused cases)."""
    case = run["case"]
    if case.x_qkv is not None:
        return run["q"], run["k"], W.bf16_bits_to_f64(case.v_from_x())
    return tuple(W.bf16_bits_to_f64(a) for a in (case.q, case.k, case.v))


def _rope_and_attention(run, end_to_end=False, heads=None):
    """Gate rope q / k (whole), and out / lse of ``heads`` (all: the whole
    tensors) against the oracle run on the kernel's own q / k, or end to end
    from x_qkv (unrounded q / k)."""
    case = run["case"]
    assert run["repeat_bitwise"] and run["finite"]
    if case.x_qkv is not None and not end_to_end:
        q_ref, k_ref = oracle.qkv_rope(W.bf16_bits_to_f64(case.x_qkv), case.positions, case.theta,
                                       case.num_heads_q, case.num_heads_kv, case.head_dim)
        assert_bf16_close(run["q"], q_ref, "rope q (whole)")
        assert_bf16_close(run["k"], k_ref, "rope k (whole)")
    if end_to_end:
        q, k = oracle.qkv_rope(W.bf16_bits_to_f64(case.x_qkv), case.positions, case.theta,
                               case.num_heads_q, case.num_heads_kv, case.head_dim)
        v = W.bf16_bits_to_f64(case.v_from_x())
    else:
        q, k, v = _attn_inputs(run)
    hs = list(range(case.num_heads_q)) if heads is None else list(heads)
    o_ref, l_ref = oracle.attention(q, k, v, case.cu_seqlens_q, case.cu_seqlens_k, case.causal,
                                    float(np.float32(case.scale)), heads=None if heads is None else hs,
                                    workers=ORACLE_WORKERS)
    tag = " (end to end)" if end_to_end else ""
    part = "" if heads is None else " heads %d-%d" % (hs[0], hs[-1])
    assert_bf16_close(run["out"][:, hs], o_ref[:, hs], "out%s%s" % (part, tag))
    assert_bf16_close(run["lse"][hs], l_ref[hs], "lse%s%s" % (part, tag))
    return o_ref, l_ref


@pytest.mark.parametrize("name", ["vision", "varlen_gqa"])
def test_full_size_whole_tensors(full_run, name):
    """Full-size vision image and varlen GQA batch: every element of rope q,
    rope k, out and lse against the oracle (attention on the kernel's own q
    and k), run-to-run bitwise equality."""
    _rope_and_attention(full_run(name))


@pytest.mark.parametrize("name", ["vision", "varlen_gqa"])
def test_full_size_whole_tensors_end_to_end(full_run, name):
    """The same outputs against the oracle chain from the fused projection
    output (q and k rotated in float64, never rounded)."""
    _rope_and_attention(full_run(name), end_to_end=True)


LONG_PARTS = 4


@pytest.mark.parametrize("part", range(LONG_PARTS))
def test_full_size_long_causal_whole(full_run, part):
    """The 32768-token causal prefill (q x 4: peaked rows), every element of
    out and lse: the oracle runs over a quarter of the heads per test (each
    about a quarter minute on 16 host cores); the last part gates the whole
    tensors from the four slices."""
    run = full_run("long_causal")
    hq = run["case"].num_heads_q
    per = hq // LONG_PARTS
    heads = range(part * per, (part + 1) * per)
    o_ref, l_ref = _rope_and_attention(run, heads=heads)
    run["ref"][part] = (list(heads), o_ref[:, list(heads)], l_ref[list(heads)])
    if part == LONG_PARTS - 1:
        assert sorted(run["ref"]) == list(range(LONG_PARTS)), "earlier parts did not run"
        o_all = np.empty_like(run["out"])
        l_all = np.empty_like(run["lse"])
        for hs, o_p, l_p in run["ref"].values():
            o_all[:, hs] = o_p
            l_all[hs] = l_p
        assert_bf16_close(run["out"], o_all, "out (whole tensor)")
        assert_bf16_close(run["lse"], l_all, "lse (whole tensor)")


# ------------------------- split of the last round of workgroups (workspace)

def _round_boundary_case(torch, d, seed):
    """One non-causal image whose 16-head tile count just exceeds one round of
    workgroups (resident workgroups per CU x CUs): the last units are split
    8 ways."""
    from tests.gpu_util import first_split_tiles
    tiles = first_split_tiles(d)
    n = tiles * 128
    return W.vision(grid_rows=n // 64, grid_cols=64, heads=16, d=d, piece_rows=n, seed=seed)


@pytest.mark.parametrize("d", [64, 128])
def test_split_at_a_round_boundary(torch, d):
    """The split rows (the first query tile of every head, cut into 8 key
    ranges and merged) and rows of whole units, against the oracle; repeated
    runs bitwise equal."""
    case = _round_boundary_case(torch, d, seed=700 + d)
    rows = np.unique(np.concatenate([np.arange(0, 128, 9), [127, 128, 129, 255, 4000 % case.total_q,
                                                              case.total_q - 1]]))
    st = _check_case(torch, case, rows=rows)
    assert st.ws is not None and st.ws.numel() > 0
    o0, l0 = st.out.clone(), st.lse.clone()
    R.run_attn(st)
    torch.cuda.synchronize()
    assert torch.equal(st.out, o0) and torch.equal(st.lse, l0)


def test_split_matches_unsplit_within_rounding(torch):
    """On the vision workload the split rows differ from whole rows only by
    the rounding of the merge; rows of whole units are bitwise equal."""
    case = W.full_case("vision")
    a = R.stage_dense(case)
    b = R.stage_dense(case, split=False)
    assert a.ws is not None and b.ws is None
    R.run_dense(a)
    R.run_dense(b)
    torch.cuda.synchronize()
    ao, bo = _f64(a.out, "bf16"), _f64(b.out, "bf16")
    assert_bf16_close(ao, bo, "split vs unsplit")
    assert_bf16_close(a.lse.cpu().numpy().astype(np.float64), b.lse.cpu().numpy().astype(np.float64),
                      "lse split vs unsplit")
    # the last piece's tiles run whole in both launches
    last = slice(5 * case.piece_rows, case.total_q)
    assert torch.equal(a.out[last], b.out[last]) and torch.equal(a.lse[:, last], b.lse[:, last])


def test_attn_workspace_too_small_is_rejected(torch):
    import vision_encoder_attention_amd as vea
    case = _round_boundary_case(torch, 64, seed=710)
    st = R.stage_dense(case)
    R.run_rope(st)
    need = st.ws.numel()
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(vea.VeaError) as e:
        vea.attn_fwd(st.q, st.k, st.v, st.cu_q, st.cu_k, False, case.scale, st.out, st.lse,
                     piece_rows=case.piece_rows, max_seqlen_q=st.max_q, max_seqlen_k=st.max_k, workspace=small)
    assert e.value.status == -6


# ------------------------------------------------------- paged K/V caches

def _page_caches(torch, k, v, cu_k, ps, extra_pages, seed):
    """Scatter packed K/V [total_k, Hkv, d] into caches of shuffled pages (one
    block-table row per sequence, garbage in unused pages)."""
    rng = np.random.default_rng(seed)
    lens = np.diff(np.asarray(cu_k, np.int64))
    pages = [-(-int(n) // ps) for n in lens]
    n_pages = sum(pages) + extra_pages
    order = rng.permutation(n_pages)
    bt = np.zeros((len(lens), max(1, max(pages) if pages else 1)), np.int32)
    rows = []
    nxt = 0
    for b, n in enumerate(lens):
        for pg in range(pages[b]):
            bt[b, pg] = order[nxt]
            nxt += 1
        rows.append(oracle.paged_rows(bt[b], ps, int(n)))
    rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    shape = (n_pages * ps,) + tuple(k.shape[1:])
    kc = torch.randn(shape, device="cuda").to(torch.bfloat16)
    vc = torch.randn(shape, device="cuda").to(torch.bfloat16)
    idx = torch.from_numpy(rows).cuda()
    kc[idx] = k
    vc[idx] = v
    return kc, vc, bt


def _run_paged(torch, st, kc, vc, bt, ps):
    import vision_encoder_attention_amd as vea
    c = st.case
    out = torch.empty_like(st.out)
    lse = torch.empty_like(st.lse)
    vea.attn_fwd_paged(st.q, kc, vc, torch.from_numpy(bt).cuda(), ps, st.cu_q, st.cu_k, c.causal, c.scale, out, lse,
                       piece_rows=c.piece_rows, max_seqlen_q=st.max_q, max_seqlen_k=st.max_k,
                       workspace=st.ws if st.split else None)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("ps", [64, 128, 1024])
def test_paged_kv_against_the_oracle_and_bitwise_unpaged(torch, ps):
    """Causal GQA varlen batch (an empty and a one-token sequence included)
    over shuffled pages: against the oracle's paged view, and bitwise equal
    to the unpaged kernel on the same logical K/V."""
    case = W.random_dense([130, 1, 257, 0, 700], [130, 1, 257, 0, 700], 8, 2, 128, True, "bf16", seed=620 + ps)
    st = R.stage_dense(case)
    R.run_attn(st)
    kc, vc, bt = _page_caches(torch, st.k, st.v, case.cu_seqlens_k, ps, extra_pages=4, seed=630 + ps)
    out, lse = _run_paged(torch, st, kc, vc, bt, ps)
    assert torch.equal(out, st.out) and torch.equal(lse, st.lse)
    o_ref, l_ref = oracle.attention_paged(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(R.tensor_to_bits(kc)),
                                          W.bf16_bits_to_f64(R.tensor_to_bits(vc)), bt, ps, case.cu_seqlens_q,
                                          case.cu_seqlens_k, True, float(np.float32(case.scale)))
    assert_bf16_close(_f64(out, "bf16"), o_ref, "paged out")
    assert_bf16_close(lse.cpu().numpy().astype(np.float64), l_ref, "paged lse")


@pytest.mark.parametrize("name,ps", [("varlen_gqa", 64), ("split", 64)])
def test_paged_kv_full_size_is_bitwise_unpaged(torch, name, ps):
    """The full varlen workload, and an image shape whose last round is split
    (workspace), give bitwise the unpaged results over shuffled pages."""
    case = W.full_case("varlen_gqa") if name == "varlen_gqa" else _round_boundary_case(torch, 64, seed=640)
    st = R.stage_dense(case)
    R.run_dense(st)
    torch.cuda.synchronize()
    kc, vc, bt = _page_caches(torch, st.k, st.v, case.cu_seqlens_k, ps, extra_pages=11, seed=650)
    out, lse = _run_paged(torch, st, kc, vc, bt, ps)
    assert torch.equal(out, st.out) and torch.equal(lse, st.lse)


def test_paged_decode_batch(torch):
    """Decode shape over a paged cache: 24 sequences of one query token each
    over 200..3000 cached keys (GQA 32/8, d 128, 64-row pages, causal =
    bottom-right, so each token sees its whole cache): against the oracle's
    paged view, and bitwise equal to the packed layout."""
    rng = np.random.default_rng(660)
    lk = [int(x) for x in rng.integers(200, 3001, 24)]
    case = W.random_dense([1] * 24, lk, 32, 8, 128, True, "bf16", seed=661)
    st = R.stage_dense(case)
    R.run_attn(st)
    kc, vc, bt = _page_caches(torch, st.k, st.v, case.cu_seqlens_k, 64, extra_pages=5, seed=662)
    out, lse = _run_paged(torch, st, kc, vc, bt, 64)
    assert torch.equal(out, st.out) and torch.equal(lse, st.lse)
    o_ref, l_ref = oracle.attention_paged(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(R.tensor_to_bits(kc)),
                                          W.bf16_bits_to_f64(R.tensor_to_bits(vc)), bt, 64, case.cu_seqlens_q,
                                          case.cu_seqlens_k, True, float(np.float32(case.scale)))
    assert_bf16_close(_f64(out, "bf16"), o_ref, "decode out")
    assert_bf16_close(lse.cpu().numpy().astype(np.float64), l_ref, "decode lse")


@pytest.mark.parametrize("hq,hkv,d,paged", [(32, 8, 128, True), (16, 16, 64, False), (64, 1, 64, False),
                                            (40, 4, 128, False), (128, 2, 64, True)])
def test_attn_decode_against_the_oracle(torch, hq, hkv, d, paged):
    """vea_attn_decode (one query token per sequence, a key/value head's query
    heads as the rows of one workgroup): sequences with no, one, a ragged
    number of and several thousand cached keys; packed and over shuffled
    64-row pages; without workspace and with the key-range split.  Each
    against the oracle, and bitwise repeatable."""
    import vision_encoder_attention_amd as vea
    rng = np.random.default_rng(670 + hq + d)
    lk = [0, 1, 63, 65, 4100] + [int(x) for x in rng.integers(100, 3000, 11)]
    b = len(lk)
    case = W.random_dense([1] * b, lk, hq, hkv, d, False, "bf16", seed=671 + hkv)
    scale = float(np.float32(case.scale))
    log("decode h=%d/%d d=%d paged=%s batch=%d keys=%d" % (hq, hkv, d, paged, b, sum(lk)))
    q = R.bits_to_tensor(case.q, "cuda")
    k = R.bits_to_tensor(case.k, "cuda")
    v = R.bits_to_tensor(case.v, "cuda")
    cuk = torch.from_numpy(np.asarray(case.cu_seqlens_k, np.int32)).cuda()
    kw = {}
    if paged:
        kc, vc, bt = _page_caches(torch, k, v, case.cu_seqlens_k, 64, extra_pages=3, seed=672)
        k, v = kc, vc
        kw = dict(block_table=torch.from_numpy(bt).cuda(), page_size=64)
        o_ref, l_ref = oracle.attention_paged(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(R.tensor_to_bits(kc)),
                                              W.bf16_bits_to_f64(R.tensor_to_bits(vc)), bt, 64, case.cu_seqlens_q,
                                              case.cu_seqlens_k, False, scale)
    else:
        o_ref, l_ref = oracle.attention(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(case.k),
                                        W.bf16_bits_to_f64(case.v), case.cu_seqlens_q, case.cu_seqlens_k, False, scale)
    ws = vea.attn_decode_workspace_size(b, max(lk), hq, hkv, d)
    log("  workspace %d bytes" % ws)
    runs = []
    for workspace in (None, "auto", "auto"):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((hq, b), float("nan"), dtype=torch.float32, device="cuda")
        vea.attn_decode(q, k, v, cuk, case.scale, out, lse, workspace=workspace, **kw)
        torch.cuda.synchronize()
        runs.append((out, lse))
        assert_bf16_close(_f64(out, "bf16"), o_ref, "decode out ws=%s" % workspace)
        assert_bf16_close(lse.cpu().numpy().astype(np.float64), l_ref, "decode lse ws=%s" % workspace)
    assert torch.equal(runs[1][0], runs[2][0]) and torch.equal(runs[1][1], runs[2][1])
    assert torch.all(runs[1][0][0] == 0) and torch.all(torch.isinf(runs[1][1][:, 0]))


def test_attn_decode_full_size_whole_tensors(torch):
    """The decode workload as the benchmark runs it (64 sequences, 512..8192
    cached keys, GQA 32/8, d 128, shuffled 64-row pages, with the key-range
    split): every element of out and lse against the oracle, and bitwise
    equal to the packed layout."""
    import vision_encoder_attention_amd as vea
    case = W.decode()
    st = R.stage_dense(case)
    lk = np.diff(np.asarray(case.cu_seqlens_k, np.int64))
    log("decode full size: %s" % case.name)
    kc, vc, bt = _page_caches(torch, st.k, st.v, case.cu_seqlens_k, 64, extra_pages=8, seed=680)
    out = torch.empty_like(st.q)
    lse = torch.empty((case.num_heads_q, len(lk)), dtype=torch.float32, device="cuda")
    vea.attn_decode(st.q, kc, vc, st.cu_k, case.scale, out, lse, block_table=torch.from_numpy(bt).cuda(),
                    page_size=64)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    vea.attn_decode(st.q, st.k, st.v, st.cu_k, case.scale, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # the sizes passed explicitly (no read-back of cu_seqlens_k), as the
    # benchmark calls it: same bits; a packed total_k other than k's rows is
    # rejected before any launch
    out3 = torch.empty_like(out)
    lse3 = torch.empty_like(lse)
    vea.attn_decode(st.q, kc, vc, st.cu_k, case.scale, out3, lse3, block_table=torch.from_numpy(bt).cuda(),
                    page_size=64, max_seqlen_k=int(lk.max()), total_k=int(lk.sum()))
    vea.attn_decode(st.q, st.k, st.v, st.cu_k, case.scale, out2, lse2, max_seqlen_k=int(lk.max()),
                    total_k=st.k.shape[0])
    torch.cuda.synchronize()
    assert torch.equal(out, out3) and torch.equal(lse, lse3)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    with pytest.raises(ValueError):
        vea.attn_decode(st.q, st.k, st.v, st.cu_k, case.scale, out2, lse2, total_k=st.k.shape[0] + 64)
    # every sequence against the oracle (one query row each), whole tensors
    cu = np.asarray(case.cu_seqlens_k, np.int64)
    got_o = _f64(out, "bf16")
    got_l = lse.cpu().numpy().astype(np.float64)
    o_ref, l_ref = oracle.attention(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(case.k),
                                    W.bf16_bits_to_f64(case.v), np.arange(len(lk) + 1), cu, False,
                                    float(np.float32(case.scale)))
    assert_bf16_close(got_o, o_ref, "decode out (all %d sequences)" % len(lk))
    assert_bf16_close(got_l, l_ref, "decode lse")
