"""GPU tests of the error paths that need device data, and of concurrent use.

* VEA_CHECK=1: malformed cu_seqlens and out-of-range top-k indices are found
  on the host and reported as VEA_ERANGE before anything is launched; valid
  calls under VEA_CHECK give bitwise the same results as without it.
* Two independent calls on two streams give bitwise the results of running
  them one after the other (no shared state, one writer per output).
* Workgroups taking their units in another order (VEA_DEBUG_WG_ORDER) give
  bitwise the same results.
* The bindings reject mismatched shapes and tensors on another device before
  anything is launched: the C entry points see only pointers and sizes, so a
  short buffer would otherwise be read or written past its end.
"""
import os

import pytest

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


@pytest.fixture
def vea_check():
    old = os.environ.get("VEA_CHECK")
    os.environ["VEA_CHECK"] = "1"
    yield
    if old is None:
        os.environ.pop("VEA_CHECK", None)
    else:
        os.environ["VEA_CHECK"] = old


def test_check_mode_accepts_valid_calls_unchanged(torch, vea_check):
    case = W.random_dense([100, 37], [100, 37], 4, 2, 128, True, "bf16", seed=701)
    st = R.stage_dense(case)
    R.run_attn(st)
    torch.cuda.synchronize()
    o1, l1 = st.out.clone(), st.lse.clone()
    os.environ.pop("VEA_CHECK")
    R.run_attn(st)
    torch.cuda.synchronize()
    assert torch.equal(st.out, o1) and torch.equal(st.lse, l1)


def test_check_mode_rejects_bad_cu_seqlens(torch, vea_check):
    import vision_encoder_attention_amd as vea
    case = W.random_dense([64, 64], [64, 64], 2, 2, 64, False, "bf16", seed=702)
    st = R.stage_dense(case)
    st.out.fill_(7)
    bad = torch.tensor([0, 129, 128], dtype=torch.int32, device="cuda")     # not monotone
    with pytest.raises(vea.VeaError) as e:
        vea.attn_fwd(st.q, st.k, st.v, bad, st.cu_k, False, case.scale, st.out, st.lse,
                     max_seqlen_q=128, max_seqlen_k=64)
    assert e.value.status == -5
    short = torch.tensor([0, 64, 100], dtype=torch.int32, device="cuda")     # does not end at total
    with pytest.raises(vea.VeaError) as e:
        vea.attn_fwd(st.q, st.k, st.v, short, st.cu_k, False, case.scale, st.out, st.lse,
                     max_seqlen_q=64, max_seqlen_k=64)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((st.out == 7).all()), "nothing may run after a rejected call"


def test_check_mode_rejects_out_of_range_topk(torch, vea_check):
    import vision_encoder_attention_amd as vea
    case = W.sparse_mqa(rows=3, heads=64, n_kv=200, k=64, seed=703)
    idx = case.topk_idx.copy()
    idx[1, 7] = 200
    st = R.stage_sparse(case, idx=idx)
    with pytest.raises(vea.VeaError) as e:
        R.run_sparse(st)
    assert e.value.status == -5


def test_two_streams_match_sequential_results(torch):
    a = W.random_dense([700, 300], [700, 300], 8, 2, 128, True, "bf16", seed=704)
    b = W.vision(grid_rows=20, grid_cols=31, heads=4, d=64, piece_rows=97, seed=705)
    sa, sb = R.stage_dense(a), R.stage_dense(b)
    sp = R.stage_sparse(W.sparse_mqa(rows=6, heads=128, n_kv=500, k=300, seed=706))
    R.run_dense(sa)
    R.run_dense(sb)
    R.run_sparse(sp)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (sa.out, sa.lse, sb.out, sb.lse, sp.out, sp.lse)]
    for t in (sa.out, sb.out, sp.out):
        t.fill_(0)
    torch.cuda.synchronize()
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            R.run_dense(sa)
        with torch.cuda.stream(s2):
            R.run_dense(sb)
        with torch.cuda.stream(s3):
            R.run_sparse(sp)
    torch.cuda.synchronize()
    got = (sa.out, sa.lse, sb.out, sb.lse, sp.out, sp.lse)
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def _order_cases(torch):
    """Launches that cover every kernel family and launch shape the order
    check touches: a pieced image with the split of the last round (its tile
    count just above one round of resident workgroups), a causal
    GQA varlen batch with empty sequences, the fp32 path, decode units with
    key-range splits, FP8 attention and sparse MQA with its split."""
    from tests.gpu_util import first_split_tiles
    tiles = first_split_tiles(64) + 4
    return dict(
        vision=W.vision(grid_rows=tiles, grid_cols=128, heads=16, d=64, piece_rows=128 * ((tiles + 1) // 2),
                        seed=720),
        varlen=W.varlen_gqa(lengths=[130, 0, 257, 1, 700], hq=8, hkv=2, d=128, seed=721),
        f32=W.single_head_f32(n=300, piece_rows=70, seed=722),
        sparse=W.sparse_mqa(rows=300, heads=128, n_kv=900, k=512, seed=723),
    )


def _run_all(torch, staged):
    import vision_encoder_attention_amd as vea
    outs = []
    for name, st in staged.items():
        if name == "sparse":
            R.run_sparse(st)
            outs += [st.out.clone(), st.lse.clone()]
        elif name == "decode":
            q, k, v, cuk, out, lse = st
            vea.attn_decode(q, k, v, cuk, 0.088, out, lse)
            outs += [out.clone(), lse.clone()]
        elif name == "fp8":
            (q8, qs), (k8, ks), (v8, vs), cu, out, lse = st
            vea.attn_fwd_fp8(q8, qs, k8, ks, v8, vs, cu, cu, True, 0.09, out, lse, max_seqlen_q=600, max_seqlen_k=600)
            outs += [out.clone(), lse.clone()]
        else:
            R.run_dense(st)
            outs += [st.out.clone(), st.lse.clone()]
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("order", ["reverse", "stride"])
def test_workgroup_order_does_not_change_results(torch, order):
    """Race smoke: the grid's workgroups take their units in reversed or
    strided order (VEA_DEBUG_WG_ORDER) and every output stays bitwise equal.
    Each unit owns its outputs (and its split chunk's workspace slot), so the
    order in which units run, and which ones are resident together, can change
    nothing."""
    import vision_encoder_attention_amd as vea
    cases = _order_cases(torch)
    staged = {n: (R.stage_sparse(c) if n == "sparse" else R.stage_dense(c)) for n, c in cases.items()}
    assert staged["vision"].ws is not None and staged["sparse"].ws is not None
    dec = W.random_dense([1] * 40, [int(x) for x in range(50, 4050, 100)], 32, 8, 128, True, "bf16", seed=724)
    dq, dk, dv = (R.bits_to_tensor(a, "cuda") for a in (dec.q, dec.k, dec.v))
    staged["decode"] = (dq, dk, dv, torch.from_numpy(dec.cu_seqlens_k.astype("int32")).cuda(),
                        torch.empty_like(dq), torch.empty((32, 40), dtype=torch.float32, device="cuda"))
    f8 = W.random_dense([600, 77], [600, 77], 8, 4, 64, True, "bf16", seed=725)
    fq, fk, fv = (R.bits_to_tensor(a, "cuda") for a in (f8.q, f8.k, f8.v))
    staged["fp8"] = (vea.quantize_fp8(fq, 0), vea.quantize_fp8(fk, 1), vea.quantize_fp8(fv, 2),
                     torch.from_numpy(f8.cu_seqlens_q.astype("int32")).cuda(), torch.empty_like(fq),
                     torch.empty((8, 677), dtype=torch.float32, device="cuda"))
    ref = _run_all(torch, staged)
    old = os.environ.get("VEA_DEBUG_WG_ORDER")
    os.environ["VEA_DEBUG_WG_ORDER"] = order
    try:
        got = _run_all(torch, staged)
    finally:
        if old is None:
            os.environ.pop("VEA_DEBUG_WG_ORDER", None)
        else:
            os.environ["VEA_DEBUG_WG_ORDER"] = old
    assert len(got) == len(ref) == 12
    for i, (g, r) in enumerate(zip(got, ref)):
        assert torch.equal(g, r), "output %d differs under %s order" % (i, order)


def test_bindings_reject_mismatched_shapes_before_launch(torch):
    """One mismatch per case; every call raises ValueError and its output,
    filled with a sentinel, is untouched (nothing was launched)."""
    import vision_encoder_attention_amd as vea
    dev = "cuda"
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    t, hq, hkv, d = 96, 4, 2, 64
    q = torch.randn(t, hq, d, device=dev).to(bf)
    k = torch.randn(t, hkv, d, device=dev).to(bf)
    v = torch.randn(t, hkv, d, device=dev).to(bf)
    cu = torch.tensor([0, 40, t], dtype=i32, device=dev)
    out = torch.full((t, hq, d), 7.0, device=dev).to(bf)
    lse = torch.full((hq, t), 7.0, device=dev)

    def rejects(fn, watch):
        before = watch.clone()
        with pytest.raises(ValueError):
            fn()
        torch.cuda.synchronize()
        assert torch.equal(watch, before)

    rejects(lambda: vea.attn_fwd(q, k, v[:50], cu, cu, False, 0.125, out, lse), out)           # v rows
    rejects(lambda: vea.attn_fwd(q, k, v[:, :, :32].contiguous(), cu, cu, False, 0.125, out), out)  # v head_dim
    rejects(lambda: vea.attn_fwd(q, k, v, cu, cu, False, 0.125, out[:50]), out)               # out rows
    rejects(lambda: vea.attn_fwd(q, k, v, cu, cu[:2], False, 0.125, out), out)                # cu lengths
    rejects(lambda: vea.attn_fwd(q, k, v, cu, cu, False, 0.125, out, lse.cpu()), out)          # lse on the host
    rejects(lambda: vea.attn_fwd_noalloc(q, k, v[:50], cu, cu, False, 0.125, out, max_seqlen_q=56,
                                         max_seqlen_k=56), out)
    kc = torch.randn(128, hkv, d, device=dev).to(bf)
    bt = torch.tensor([[0, 1], [0, 1]], dtype=i32, device=dev)
    rejects(lambda: vea.attn_fwd_paged(q, kc, kc[:, :1].contiguous(), bt, 64, cu, cu, False, 0.125, out,
                                       max_seqlen_q=56, max_seqlen_k=56, total_k=t), out)      # v_cache heads
    qd = torch.randn(2, hq, d, device=dev).to(bf)
    od = torch.full((2, hq, d), 7.0, device=dev).to(bf)
    rejects(lambda: vea.attn_decode(qd, k[:, :, :32].contiguous(), v[:, :, :32].contiguous(), cu, 0.125, od), od)
    # rope: outputs shorter than the projection output, positions of the wrong length
    x = torch.randn(t, (hq + 2 * hkv) * d, device=dev).to(bf)
    pos = torch.arange(t, dtype=i32, device=dev)
    qo = torch.full((t, hq, d), 7.0, device=dev).to(bf)
    ko = torch.full((t, hkv, d), 7.0, device=dev).to(bf)
    rejects(lambda: vea.qkv_rope(x, pos, 1e4, qo[:50], ko), qo)
    rejects(lambda: vea.qkv_rope(x, pos[:50], 1e4, qo, ko), qo)
    # FP8: a q scale of the wrong shape
    q8 = torch.zeros(t, hq, d, dtype=torch.uint8, device=dev)
    k8 = torch.zeros(t, hkv, d, dtype=torch.uint8, device=dev)
    rejects(lambda: vea.attn_fwd_fp8(q8, torch.ones(t, device=dev), k8, torch.ones(hkv, device=dev), k8,
                                     torch.ones(hkv, d, device=dev), cu, cu, False, 0.125, out), out)
    # projection: a weight of the wrong height
    hid = 128
    xp = torch.randn(t, hid, device=dev).to(bf)
    wp = torch.randn(hid // 2, (hq + 2 * hkv) * d, device=dev).to(bf)
    vo = torch.full((t, hkv, d), 7.0, device=dev).to(bf)
    rejects(lambda: vea.qkv_proj_rope(xp, wp, None, None, qo, ko, vo), qo)
    # sparse MQA: latent rows narrower than q's d_qk, out with the wrong heads
    r, h, dqk, dv, kk = 3, 128, 576, 512, 64
    qs_ = torch.randn(r, h, dqk, device=dev).to(bf)
    kv = torch.randn(100, dqk, device=dev).to(bf)
    idx = torch.zeros(r, kk, dtype=i32, device=dev)
    os_ = torch.full((r, h, dv), 7.0, device=dev).to(bf)
    rejects(lambda: vea.sparse_mqa_fwd(qs_, kv[:, :512].contiguous(), idx, kk, 0.04, os_), os_)
    rejects(lambda: vea.sparse_mqa_fwd(qs_, kv, idx, kk, 0.04, os_[:, :64].contiguous()), os_)
    pt = torch.arange(2, dtype=i32, device=dev)
    rejects(lambda: vea.sparse_mqa_paged_fwd(qs_, kv[:64, :512].contiguous(), pt, 64, 100, idx, kk, 0.04, os_), os_)
    # top-k: an output on the host
    lg = torch.randn(4, 300, device=dev)
    ot = torch.full((4, 32), 7, dtype=i32, device=dev)
    rejects(lambda: vea.topk_indices(lg, 32, ot.cpu()), ot)
    # probability export: a piece past k's rows
    pb = torch.full((10, t), 7.0, device=dev)
    rejects(lambda: vea.attn_probs_piece(q, k, lse, 0, 0, t, 0, t + 5, 0, 10, False, 0.125, pb), pb)
