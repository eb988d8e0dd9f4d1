"""GPU tests of the error paths that need device data, and of concurrent use.

* VEA_CHECK=1: malformed cu_seqlens and out-of-range top-k indices are found
  on the host and reported as VEA_ERANGE before anything is launched; valid
  calls under VEA_CHECK give bitwise the same results as without it.
* Two independent calls on two streams give bitwise the results of running
  them one after the other (no shared state, one writer per output).
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
