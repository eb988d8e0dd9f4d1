"""GPU parity of the top-k sparse MQA path against the float64 oracle."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import ORACLE_WORKERS, assert_bf16_close, log
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


def _run(torch, case, idx=None, split=True):
    st = R.stage_sparse(case, idx=idx, split=split)
    R.run_sparse(st)
    torch.cuda.synchronize()
    return st


def _check(torch, case, idx=None, rows=None, name="", split=True):
    log("sparse case %s %s split=%s" % (case.name, name, split))
    st = _run(torch, case, idx, split)
    ix = case.topk_idx if idx is None else idx
    o_ref, l_ref = oracle.sparse_mqa(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(case.kv_latent), ix, case.d_v,
                                     float(np.float32(case.scale)), rows=rows, workers=ORACLE_WORKERS)
    sel = slice(None) if rows is None else np.asarray(rows)
    out = W.bf16_bits_to_f64(R.tensor_to_bits(st.out))
    lse = st.lse.cpu().numpy().astype(np.float64)
    assert_bf16_close(out[sel], o_ref[sel], "out")
    assert_bf16_close(lse[:, sel], l_ref[:, sel], "lse")
    return st


def test_small_sparse(torch):
    _check(torch, W.small_cases()[4])


def test_index_order_is_irrelevant_bitwise(torch):
    """The same index sets in other orders give bitwise the same output (the
    pages' kernel moved by 2^-8; here the rows are sorted on the device)."""
    case = W.small_cases()[4]
    a = _run(torch, case)
    for seed in (105, 106):
        b = _run(torch, case, W.permute_rows(case.topk_idx, seed))
        assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)


def test_padding_duplicates_and_out_of_range(torch):
    """-1 padding and indices >= n_kv are skipped, repeated indices count
    twice, an all-padding row gives o = 0 and lse = -inf, k = 1 selects one
    row."""
    case = W.sparse_mqa(rows=5, heads=64, n_kv=300, k=96, seed=16)
    idx = case.topk_idx.copy()
    idx[0, ::3] = -1
    idx[1, :] = -1
    idx[2, 10:20] = idx[2, 0:10]                   # duplicates
    idx[3, 5] = 100000                             # out of range: skipped by the kernel
    st = _run(torch, case, idx)
    ref_idx = idx.copy()
    ref_idx[3, 5] = -1                             # the oracle's view of a skipped entry
    o_ref, l_ref = oracle.sparse_mqa(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(case.kv_latent), ref_idx,
                                     case.d_v, float(np.float32(case.scale)))
    out = W.bf16_bits_to_f64(R.tensor_to_bits(st.out))
    lse = st.lse.cpu().numpy().astype(np.float64)
    assert np.all(out[1] == 0) and np.all(lse[:, 1] == -np.inf)
    assert_bf16_close(out, o_ref, "out")
    assert_bf16_close(lse, l_ref, "lse")
    one = W.SparseCase("k1", case.q, case.kv_latent, case.topk_idx[:, :1].copy(), case.d_v, case.scale)
    st1 = _run(torch, one)
    out1 = W.bf16_bits_to_f64(R.tensor_to_bits(st1.out))
    kv = W.bf16_bits_to_f64(case.kv_latent)
    for r in range(5):
        assert np.array_equal(out1[r], np.broadcast_to(kv[one.topk_idx[r, 0], :case.d_v], out1[r].shape))


def test_heads_not_a_multiple_of_the_workgroup(torch):
    _check(torch, W.sparse_mqa(rows=3, heads=40, n_kv=200, k=70, seed=17), name="40 heads")


def test_full_size_whole_tensors(torch):
    """The full workload (323 rows x 128 heads, k = 2048 of 2590) in the
    benchmark's launch configuration (with the split of the last round):
    every element of out and lse against the oracle, the output bitwise
    invariant to a permutation of every index row, repeated runs bitwise
    equal, and the batch-invariant launch (no split) within tolerance."""
    case = W.full_case("sparse_mqa")
    st = _check(torch, case, name="full")
    assert st.ws is not None
    o0, l0 = st.out.clone(), st.lse.clone()
    R.run_sparse(st)
    torch.cuda.synchronize()
    assert torch.equal(st.out, o0) and torch.equal(st.lse, l0)
    perm = _run(torch, case, W.permute_rows(case.topk_idx, 105))
    assert torch.equal(perm.out, o0) and torch.equal(perm.lse, l0)
    whole = _run(torch, case, split=False)
    assert_bf16_close(W.bf16_bits_to_f64(R.tensor_to_bits(whole.out)), W.bf16_bits_to_f64(R.tensor_to_bits(o0)),
                      "no split vs split")


def test_large_cache_uses_the_sorting_network(torch):
    """A latent cache too large for the in-LDS counting sort (80000 rows) takes
    the bitonic path: same results, padding / duplicates / out-of-range entries
    handled the same way, still bitwise invariant to index order."""
    case = W.sparse_mqa(rows=3, heads=128, n_kv=80000, k=300, seed=18)
    idx = case.topk_idx.copy()
    idx[0, ::5] = -1
    idx[1, 20:40] = idx[1, 0:20]                   # duplicates
    idx[2, 7] = 80000                              # out of range: skipped
    st = _run(torch, case, idx)
    ref_idx = idx.copy()
    ref_idx[2, 7] = -1
    o_ref, l_ref = oracle.sparse_mqa(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(case.kv_latent), ref_idx,
                                     case.d_v, float(np.float32(case.scale)))
    assert_bf16_close(W.bf16_bits_to_f64(R.tensor_to_bits(st.out)), o_ref, "out")
    assert_bf16_close(st.lse.cpu().numpy().astype(np.float64), l_ref, "lse")
    perm = _run(torch, case, W.permute_rows(idx, 107))
    assert torch.equal(perm.out, st.out) and torch.equal(perm.lse, st.lse)


@pytest.mark.parametrize("n_kv,k", [(10000, 1024), (20000, 3000)])
def test_counts_in_the_stage_ring(torch, n_kv, k):
    """Counting-sort counts too many for their own LDS array (more than 4088
    cache rows up to 2048 indices, 18424 up to 4096) are kept in the stage
    ring, so Q is loaded after the sort rather than under it: same results,
    bitwise invariant to index order."""
    case = W.sparse_mqa(rows=3, heads=128, n_kv=n_kv, k=k, seed=31 + k)
    st = _check(torch, case, name="n_kv %d k %d" % (n_kv, k))
    perm = _run(torch, case, W.permute_rows(case.topk_idx, 109))
    assert torch.equal(perm.out, st.out) and torch.equal(perm.lse, st.lse)


def test_more_than_2048_indices(torch):
    """k in (2048, 4096] uses the three-stage variant of the kernel."""
    case = W.sparse_mqa(rows=2, heads=128, n_kv=3500, k=3000, seed=19)
    st = _check(torch, case, name="k3000")
    perm = _run(torch, case, W.permute_rows(case.topk_idx, 108))
    assert torch.equal(perm.out, st.out) and torch.equal(perm.lse, st.lse)


# ---- the split of the last, partial round of workgroups (a caller workspace)

def _cus(torch):
    return torch.cuda.get_device_properties(0).multi_processor_count


def test_without_workspace_rows_are_batch_invariant(torch):
    """Without a workspace every row runs whole: right against the oracle, and
    a row's bits do not depend on the other rows of the batch."""
    case = W.sparse_mqa(rows=5, heads=128, n_kv=700, k=256, seed=21)
    st = _check(torch, case, split=False, name="unsplit")
    assert st.ws is None
    sub = W.SparseCase("rows 2..3", case.q[2:4].copy(), case.kv_latent, case.topk_idx[2:4].copy(), case.d_v,
                       case.scale)
    st2 = _run(torch, sub, split=False)
    assert torch.equal(st2.out, st.out[2:4]) and torch.equal(st2.lse, st.lse[:, 2:4])


def test_split_matches_unsplit_within_rounding(torch):
    """Split rows differ from whole rows only by the rounding of the merge."""
    case = W.sparse_mqa(rows=3, heads=128, n_kv=2600, k=2048, seed=22)
    a = _check(torch, case, name="split")
    assert a.ws is not None and a.ws.numel() > 0
    b = _check(torch, case, split=False, name="unsplit")
    ao, bo = W.bf16_bits_to_f64(R.tensor_to_bits(a.out)), W.bf16_bits_to_f64(R.tensor_to_bits(b.out))
    assert_bf16_close(ao, bo, "split vs unsplit")


def test_split_empty_chunks_and_padding(torch):
    """k = 64 (two tiles, so two key ranges): a row with 5 valid entries (its
    first range is empty), an all-padding row (both empty: o = 0, lse =
    -inf), a row with one partial tile past a full one, a full row."""
    case = W.sparse_mqa(rows=4, heads=128, n_kv=500, k=64, seed=23)
    idx = case.topk_idx.copy()
    idx[0, 5:] = -1
    idx[1, :] = -1
    idx[2, 33:] = -1
    st = _check(torch, case, idx=idx, name="empty chunks")
    assert st.ws is not None
    out = W.bf16_bits_to_f64(R.tensor_to_bits(st.out))
    assert np.all(out[1] == 0) and np.all(st.lse[:, 1].cpu().numpy() == -np.inf)


def test_split_order_invariant_and_repeatable_bitwise(torch):
    """Key ranges are cut in sorted order, so the split output is still
    bitwise independent of the index order, and bitwise repeatable."""
    case = W.sparse_mqa(rows=3, heads=128, n_kv=2600, k=2048, seed=24)
    a = _run(torch, case)
    o0, l0 = a.out.clone(), a.lse.clone()
    R.run_sparse(a)
    torch.cuda.synchronize()
    assert torch.equal(a.out, o0) and torch.equal(a.lse, l0)
    for seed in (109, 110):
        b = _run(torch, case, W.permute_rows(case.topk_idx, seed))
        assert torch.equal(b.out, o0) and torch.equal(b.lse, l0)


def test_split_at_a_round_boundary(torch):
    """CUs + 3 rows: the first CUs rows run whole, the last 3 are split; both
    sides of the boundary against the oracle, two head blocks (200 heads)."""
    cus = _cus(torch)
    case = W.sparse_mqa(rows=cus + 3, heads=200, n_kv=900, k=320, seed=25)
    rows = [0, cus // 2 - 1, cus // 2, cus // 2 + 1, cus - 1, cus, cus + 1, cus + 2]
    st = _check(torch, case, rows=rows, name="round boundary")
    assert st.ws is not None


def test_workspace_too_small_is_rejected(torch):
    import vision_encoder_attention_amd as vea
    case = W.sparse_mqa(rows=3, heads=128, n_kv=500, k=256, seed=26)
    st = R.stage_sparse(case)
    need = vea.sparse_mqa_workspace_size(3, 128, case.d_qk, case.d_v, 256)
    assert need > 0 and st.ws.numel() == need
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(vea.VeaError) as e:
        vea.sparse_mqa_fwd(st.q, st.kv, st.idx, 256, case.scale, st.out, st.lse, workspace=small)
    assert e.value.status == -6


# ------------------------------------------------------------ paged cache

def _page_out(kv_bits, ps, extra_pages, seed):
    """Scatter a logical latent cache into shuffled physical pages, with
    unused garbage pages in between; returns (cache bits, page table)."""
    rng = np.random.default_rng(seed)
    n_kv, dqk = kv_bits.shape
    n_pages = -(-n_kv // ps)
    table = rng.permutation(n_pages + extra_pages)[:n_pages].astype(np.int32)
    cache = W.randn_bf16_bits(rng, ((n_pages + extra_pages) * ps, dqk))
    rows = oracle.paged_rows(table, ps, n_kv)
    cache[rows] = kv_bits
    return cache, table


def _run_paged(torch, case, cache, table, ps, idx=None):
    import vision_encoder_attention_amd as vea
    dev = "cuda"
    q = R.bits_to_tensor(case.q, dev)
    kvc = R.bits_to_tensor(cache, dev)
    pt = torch.from_numpy(table).to(dev)
    ix = torch.from_numpy(np.ascontiguousarray(case.topk_idx if idx is None else idx, np.int32)).to(dev)
    out = torch.empty((case.num_rows, case.num_heads, case.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.num_heads, case.num_rows), dtype=torch.float32, device=dev)
    vea.sparse_mqa_paged_fwd(q, kvc, pt, ps, case.kv_latent.shape[0], ix, ix.shape[1], case.scale, out, lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("ps", [1, 16, 64])
def test_paged_cache_against_the_oracle(torch, ps):
    """Logical positions resolved through a shuffled page table (garbage in
    the unused pages), with padding; against the oracle's paged view."""
    case = W.sparse_mqa(rows=5, heads=128, n_kv=700, k=256, seed=40 + ps)
    idx = case.topk_idx.copy()
    idx[1, ::4] = -1
    cache, table = _page_out(case.kv_latent, ps, extra_pages=5, seed=50 + ps)
    out, lse = _run_paged(torch, case, cache, table, ps, idx)
    o_ref, l_ref = oracle.sparse_mqa_paged(W.bf16_bits_to_f64(case.q), W.bf16_bits_to_f64(cache), table, ps,
                                           case.kv_latent.shape[0], idx, case.d_v, float(np.float32(case.scale)))
    assert_bf16_close(W.bf16_bits_to_f64(R.tensor_to_bits(out)), o_ref, "paged out")
    assert_bf16_close(lse.cpu().numpy().astype(np.float64), l_ref, "paged lse")


def test_paged_result_is_independent_of_page_placement(torch):
    """The full workload in two different page layouts (and with each row's
    indices in another order) gives bitwise the unpaged result: the indices
    are ordered by logical position before the table is applied."""
    case = W.full_case("sparse_mqa")
    st = _run(torch, case)
    for ps, seed in ((64, 61), (16, 62)):
        cache, table = _page_out(case.kv_latent, ps, extra_pages=9, seed=seed)
        out, lse = _run_paged(torch, case, cache, table, ps)
        assert torch.equal(out, st.out) and torch.equal(lse, st.lse), ps
    out, lse = _run_paged(torch, case, cache, table, 16, W.permute_rows(case.topk_idx, 111))
    assert torch.equal(out, st.out) and torch.equal(lse, st.lse)
