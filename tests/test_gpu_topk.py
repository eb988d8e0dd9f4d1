"""GPU parity of the deterministic top-k indexer against the oracle (bit-exact:
this is index work), and its composition with the sparse MQA kernel."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_bf16_close, log
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


def _run(torch, logits, k, starts=None, lens=None):
    import vision_encoder_attention_amd as vea
    x = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    out = torch.full((x.shape[0], k), 12345, dtype=torch.int32, device="cuda")
    st = None if starts is None else torch.from_numpy(np.asarray(starts, np.int32)).cuda()
    ln = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    vea.topk_indices(x, k, out, st, ln)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(torch, logits, k, starts=None, lens=None, name=""):
    log("topk %s rows=%d n=%d k=%d" % (name, logits.shape[0], logits.shape[1], k))
    got = _run(torch, logits, k, starts, lens)
    want = oracle.topk_indices(logits, k, starts, lens)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first mismatch at %s: got %d want %d" % (
        bad[0], got[tuple(bad[0])], want[tuple(bad[0])])
    return got


def test_full_size_indexer_with_ties_at_the_edge(torch):
    """[323, 2590] logits on a 1/16 grid (ties everywhere, including at the
    2048th position), row r seeing positions [0, 2268 + r): bit-exact, and
    bitwise the same on a second run."""
    case = W.indexer()
    got = _check(torch, case.logits, case.k, None, case.row_lens, "full")
    # the edge of the selection does split tie classes in this workload
    x = case.logits
    split = 0
    for r in range(0, x.shape[0], 17):
        kth = x[r, got[r, -1]]
        tied = np.flatnonzero(x[r, :case.row_lens[r]] == kth)
        split += int(0 < np.isin(tied, got[r]).sum() < tied.size)
    assert split > 0
    again = _run(torch, case.logits, case.k, None, case.row_lens)
    assert np.array_equal(got, again)


def test_continuous_logits(torch):
    rng = np.random.default_rng(31)
    _check(torch, rng.standard_normal((40, 2590), dtype=np.float32), 2048, name="continuous")
    _check(torch, rng.standard_normal((5, 4096), dtype=np.float32) * 50, 4096, name="n=k=4096")


def test_special_values(torch):
    """NaN after every number, +inf first, -inf last among numbers, -0.0 ties
    +0.0, all-equal rows keep position order."""
    rng = np.random.default_rng(32)
    x = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan], np.float32), size=(16, 333))
    _check(torch, x, 100, name="specials")
    _check(torch, np.full((3, 777), 2.5, np.float32), 500, name="all equal")
    _check(torch, np.full((2, 50), np.nan, np.float32), 60, name="all NaN")


def test_spans_padding_and_sizes(torch):
    """Row spans with starts and lengths (some shorter than k, some empty):
    absolute positions, -1 past the span; n not a power of two, n = 1, k > n."""
    rng = np.random.default_rng(33)
    n = 1500
    x = np.round(rng.standard_normal((30, n)) * 4).astype(np.float32)
    starts = rng.integers(0, n, 30)
    lens = np.array([int(rng.integers(0, n - s + 1)) for s in starts])
    lens[0], starts[0] = 0, 7
    lens[1] = n - starts[1]
    _check(torch, x, 300, starts, lens, "spans")
    _check(torch, x, 300, None, lens, "lens only")
    _check(torch, x[:, :1], 3, name="n=1")
    _check(torch, x[:, :97], 200, name="k>n")


def test_topk_then_sparse_attention_matches_the_oracle_pipeline(torch):
    """Indexer logits -> GPU top-k -> GPU sparse MQA, against oracle top-k ->
    oracle sparse MQA on the same inputs (reduced rows)."""
    import vision_encoder_attention_amd as vea
    ic = W.indexer(rows=12, n=700, k=256, seed=34)
    sc = W.sparse_mqa(rows=12, heads=128, n_kv=700, k=256, seed=35)
    idx_gpu = _check(torch, ic.logits, ic.k, None, ic.row_lens, "pipeline")
    case = W.SparseCase("pipeline", sc.q, sc.kv_latent, idx_gpu, sc.d_v, sc.scale)
    st = R.stage_sparse(case)
    R.run_sparse(st)
    torch.cuda.synchronize()
    idx_ref = oracle.topk_indices(ic.logits, ic.k, None, ic.row_lens)
    o_ref, l_ref = oracle.sparse_mqa(W.bf16_bits_to_f64(sc.q), W.bf16_bits_to_f64(sc.kv_latent), idx_ref, sc.d_v,
                                     float(np.float32(sc.scale)))
    assert_bf16_close(W.bf16_bits_to_f64(R.tensor_to_bits(st.out)), o_ref, "out")
    assert_bf16_close(st.lse.cpu().numpy().astype(np.float64), l_ref, "lse")
    assert vea is not None
