"""vea_attn_fwd_noalloc (the entry point for callers that cannot allocate)
against vea_attn_fwd with a caller workspace: the same kernels and the same
split plan, so the outputs must be bitwise equal.  Two calls in a row, the
second on a smaller input; also a call that needs no scratch at all."""
import numpy as np
import pytest

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


def _both(torch, case):
    import vision_encoder_attention_amd as vea
    st = R.stage_dense(case)
    R.run_rope(st)
    R.run_attn(st)                       # vea_attn_fwd with the workspace its split asks for
    torch.cuda.synchronize()
    out = torch.full_like(st.out, float("nan"))
    lse = torch.full_like(st.lse, float("nan"))
    vea.attn_fwd_noalloc(st.q, st.k, st.v, st.cu_q, st.cu_k, case.causal, case.scale, out, lse,
                         piece_rows=case.piece_rows, max_seqlen_q=st.max_q, max_seqlen_k=st.max_k)
    torch.cuda.synchronize()
    return st, out, lse


def test_noalloc_equals_the_workspace_entry_point(torch):
    import vision_encoder_attention_amd as vea
    from tests.gpu_util import first_split_tiles
    tiles = first_split_tiles(64) + 4
    cases = [W.vision(),                                             # the benchmarked image: 23.8 MB of split chunks
             W.vision(grid_rows=tiles, grid_cols=128, heads=16, d=64, piece_rows=128 * ((tiles + 1) // 2), seed=730),
             W.random_dense([5000], [5000], 16, 16, 128, False, "bf16", seed=731),   # d 128: the largest split
             W.random_dense([300, 77], [300, 77], 4, 2, 128, True, "bf16", seed=732)]  # no split: no scratch
    for i, case in enumerate(cases):
        need = vea.attn_fwd_workspace_size(1, case.batch, case.total_q, case.total_k, int(case.seqlens_q.max()),
                                           int(case.seqlens_k.max()), case.num_heads_q, case.num_heads_kv,
                                           case.head_dim, case.causal, case.piece_rows)
        log("noalloc case %d: %s, split workspace %d bytes" % (i, case.name, need))
        assert need <= (36 << 20)
        if i < 3:
            assert need > 0
        st, out, lse = _both(torch, case)
        assert torch.equal(out, st.out), case.name
        assert torch.equal(lse, st.lse), case.name
        assert bool(torch.isfinite(out.float()).all())
