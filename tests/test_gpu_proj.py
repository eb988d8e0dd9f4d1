"""GPU parity of the fused QKV projection with its RoPE epilogue
(vea_qkv_proj_rope) and of the rotation table (vea_rope_cos_sin), against
the float64 oracle on the same seeded inputs.

Tolerance of the projection, per output element: |got - ref| <= one bf16 ulp
of ref + 1e-5 * rms(ref).  The kernel rounds an fp32 value to bf16 once
(half an ulp); fp32 accumulation over hidden <= 4096 products and the fp32
table add far less than the other half.  The general bf16 bar (max abs 2e-2,
cosine 0.999) is checked as well.  The table: within one fp32 ulp of the
oracle's float64 cos / sin."""
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


def _f64(t):
    return W.bf16_bits_to_f64(R.tensor_to_bits(t))


def _assert_ulp(got, ref, name):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt((ref * ref).mean())) if ref.size else 0.0
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126)))
    tol = 2.0 ** (e - 7) + 1e-5 * rms
    err = np.abs(got - ref)
    bad = np.argwhere(err > tol)
    log("  %-10s max err/ulp-bound %.3f over %d values" % (name, float((err / tol).max()) if ref.size else 0.0,
                                                         ref.size))
    assert bad.size == 0, "%s: %d values beyond one bf16 ulp, first at %s: got %r want %r" % (
        name, len(bad), bad[0], got[tuple(bad[0])], ref[tuple(bad[0])])
    if ref.size:
        assert_bf16_close(got, ref, name)


def _oracle(case, rows=None, rotate=True):
    x = W.bf16_bits_to_f64(case.x if rows is None else case.x[rows])
    pos = case.positions if rows is None else case.positions[rows]
    b = None if case.bias is None else W.bf16_bits_to_f64(case.bias)
    return oracle.qkv_proj_rope(x, W.bf16_bits_to_f64(case.w), b, pos, float(np.float32(case.theta)), case.hq,
                                case.hkv, case.d, rotate=rotate)


def _run(torch, case, rotate=True):
    st = R.stage_proj(case, rotate=rotate)
    R.run_rope_table(st)
    R.run_proj(st)
    torch.cuda.synchronize()
    return st


def _check(torch, case, rotate=True, name=""):
    log("proj %s T=%d hidden=%d h=%d/%d d=%d bias=%s rotate=%s" % (
        name, case.x.shape[0], case.x.shape[1], case.hq, case.hkv, case.d, case.bias is not None, rotate))
    st = _run(torch, case, rotate)
    q, k, v = _oracle(case, rotate=rotate)
    _assert_ulp(_f64(st.q), q, "q")
    _assert_ulp(_f64(st.k), k, "k")
    _assert_ulp(_f64(st.v), v, "v")
    return st


@pytest.mark.parametrize("t,hidden,hq,hkv,d,grid,bias", [
    (300, 96, 3, 1, 64, None, True),         # ragged tokens; 320 features: a ragged feature tile; 3 k-steps
    (667, 256, 4, 4, 64, (23, 29), False),   # a small image, 2D positions
    (129, 64, 2, 2, 128, None, True),        # d 128; two k-steps (one zero step in the ring)
    (1, 32, 1, 1, 32, None, True),           # one token, one k-step, head_dim 32
    (520, 1024, 8, 2, 128, None, False),     # GQA, 32 k-steps
])
def test_projection_against_the_oracle(torch, t, hidden, hq, hkv, d, grid, bias):
    case = W.qkv_proj(tokens=t, hidden=hidden, hq=hq, hkv=hkv, d=d, grid=grid, bias=bias, seed=700 + t)
    _check(torch, case, name="small")


def test_without_rotation_and_positions_zero(torch):
    """cos_sin NULL gives the plain projection split; positions all 0 give the
    same through the table (cos 1, sin 0)."""
    case = W.qkv_proj(tokens=200, hidden=128, hq=2, hkv=1, d=64, grid=None, bias=True, seed=711)
    plain = _check(torch, case, rotate=False, name="plain")
    case0 = W.ProjCase("zero", case.x, case.w, case.bias, np.zeros(200, np.int32), case.hq, case.hkv, case.d,
                       case.theta)
    st0 = _run(torch, case0)
    assert torch.equal(st0.q, plain.q) and torch.equal(st0.k, plain.k) and torch.equal(st0.v, plain.v)


def test_rotation_table_against_the_oracle(torch):
    for case in (W.vision_proj(), W.qkv_proj(tokens=3000, hidden=32, hq=1, hkv=1, d=128, grid=None, seed=712)):
        pos = case.positions.copy()
        if pos.ndim == 1:
            pos = pos * 11                                # positions up to ~33000
        c2 = W.ProjCase(case.name, case.x, case.w, None, pos.astype(np.int32), case.hq, case.hkv, case.d,
                        case.theta)
        st = R.stage_proj(c2)
        R.run_rope_table(st)
        torch.cuda.synchronize()
        got = st.cs.cpu().numpy().astype(np.float64)
        ref = oracle.rope_cos_sin(pos, float(np.float32(case.theta)), case.d)
        err = np.abs(got - ref).max()
        log("table %s d=%d max err %.3g" % (case.name, case.d, err))
        assert err <= 2.0 ** -23, err


@pytest.mark.parametrize("name", ["vision", "varlen"])
def test_full_size_whole_tensors_and_bitwise_repeat(torch, name):
    """The full projections (vision: 8547 x 1024 -> 3072, 2D; varlen: 32876 x
    4096 -> 6144, GQA, 1D): every element of q, k and v within one bf16 ulp
    of the oracle, and bitwise equal on a second run."""
    case = W.vision_proj() if name == "vision" else W.varlen_proj()
    t = case.x.shape[0]
    log("proj full %s T=%d hidden=%d" % (name, t, case.x.shape[1]))
    st = _run(torch, case)
    q, k, v = _oracle(case)
    _assert_ulp(_f64(st.q), q, "q")
    del q
    _assert_ulp(_f64(st.k), k, "k")
    _assert_ulp(_f64(st.v), v, "v")
    del k, v
    q1, k1, v1 = st.q.clone(), st.k.clone(), st.v.clone()
    R.run_proj(st)
    torch.cuda.synchronize()
    assert torch.equal(q1, st.q) and torch.equal(k1, st.k) and torch.equal(v1, st.v)


def test_projection_then_attention_matches_the_oracle_pipeline(torch):
    """x -> fused projection + 2D RoPE (GPU) -> attention over query pieces
    (GPU), against the same chain in the oracle (small image)."""
    import vision_encoder_attention_amd as vea
    case = W.qkv_proj(hidden=256, hq=4, hkv=4, d=64, grid=(23, 29), seed=714)
    st = _run(torch, case)
    t = case.x.shape[0]
    cu = torch.tensor([0, t], dtype=torch.int32, device="cuda")
    out = torch.empty_like(st.q)
    lse = torch.empty((case.hq, t), dtype=torch.float32, device="cuda")
    scale = 0.125
    vea.attn_fwd(st.q, st.k, st.v, cu, cu, False, scale, out, lse, piece_rows=150)
    torch.cuda.synchronize()
    q, k, v = _oracle(case)
    o_ref, l_ref = oracle.attention(q, k, v, np.array([0, t]), np.array([0, t]), False, scale)
    assert_bf16_close(_f64(out), o_ref, "out")
    assert_bf16_close(lse.cpu().numpy().astype(np.float64), l_ref, "lse")


@pytest.mark.parametrize("d,grid", [(64, None), (128, None), (64, (13, 17)), (128, (13, 17))])
def test_rotate_half_pairing(torch, d, grid):
    """Rotate-half pairs (i, i + span/2), span d (1D) or d/2 (2D): the fused
    projection (with bias) and qkv_rope on its unrotated output, both against
    the oracle."""
    import vision_encoder_attention_amd as vea
    t = 221 if grid is None else grid[0] * grid[1]
    case = W.qkv_proj(tokens=t, hidden=96, hq=4, hkv=2, d=d, grid=grid, bias=True, seed=730 + d)
    span = d if grid is None else d // 2
    log("rotate-half d=%d span=%d" % (d, span))
    st = R.stage_proj(case)
    R.run_rope_table(st)
    vea.qkv_proj_rope(st.x, st.w, st.bias, st.cs, st.q, st.k, st.v, rotate_half_span=span)
    torch.cuda.synchronize()
    x = W.bf16_bits_to_f64(case.x)
    b = W.bf16_bits_to_f64(case.bias)
    th = float(np.float32(case.theta))
    q, k, v = oracle.qkv_proj_rope(x, W.bf16_bits_to_f64(case.w), b, case.positions, th, case.hq, case.hkv, d,
                                   rotate_half=True)
    _assert_ulp(_f64(st.q), q, "q")
    _assert_ulp(_f64(st.k), k, "k")
    _assert_ulp(_f64(st.v), v, "v")
    # qkv_rope on the (bf16) unrotated projection output, rotate-half
    plain = R.stage_proj(case, rotate=False)
    R.run_proj(plain)
    y = torch.cat([plain.q.reshape(t, -1), plain.k.reshape(t, -1), plain.v.reshape(t, -1)], 1).contiguous()
    qr = torch.empty_like(plain.q)
    kr = torch.empty_like(plain.k)
    vea.qkv_rope(y, st.positions, case.theta, qr, kr, rotate_half=True)
    torch.cuda.synchronize()
    q2, k2 = oracle.qkv_rope(_f64(y), case.positions, th, case.hq, case.hkv, d, rotate_half=True)
    assert_bf16_close(_f64(qr), q2, "qkv_rope q")
    assert_bf16_close(_f64(kr), k2, "qkv_rope k")
