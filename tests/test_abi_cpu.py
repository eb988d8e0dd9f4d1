"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status before
any launch.  Also checks the oracle / HIP path separation."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vea.h")

VEA_OK, VEA_EINVAL, VEA_EDTYPE, VEA_ESHAPE, VEA_EUNSUPPORTED, VEA_EWORKSPACE = 0, -1, -2, -3, -4, -6


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vea_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from vision_encoder_attention_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        pytest.fail("libvea.so is not built (run __graft_entry__.build())")
    return _binding.load_library()


def test_header_declares_the_operations():
    names = _declared()
    for n in ("vea_attn_fwd", "vea_attn_fwd_workspace_size", "vea_qkv_rope", "vea_sparse_mqa_fwd",
              "vea_sparse_mqa_workspace_size", "vea_topk_indices", "vea_sparse_mqa_paged_fwd", "vea_attn_fwd_paged", "vea_attn_decode", "vea_attn_decode_workspace_size",
              "vea_attn_probs_piece", "vea_status_str", "vea_rope_cos_sin", "vea_qkv_proj_rope",
              "vea_quantize_fp8", "vea_attn_fwd_fp8"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from vision_encoder_attention_amd import _binding
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (vea_[a-z0-9_]+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert lib.vea_status_str(st).decode().startswith("VEA_")
    assert lib.vea_version().decode().startswith("vea ")


FAKE = 0x10000   # 16-byte aligned, never dereferenced: every call below fails validation first


def _attn(lib, **kw):
    a = dict(dtype=1, q=FAKE, qs=128, k=FAKE, ks=128, v=FAKE, vs=128, cuq=FAKE, cuk=FAKE, batch=1, tq=10, tk=10,
             mq=10, mk=10, hq=2, hkv=2, d=64, causal=0, scale=0.125, qb=0, out=FAKE, os=128, lse=None, ws=None,
             wsb=0)
    a.update(kw)
    return lib.vea_attn_fwd(a["dtype"], a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["cuq"], a["cuk"],
                            a["batch"], a["tq"], a["tk"], a["mq"], a["mk"], a["hq"], a["hkv"], a["d"],
                            a["causal"], a["scale"], a["qb"], a["out"], a["os"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), VEA_EDTYPE),
    (dict(hq=3, hkv=2), VEA_ESHAPE),
    (dict(hkv=0), VEA_ESHAPE),
    (dict(batch=-1), VEA_ESHAPE),
    (dict(qb=-5), VEA_ESHAPE),
    (dict(d=96), VEA_EUNSUPPORTED),
    (dict(dtype=0, d=128), VEA_EUNSUPPORTED),
    (dict(scale=float("nan")), VEA_EINVAL),
    (dict(scale=float("inf")), VEA_EINVAL),
    (dict(causal=2), VEA_EINVAL),
    (dict(q=None), VEA_EINVAL),
    (dict(cuk=None), VEA_EINVAL),
    (dict(q=FAKE + 2), VEA_EINVAL),
    (dict(qs=100), VEA_ESHAPE),          # shorter than Hq * d
    (dict(vs=132), VEA_EINVAL),          # not a multiple of 16 bytes
    (dict(mq=11), VEA_ESHAPE),           # longer than total
    (dict(batch=0), VEA_OK),             # nothing to do, nothing launched
    (dict(tq=0, mq=0), VEA_OK),
    (dict(ws=FAKE + 8, wsb=1 << 20), VEA_EWORKSPACE),   # misaligned workspace
])
def test_attn_fwd_validation(lib, kw, status):
    assert _attn(lib, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((7, 1, 10, 10, 10, 10, 2, 2, 64, 0, 0), VEA_EDTYPE),
    ((1, 1, 10, 10, 10, 10, 3, 2, 64, 0, 0), VEA_ESHAPE),
    ((1, 1, 10, 10, 10, 10, 2, 2, 96, 0, 0), VEA_EUNSUPPORTED),
    ((1, 1, 10, 10, 11, 10, 2, 2, 64, 0, 0), VEA_ESHAPE),
    ((1, 1, 10, 10, 10, 10, 2, 2, 64, 2, 0), VEA_EINVAL),
    ((1, 0, 0, 0, 0, 0, 2, 2, 64, 0, 0), VEA_OK),
    ((1, 2, 10, 10, 5, 5, 2, 2, 64, 0, 0), VEA_OK),       # batch > 1: never split, no device query
    ((1, 1, 10, 10, 10, 10, 2, 2, 64, 1, 0), VEA_OK),     # causal: never split
    ((0, 1, 10, 10, 10, 10, 2, 2, 64, 0, 0), VEA_OK),     # fp32: never split
])
def test_attn_fwd_workspace_size_validation(lib, args, status):
    n = ctypes.c_size_t(12345)
    assert lib.vea_attn_fwd_workspace_size(*args, ctypes.byref(n)) == status
    assert n.value == 0
    assert lib.vea_attn_fwd_workspace_size(*args, None) == VEA_EINVAL


def _rope(lib, **kw):
    a = dict(x=FAKE, xs=3 * 4 * 64, pos=FAKE, pd=2, t=5, hq=4, hkv=4, d=64, theta=1e4, rh=0, q=FAKE, k=FAKE)
    a.update(kw)
    return lib.vea_qkv_rope(a["x"], a["xs"], a["pos"], a["pd"], a["t"], a["hq"], a["hkv"], a["d"], a["theta"],
                            a["rh"], a["q"], a["k"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(pd=3), VEA_EINVAL),
    (dict(rh=2), VEA_EINVAL),
    (dict(rh=1, d=48, xs=3 * 4 * 48), VEA_EUNSUPPORTED),      # rotate-half: whole chunks per half span
    (dict(theta=0.0), VEA_EINVAL),
    (dict(theta=-1.0), VEA_EINVAL),
    (dict(theta=float("nan")), VEA_EINVAL),
    (dict(d=36, xs=3 * 4 * 36), VEA_EUNSUPPORTED),
    (dict(d=512, xs=3 * 4 * 512), VEA_EUNSUPPORTED),
    (dict(xs=100), VEA_ESHAPE),
    (dict(x=None), VEA_EINVAL),
    (dict(k=FAKE + 8), VEA_EINVAL),
    (dict(t=-1), VEA_ESHAPE),
    (dict(t=0), VEA_OK),
])
def test_qkv_rope_validation(lib, kw, status):
    assert _rope(lib, **kw) == status


def _sparse(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, idx=FAKE, r=3, h=128, nkv=100, dqk=576, dv=512, k=64, scale=0.04, out=FAKE, lse=None,
             ws=None, wsb=0)
    a.update(kw)
    return lib.vea_sparse_mqa_fwd(a["q"], a["kv"], a["idx"], a["r"], a["h"], a["nkv"], a["dqk"], a["dv"], a["k"],
                                  a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dqk=512), VEA_EUNSUPPORTED),
    (dict(dv=600), VEA_ESHAPE),
    (dict(k=0), VEA_ESHAPE),
    (dict(k=5000), VEA_EUNSUPPORTED),
    (dict(scale=math.nan), VEA_EINVAL),
    (dict(idx=None), VEA_EINVAL),
    (dict(out=FAKE + 4), VEA_EINVAL),
    (dict(r=0), VEA_OK),
    (dict(ws=FAKE + 8, wsb=1 << 20), VEA_EWORKSPACE),
    (dict(nkv=-1), VEA_ESHAPE),
])
def test_sparse_validation(lib, kw, status):
    assert _sparse(lib, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((3, 128, 512, 512, 64), VEA_EUNSUPPORTED),
    ((3, 128, 576, 600, 64), VEA_ESHAPE),
    ((3, 0, 576, 512, 64), VEA_ESHAPE),
    ((3, 128, 576, 512, 0), VEA_ESHAPE),
    ((3, 128, 576, 512, 4097), VEA_EUNSUPPORTED),
    ((0, 128, 576, 512, 64), VEA_OK),
])
def test_sparse_workspace_size_validation(lib, args, status):
    n = ctypes.c_size_t(12345)
    assert lib.vea_sparse_mqa_workspace_size(*args, ctypes.byref(n)) == status
    assert n.value == 0
    assert lib.vea_sparse_mqa_workspace_size(*args, None) == VEA_EINVAL


def _attn_paged(lib, **kw):
    a = dict(q=FAKE, qs=128, kc=FAKE, ks=128, vc=FAKE, vs=128, bt=FAKE, mp=4, ps=64, npg=10, cuq=FAKE, cuk=FAKE,
             batch=2, tq=100, tk=100, mq=60, mk=60, hq=2, hkv=2, d=64, causal=1, scale=0.125, qb=0, out=FAKE, os=128,
             lse=None)
    a.update(kw)
    return lib.vea_attn_fwd_paged(a["q"], a["qs"], a["kc"], a["ks"], a["vc"], a["vs"], a["bt"], a["mp"], a["ps"],
                                  a["npg"], a["cuq"], a["cuk"], a["batch"], a["tq"], a["tk"], a["mq"], a["mk"],
                                  a["hq"], a["hkv"], a["d"], a["causal"], a["scale"], a["qb"], a["out"], a["os"],
                                  a["lse"], None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ps=32), VEA_ESHAPE),               # below the 64-key tile
    (dict(ps=96), VEA_ESHAPE),               # not a power of two
    (dict(mp=0), VEA_ESHAPE),                # fewer block-table columns than max_seqlen_k needs
    (dict(npg=-1), VEA_ESHAPE),
    (dict(bt=None), VEA_EINVAL),
    (dict(d=96), VEA_EUNSUPPORTED),
    (dict(batch=0), VEA_OK),
])
def test_attn_paged_validation(lib, kw, status):
    assert _attn_paged(lib, **kw) == status


def _decode(lib, **kw):
    a = dict(q=FAKE, qs=512, k=FAKE, ks=128, v=FAKE, vs=128, bt=None, mp=0, ps=0, npg=0, cuk=FAKE, batch=2, tk=100,
             mk=60, hq=8, hkv=2, d=64, scale=0.125, out=FAKE, os=512, lse=None)
    a.update(kw)
    return lib.vea_attn_decode(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["bt"], a["mp"], a["ps"], a["npg"],
                               a["cuk"], a["batch"], a["tk"], a["mk"], a["hq"], a["hkv"], a["d"], a["scale"],
                               a["out"], a["os"], a["lse"], None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), VEA_EUNSUPPORTED),
    (dict(hq=258, hkv=1), VEA_EUNSUPPORTED),  # a key/value head's query heads exceed one 128-row tile
    (dict(hq=6, hkv=4), VEA_ESHAPE),          # not a divisor
    (dict(mk=101), VEA_ESHAPE),               # packed: max_seqlen_k > total_k
    (dict(bt=FAKE, ps=32, mp=4, npg=10), VEA_ESHAPE),
    (dict(bt=FAKE, ps=64, mp=0, npg=10), VEA_ESHAPE),
    (dict(qs=256), VEA_ESHAPE),               # sequence stride shorter than Hq * d
    (dict(q=None), VEA_EINVAL),
    (dict(out=FAKE + 2), VEA_EINVAL),
    (dict(scale=float("nan")), VEA_EINVAL),
    (dict(batch=0), VEA_OK),
])
def test_attn_decode_validation(lib, kw, status):
    assert _decode(lib, **kw) == status
    n = ctypes.c_size_t(7)
    if status == VEA_EUNSUPPORTED:
        assert lib.vea_attn_decode_workspace_size(2, 60, kw.get("hq", 8), kw.get("hkv", 2), kw.get("d", 64),
                                                  ctypes.byref(n)) == status
        assert n.value == 0


def test_decode_binding_packed_total_k():
    """Packed K/V: the binding passes k's row count as total_k and rejects any
    other value, and k/v of unequal lengths (the kernel bounds its key rows by
    total_k, so a larger value would read past the buffers)."""
    from vision_encoder_attention_amd._binding import packed_total_k
    assert packed_total_k(100, 100) == 100
    assert packed_total_k(100, 100, 100) == 100
    assert packed_total_k(0, 0, None) == 0
    with pytest.raises(ValueError):
        packed_total_k(100, 100, 101)
    with pytest.raises(ValueError):
        packed_total_k(100, 100, 99)
    with pytest.raises(ValueError):
        packed_total_k(100, 99)


def _paged(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, pt=FAKE, ps=64, npg=41, idx=FAKE, r=3, h=128, nkv=2590, dqk=576, dv=512, k=64,
             scale=0.04, out=FAKE, lse=None)
    a.update(kw)
    return lib.vea_sparse_mqa_paged_fwd(a["q"], a["kv"], a["pt"], a["ps"], a["npg"], a["idx"], a["r"], a["h"],
                                        a["nkv"], a["dqk"], a["dv"], a["k"], a["scale"], a["out"], a["lse"], None, 0,
                                        None)


@pytest.mark.parametrize("kw,status", [
    (dict(ps=48), VEA_ESHAPE),               # not a power of two
    (dict(ps=0), VEA_ESHAPE),
    (dict(npg=-1), VEA_ESHAPE),
    (dict(pt=None), VEA_EINVAL),
    (dict(npg=1 << 20), VEA_EUNSUPPORTED),   # rows past 32-bit byte offsets
    (dict(dqk=512), VEA_EUNSUPPORTED),
    (dict(r=0), VEA_OK),
])
def test_sparse_paged_validation(lib, kw, status):
    assert _paged(lib, **kw) == status


def _topk(lib, **kw):
    a = dict(x=FAKE, rs=2590, st=None, ln=None, r=3, n=2590, k=2048, out=FAKE)
    a.update(kw)
    return lib.vea_topk_indices(a["x"], a["rs"], a["st"], a["ln"], a["r"], a["n"], a["k"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=4097, rs=4097), VEA_EUNSUPPORTED),
    (dict(k=0), VEA_ESHAPE),
    (dict(n=0), VEA_ESHAPE),
    (dict(r=-1), VEA_ESHAPE),
    (dict(rs=100), VEA_ESHAPE),              # row stride shorter than n
    (dict(x=None), VEA_EINVAL),
    (dict(out=FAKE + 2), VEA_EINVAL),        # not 4-byte aligned
    (dict(r=0), VEA_OK),
])
def test_topk_validation(lib, kw, status):
    assert _topk(lib, **kw) == status


def _proj(lib, **kw):
    a = dict(x=FAKE, xs=1024, w=FAKE, ws=3072, b=None, cs=None, t=100, hid=1024, hq=16, hkv=16, d=64, rh=0,
             q=FAKE, k=FAKE, v=FAKE)
    a.update(kw)
    return lib.vea_qkv_proj_rope(a["x"], a["xs"], a["w"], a["ws"], a["b"], a["cs"], a["t"], a["hid"], a["hq"],
                                 a["hkv"], a["d"], a["rh"], a["q"], a["k"], a["v"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(hid=1000, xs=1000), VEA_EUNSUPPORTED),   # hidden not a multiple of 32
    (dict(rh=48), VEA_EINVAL),                     # rotate-half span neither d nor d/2
    (dict(rh=96, d=96, ws=96 * 48), VEA_EUNSUPPORTED),   # rotate-half needs d 64 or 128
    (dict(d=48, ws=2304), VEA_EUNSUPPORTED),       # head_dim not a multiple of 32
    (dict(d=288, ws=288 * 48), VEA_EUNSUPPORTED),
    (dict(xs=512), VEA_ESHAPE),                    # x stride shorter than hidden
    (dict(ws=3000), VEA_ESHAPE),                   # w stride shorter than (Hq + 2 Hkv) d
    (dict(t=-1), VEA_ESHAPE),
    (dict(hkv=0), VEA_ESHAPE),
    (dict(x=None), VEA_EINVAL),
    (dict(v=None), VEA_EINVAL),
    (dict(w=FAKE + 8), VEA_EINVAL),                # misaligned
    (dict(b=FAKE + 4), VEA_EINVAL),
    (dict(cs=FAKE + 8), VEA_EINVAL),
    (dict(xs=1028), VEA_EINVAL),                   # stride not 16 bytes
    (dict(t=1 << 20), VEA_EUNSUPPORTED),           # x beyond 32-bit byte ranges
    (dict(hid=1 << 19, xs=1 << 19, t=1), VEA_EUNSUPPORTED),
    (dict(t=0), VEA_OK),
])
def test_qkv_proj_validation(lib, kw, status):
    assert _proj(lib, **kw) == status


def _fp8(lib, **kw):
    a = dict(q=FAKE, qs=128, k=FAKE, ks=128, v=FAKE, vs=128, qsc=FAKE, ksc=FAKE, vsc=FAKE, cuq=FAKE, cuk=FAKE,
             batch=1, tq=10, tk=10, mq=10, mk=10, hq=2, hkv=2, d=64, causal=0, scale=0.125, qb=0, out=FAKE, os=128,
             lse=None)
    a.update(kw)
    return lib.vea_attn_fwd_fp8(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["qsc"], a["ksc"], a["vsc"],
                                a["cuq"], a["cuk"], a["batch"], a["tq"], a["tk"], a["mq"], a["mk"], a["hq"],
                                a["hkv"], a["d"], a["causal"], a["scale"], a["qb"], a["out"], a["os"], a["lse"],
                                None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96, qs=192, ks=192, vs=192, os=192), VEA_EUNSUPPORTED),
    (dict(hq=3), VEA_ESHAPE),                       # Hq % Hkv
    (dict(qs=64), VEA_ESHAPE),                      # q stride shorter than a row
    (dict(qs=136), VEA_EINVAL),                     # stride not a multiple of 16 bytes
    (dict(qsc=None), VEA_EINVAL),
    (dict(vsc=None), VEA_EINVAL),
    (dict(vsc=FAKE + 4), VEA_EINVAL),               # v scales read 16 bytes at a time
    (dict(scale=float("nan")), VEA_EINVAL),
    (dict(causal=2), VEA_EINVAL),
    (dict(ks=1 << 25, vs=1 << 25), VEA_EUNSUPPORTED),
    (dict(tq=0, mq=0), VEA_OK),
])
def test_fp8_attention_validation(lib, kw, status):
    assert _fp8(lib, **kw) == status


def test_quantiser_validation(lib):
    f = lib.vea_quantize_fp8
    assert f(FAKE, 128, 10, 2, 64, 3, FAKE, FAKE, None) == VEA_EINVAL      # granularity
    assert f(FAKE, 128, 10, 2, 96, 0, FAKE, FAKE, None) == VEA_EUNSUPPORTED
    assert f(FAKE, 64, 10, 2, 64, 0, FAKE, FAKE, None) == VEA_ESHAPE       # stride shorter than a row
    assert f(FAKE, 128, -1, 2, 64, 0, FAKE, FAKE, None) == VEA_ESHAPE
    assert f(FAKE, 128, 10, 2, 64, 1, FAKE, None, None) == VEA_EINVAL
    assert f(FAKE + 8, 128, 10, 2, 64, 1, FAKE, FAKE, None) == VEA_EINVAL
    assert f(FAKE, 132, 10, 2, 64, 1, FAKE, FAKE, None) == VEA_EINVAL      # stride not 16 bytes
    assert f(FAKE, 128, 0, 2, 64, 0, FAKE, FAKE, None) == VEA_OK


def test_rope_table_validation(lib):
    f = lib.vea_rope_cos_sin
    assert f(FAKE, 3, 10, 64, 1e4, FAKE, None) == VEA_EINVAL          # pos_dims
    assert f(FAKE, 1, 10, 64, -1.0, FAKE, None) == VEA_EINVAL         # theta
    assert f(FAKE, 1, 10, 64, float("inf"), FAKE, None) == VEA_EINVAL
    assert f(FAKE, 1, 10, 63, 1e4, FAKE, None) == VEA_EUNSUPPORTED    # odd head_dim
    assert f(FAKE, 2, 10, 66, 1e4, FAKE, None) == VEA_EUNSUPPORTED    # 2D needs a multiple of 4
    assert f(FAKE, 1, 10, 512, 1e4, FAKE, None) == VEA_EUNSUPPORTED
    assert f(FAKE, 1, -1, 64, 1e4, FAKE, None) == VEA_ESHAPE
    assert f(None, 1, 10, 64, 1e4, FAKE, None) == VEA_EINVAL
    assert f(FAKE, 1, 10, 64, 1e4, FAKE + 4, None) == VEA_EINVAL      # table not 8-byte aligned
    assert f(FAKE, 1, 0, 64, 1e4, FAKE, None) == VEA_OK


def test_probs_validation(lib):
    f = lib.vea_attn_probs_piece
    # piece beyond its sequence
    assert f(1, FAKE, 128, FAKE, 128, FAKE, 50, 0, 2, 2, 64, 0, 10, 0, 10, 5, 6, 0, 0.1, FAKE, 10, None) == VEA_ESHAPE
    # p_out rows shorter than the sequence's keys
    assert f(1, FAKE, 128, FAKE, 128, FAKE, 50, 0, 2, 2, 64, 0, 10, 0, 10, 0, 5, 0, 0.1, FAKE, 9, None) == VEA_ESHAPE
    assert f(1, FAKE, 128, FAKE, 128, FAKE, 50, 2, 2, 2, 64, 0, 10, 0, 10, 0, 5, 0, 0.1, FAKE, 10, None) == VEA_ESHAPE
    assert f(5, FAKE, 128, FAKE, 128, FAKE, 50, 0, 2, 2, 64, 0, 10, 0, 10, 0, 5, 0, 0.1, FAKE, 10, None) == VEA_EDTYPE
    assert f(1, FAKE, 128, FAKE, 128, FAKE, 50, 0, 2, 2, 64, 0, 10, 0, 10, 0, 0, 0, 0.1, FAKE, 10, None) == VEA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    import vision_encoder_attention_amd as vea
    q = torch.zeros(4, 1, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        vea.attn_fwd(q, q, q, cu, cu, False, 0.125, q.clone())


# ------------------------------------------------------- separation checks

def _py_files(d):
    for base, _, files in os.walk(os.path.join(ROOT, d)):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(base, f)


def test_oracle_imports_nothing_from_the_hip_path():
    for f in _py_files("oracle"):
        src = open(f).read()
        imports = re.findall(r"^\s*(?:import|from)\s+([\w.]+)", src, flags=re.M)
        for mod in imports:
            assert not mod.startswith(("vision_encoder_attention_amd", "ctypes", "torch")), (f, mod)
        assert "libvea" not in src, f


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "vision_encoder_attention_amd")
    for base, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(base, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, flags=re.M), f
                assert "oracle/" not in src and "import oracle" not in src, f


def test_roctx_ranges_do_not_change_validation():
    """VEA_ROCTX=1 wraps every entry point in a roctx range (the library opens
    the roctx library on first use): calls still validate and return as
    before, in a fresh process where the variable is set from the start."""
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
from vision_encoder_attention_amd import _binding
lib = _binding.load_library()
a = [1, 0x10000, 128, 0x10000, 128, 0x10000, 128, 0x10000, 0x10000, 0, 0, 0, 0, 0, 8, 2, 64, 0, 0.125, 0,
     0x10000, 128, None, None, 0, None]
assert lib.vea_attn_fwd(*a) == 0                      # batch 0: nothing to compute
a[9] = 1; a[10] = 10; a[11] = 10; a[12] = 10; a[13] = 10; a[16] = 96
assert lib.vea_attn_fwd(*a) == -4                     # head_dim 96: unsupported
import os
if os.path.exists("/opt/rocm/lib/librocprofiler-sdk-roctx.so.1"):
    assert "rocprofiler-sdk-roctx" in open("/proc/self/maps").read(), "roctx library not opened"
print("ok")
""" % ROOT
    env = dict(os.environ, VEA_ROCTX="1")
    res = subprocess.run([os.sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stderr
