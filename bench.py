#!/usr/bin/env python3
"""Benchmark of the tiled-attention hot path on one MI355X.

A step is one pass of the dense hot path over the vision-encoder workload:
qkv_rope (fused QKV split + 2D-grid RoPE, 8547 tokens, 16 heads, d = 64) then
attn_fwd (non-causal, query pieces of 1462 rows).  Inputs are seeded synthetic
tensors already resident in device memory.  Prints ONE JSON line on stdout;
details go to stderr.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
    python bench.py --only WORKLOAD      (one workload, its JSON on stderr)

The other workloads (the fp32 single-head case, the varlen causal GQA
prefill, the 32K causal prefill, top-k sparse MQA, and the next-step kernels)
are timed too and reported under "workloads" in the same line, each with a
roofline object.  Kernel times come from HIP events recorded on the stream the
kernels run on (torch's current stream); mean, median and min over the timed
launches are reported.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 MFMA (twice the bf16 rate)
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 (matrix and vector)
EVICT_BYTES = 1 << 30          # a 1 GiB fill evicts L2 (4 MB per XCD) and the 256 MB MALL


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def dense_flops(case) -> float:
    """2 flops per MAC over Q K^T and P V, allowed (query, key) pairs only."""
    import numpy as np
    lq, lk = case.seqlens_q.astype(np.int64), case.seqlens_k.astype(np.int64)
    if case.causal:
        pairs = 0
        for a, b in zip(lq, lk):
            i = np.arange(a)
            pairs += int(np.clip(i + (b - a) + 1, 0, b).sum())
    else:
        pairs = int((lq * lk).sum())
    return 4.0 * case.head_dim * case.num_heads_q * pairs


def attn_bytes(case) -> float:
    """Algorithmic HBM bytes of one attn_fwd launch: q and out (Hq heads), k
    and v (Hkv heads) once each, and lse (fp32)."""
    e = 2 if case.dtype == "bf16" else 4
    d = case.head_dim
    return float(case.total_q * 2 * case.num_heads_q * d * e + case.total_k * 2 * case.num_heads_kv * d * e
                 + case.total_q * case.num_heads_q * 4)


def rope_bytes(case) -> float:
    """Algorithmic HBM bytes of qkv_rope: read Q and K columns, write q and k, read positions."""
    t = case.total_q
    qk = (case.num_heads_q + case.num_heads_kv) * case.head_dim * 2
    return float(t * (2 * qk + case.positions.itemsize * (case.positions.size // t)))


def sparse_bytes(case) -> float:
    """Gathered latent rows counted once per query row (all heads share them),
    plus Q, O, indices and lse."""
    r, h, dqk, dv, k = case.num_rows, case.num_heads, case.d_qk, case.d_v, case.k
    return float(r * k * dqk * 2 + r * h * dqk * 2 + r * h * dv * 2 + r * k * 4 + r * h * 4)


def indexer_bytes(case) -> float:
    """Logits of each row's span read once, the k indices written, the row
    lengths read."""
    lens = case.row_lens if case.row_lens is not None else [case.logits.shape[1]] * case.logits.shape[0]
    return float(sum(int(n) for n in lens) * 4 + case.logits.shape[0] * case.k * 4 + len(lens) * 4)


def sparse_flops(case) -> float:
    return 2.0 * case.num_rows * case.num_heads * case.k * (case.d_qk + case.d_v)


WARM_MS = 200.0   # untimed GPU work before any timed step


def warm_up(torch, fn, steps):
    """Untimed warmup: at least `steps` calls of fn and at least WARM_MS of
    wall time.  The GPU's clock ramps up over tens of milliseconds of
    sustained load (the vision step runs ~20% slower over its first ~80
    launches), so a fixed handful of warmup launches would time the ramp.
    Returns the number of calls made.  Python's cyclic garbage collector is
    off while the GPU is timed (main turns it off); it runs here instead,
    first, so that no collection pause falls between an event and the launch
    it times, and none leaves the GPU idle (and its clock falling) between the
    warm-up and the timed launches."""
    gc.collect()
    n = 0
    t0 = time.perf_counter()
    while n < steps or (time.perf_counter() - t0) * 1e3 < WARM_MS:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


_EVENT_POOL = []


def reserve_events(torch, n):
    """Create n event pairs and record each once, untimed.  The HIP event
    behind a torch event is created at its first record; made inside a timed
    loop, the first few hundred hold the host back long enough for the GPU to
    run dry between launches, and the idle time lands inside the timings."""
    fresh = []
    while len(_EVENT_POOL) + len(fresh) < n:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        fresh.append((e0, e1))
    torch.cuda.synchronize()
    _EVENT_POOL.extend(fresh)


class Timer:
    """Per-launch HIP event pairs on torch's current stream (the stream the
    binding launches the kernels on), taken from the pool that
    reserve_events fills, and returned to it once read."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}
        self.vals = {}

    def run(self, name, fn):
        if _EVENT_POOL:
            e0, e1 = _EVENT_POOL.pop()
        else:
            e0 = self.torch.cuda.Event(enable_timing=True)
            e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.pairs.setdefault(name, []).append((e0, e1))

    def times(self, name):
        """Milliseconds per launch (read once, after the caller's synchronize;
        the events then go back to the pool)."""
        if name not in self.vals:
            pairs = self.pairs.pop(name)
            self.vals[name] = [a.elapsed_time(b) for a, b in pairs]
            _EVENT_POOL.extend(pairs)
        return self.vals[name]

    def ms(self, name):
        v = self.times(name)
        return sum(v) / len(v), min(v)

    def stats(self, name):
        """mean, median and min in ms."""
        import statistics
        v = self.times(name)
        return {"mean": sum(v) / len(v), "median": statistics.median(v), "min": min(v)}


def roofline(bound, kernel, achieved, peak, unit, traffic_profile=None, algorithmic_bytes=None, **extra):
    """The roofline object of one kernel launch: achieved against the
    published peak, and the counter-measured HBM bytes per launch from a
    committed summary (null when absent or stale)."""
    r = {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4),
         "traffic": None}
    if traffic_profile:                                  # file name, or (file name, workload label)
        prof, entry = traffic_profile if isinstance(traffic_profile, tuple) else (traffic_profile, None)
        r["traffic"] = committed_traffic(prof, entry)
    if algorithmic_bytes is not None:
        r["algorithmic_bytes"] = algorithmic_bytes
    r.update(extra)
    return r


def rope_cold(torch, st, steps):
    """qkv_rope with L2 and MALL evicted before every launch (a 1 GiB fill,
    untimed): its inputs then come from HBM, as they would straight after
    the projection of a batch larger than the caches."""
    from vision_encoder_attention_amd import runner as R
    scratch = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")
    tm = Timer(torch)
    for _ in range(steps):
        scratch.fill_(1)
        tm.run("rope", lambda: R.run_rope(st))
    torch.cuda.synchronize()
    del scratch
    return tm.stats("rope")


def _r(x, n=4):
    return round(x, n)


def dense_entry(torch, wname, case, st, tm, steps, with_rope):
    """Workload entry of a dense bf16 case: attn_fwd times and roofline, and
    qkv_rope warm (inputs resident in L2 / MALL from the step before) and
    cold (L2 and MALL evicted before each launch)."""
    fl = dense_flops(case)
    a = tm.stats("attn_fwd")
    tflops = fl / a["mean"] / 1e9
    d, causal = case.head_dim, case.causal
    if d == 64 and not causal:
        kname = "attn_fwd_d64_kernel<false>"
    else:
        kname = "attn_fwd_bf16_kernel<%d,%s,false,false>" % (d, "true" if causal else "false")
    split = st.ws is not None
    if split:
        kname += " + attn_merge_kernel<%d>" % d
    prof = "attn_fwd_bf16_d%d%s_%s_counters.txt" % (d, "_causal" if causal else "", wname)
    ent = {"attn_fwd_ms": _r(a["mean"]), "attn_fwd_median_ms": _r(a["median"]), "attn_fwd_min_ms": _r(a["min"]),
           "attn_tflops": round(tflops, 2), "attn_frac_bf16_peak": _r(tflops / PEAK_BF16_TFLOPS),
           "flops": fl, "tokens": case.total_q, "causal": causal,
           "heads": [case.num_heads_q, case.num_heads_kv], "head_dim": d, "piece_rows": case.piece_rows,
           "last_round_split": split,
           "roofline": roofline("mfma", kname, tflops, PEAK_BF16_TFLOPS, "TFLOP/s", prof, attn_bytes(case))}
    if with_rope:
        rb = rope_bytes(case)
        r = tm.stats("qkv_rope")
        c = rope_cold(torch, st, steps)
        rprof = "qkv_rope_%s_counters.txt" % wname
        ent.update({"qkv_rope_ms": _r(r["mean"], 5), "qkv_rope_median_ms": _r(r["median"], 5),
                    "qkv_rope_min_ms": _r(r["min"], 5),
                    "qkv_rope_warm_gbs": round(rb / r["mean"] / 1e6, 1),
                    "qkv_rope_cold_ms": _r(c["mean"], 5), "qkv_rope_cold_median_ms": _r(c["median"], 5),
                    "qkv_rope_cold_min_ms": _r(c["min"], 5),
                    "qkv_rope_bytes": rb,
                    "qkv_rope_roofline": roofline("hbm", "qkv_rope_kernel (L2 and MALL evicted before each launch)",
                                                  rb / c["mean"] / 1e6, PEAK_HBM_GBS, "GB/s", rprof, rb)})
    return ent


def bench_vision(torch, args):
    """The headline step: qkv_rope then attn_fwd over the vision image.  After
    the warm-up, K steps run back to back between two synchronizations with
    nothing else on the stream; their wall time per step is the headline.  A
    second pass of K steps with one event pair per step gives the median and
    minimum of single steps, and a third times each kernel with its own
    events, for the rooflines."""
    from vision_encoder_attention_amd import runner as R
    from vision_encoder_attention_amd import workloads as W
    case = W.vision()
    st = R.stage_dense(case)
    args.warmup_done = warm_up(torch, lambda: R.run_dense(st), args.warmup)
    reserve_events(torch, 3 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        R.run_dense(st)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    steps = Timer(torch)
    for _ in range(args.steps):
        steps.run("step", lambda: R.run_dense(st))
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(args.steps):
        tm.run("qkv_rope", lambda: R.run_rope(st))
        tm.run("attn_fwd", lambda: R.run_attn(st))
    torch.cuda.synchronize()
    tm.vals["step"] = steps.times("step")
    ent = dense_entry(torch, "vision", case, st, tm, max(5, min(args.steps, 20)), with_rope=True)
    del st
    torch.cuda.empty_cache()
    return case, tm, wall_ms, ent


def bench_single_head(torch, steps, warmup):
    """The fp32 single-head case (N = 256, d 64, 4 pieces of 64): a
    latency-bound launch of 16 workgroups; TFLOP/s against the fp32 peak as
    context."""
    from vision_encoder_attention_amd import runner as R
    from vision_encoder_attention_amd import workloads as W
    case = W.single_head_f32()
    st = R.stage_dense(case)
    warm_up(torch, lambda: R.run_attn(st), max(1, warmup))
    tm = Timer(torch)
    for _ in range(steps):
        tm.run("attn_fwd", lambda: R.run_attn(st))
    torch.cuda.synchronize()
    fl = dense_flops(case)
    a = tm.stats("attn_fwd")
    tf = fl / a["mean"] / 1e9
    return {case.name: {"attn_fwd_us": round(a["mean"] * 1e3, 2), "attn_fwd_median_us": round(a["median"] * 1e3, 2),
                        "attn_fwd_min_us": round(a["min"] * 1e3, 2), "attn_tflops": round(tf, 4),
                        "flops": fl, "piece_rows": case.piece_rows,
                        "roofline": roofline("mfma", "attn_fwd_f32_kernel<64,false>", tf, PEAK_FP32_TFLOPS, "TFLOP/s",
                                             note="latency-bound: 8 workgroups of 128 rows for 1.7e7 flops")}}


def bench_dense(torch, name, steps, warmup):
    """varlen_gqa or long_causal: qkv_rope (varlen) and attn_fwd, each launch
    timed; the varlen batch also over 64-row pages."""
    from vision_encoder_attention_amd import runner as R
    from vision_encoder_attention_amd import workloads as W
    res = {}
    case = W.full_case(name)
    st = R.stage_dense(case)
    warm_up(torch, lambda: R.run_dense(st), max(1, warmup))
    tm = Timer(torch)
    for _ in range(steps):
        if case.x_qkv is not None:
            tm.run("qkv_rope", lambda: R.run_rope(st))
        tm.run("attn_fwd", lambda: R.run_attn(st))
    torch.cuda.synchronize()
    res[case.name] = dense_entry(torch, name, case, st, tm, steps, with_rope=case.x_qkv is not None)
    if name == "varlen_gqa":
        fl = dense_flops(case)
        p = bench_dense_paged(torch, st, steps, warmup)
        res[case.name + "_paged64"] = {"attn_fwd_ms": _r(p["mean"]), "attn_fwd_median_ms": _r(p["median"]),
                                       "attn_fwd_min_ms": _r(p["min"]),
                                       "attn_frac_bf16_peak": _r(fl / p["mean"] / 1e9 / PEAK_BF16_TFLOPS),
                                       "page_size": 64}
    del st
    torch.cuda.empty_cache()
    return res


WORKLOADS = ("single_head_f32", "vision", "varlen_gqa", "long_causal", "sparse_mqa", "indexer", "qkv_proj", "fp8",
             "decode")


def bench_other(torch, steps, warmup, only=None):
    """The workloads other than the headline step, each after its own warm-up
    (the clock ramps up over the first launches)."""
    res = {}
    want = (lambda n: only is None or n == only)
    if want("single_head_f32"):
        res.update(bench_single_head(torch, steps, warmup))
    for name in ("varlen_gqa", "long_causal"):
        if want(name):
            res.update(bench_dense(torch, name, steps, warmup))
    if want("sparse_mqa"):
        res.update(bench_sparse(torch, steps, warmup))
    if want("indexer"):
        res.update(bench_indexer(torch, steps, warmup))
    if want("qkv_proj"):
        res.update(bench_proj(torch, steps, warmup))
    if want("fp8"):
        res.update(bench_fp8(torch, steps, warmup))
    if want("decode"):
        res.update(bench_decode(torch, steps, warmup))
    return res


def bench_decode(torch, steps, warmup):
    """Decode over paged caches: 64 sequences of one query token each over
    512..8192 cached keys (GQA 32/8, d 128, 64-row pages in shuffled places)
    through attn_decode (a key/value head's 4 query heads in one workgroup,
    each cache cut into key ranges that are merged after), beside the
    prefill kernel on the same caches (attn_fwd_paged, one query row per
    128-row tile).  Decode reads the whole cache once per step, so the figure
    is the K/V read rate against HBM peak."""
    import numpy as np
    import vision_encoder_attention_amd as vea
    from vision_encoder_attention_amd import runner as R
    from vision_encoder_attention_amd import workloads as W
    case = W.decode()
    lk = [int(x) for x in np.diff(np.asarray(case.cu_seqlens_k, np.int64))]
    st = R.stage_dense(case)
    prefill_ms = bench_dense_paged(torch, st, steps, warmup)["mean"]
    kc, vc, btd = paged_copy(torch, st, 64)
    out = torch.empty_like(st.q)
    lse = torch.empty((32, 64), dtype=torch.float32, device="cuda")
    nbytes = vea.attn_decode_workspace_size(64, max(lk), 32, 8, 128)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")

    def run():
        vea.attn_decode(st.q, kc, vc, st.cu_k, c_scale, out, lse, block_table=btd, page_size=64,
                        max_seqlen_k=max(lk), total_k=sum(lk), workspace=ws if nbytes else None)

    c_scale = case.scale
    warm_up(torch, run, max(1, warmup))
    tm = Timer(torch)
    for _ in range(steps):
        tm.run("decode", run)
    torch.cuda.synchronize()
    t = tm.stats("decode")
    kv_bytes = float(sum(lk)) * 8 * 128 * 2 * 2
    name = case.name + "_paged64"
    res = {name: {"attn_decode_ms": _r(t["mean"]), "attn_decode_median_ms": _r(t["median"]),
                  "attn_decode_min_ms": _r(t["min"]), "kv_bytes": kv_bytes,
                  "kv_gbs": round(kv_bytes / t["mean"] / 1e6, 1),
                  "kv_frac_hbm": _r(kv_bytes / t["mean"] / 1e6 / PEAK_HBM_GBS),
                  "workspace_bytes": nbytes, "prefill_kernel_ms": _r(prefill_ms),
                  "roofline": roofline("hbm", "attn_fwd_bf16_kernel<128,false,true,true> + attn_merge_kernel<128>",
                                       kv_bytes / t["mean"] / 1e6, PEAK_HBM_GBS, "GB/s", None, kv_bytes)}}
    del st, kc, vc, ws
    torch.cuda.empty_cache()
    return res


def paged_copy(torch, st, ps):
    """The staged case's K/V copied into caches of shuffled ps-row pages (one
    block-table row per sequence)."""
    import numpy as np
    c = st.case
    lens = np.diff(np.asarray(c.cu_seqlens_k, np.int64))
    pages = [-(-int(n) // ps) for n in lens]
    n_pages = sum(pages) + 8
    order = np.random.default_rng(65).permutation(n_pages)
    bt = np.zeros((len(lens), max(pages)), np.int32)
    rows, nxt = [], 0
    for b, n in enumerate(lens):
        bt[b, :pages[b]] = order[nxt:nxt + pages[b]]
        nxt += pages[b]
        j = np.arange(int(n))
        rows.append(bt[b, j // ps].astype(np.int64) * ps + j % ps)
    idx = torch.from_numpy(np.concatenate(rows)).cuda()
    shape = (n_pages * ps,) + tuple(st.k.shape[1:])
    kc = torch.zeros(shape, dtype=st.k.dtype, device="cuda")
    vc = torch.zeros(shape, dtype=st.v.dtype, device="cuda")
    kc[idx] = st.k
    vc[idx] = st.v
    return kc, vc, torch.from_numpy(bt).cuda()


def bench_dense_paged(torch, st, steps, warmup, ps=64):
    """attn_fwd over the staged case's K/V copied into caches of shuffled
    64-row pages (one block-table row per sequence)."""
    import vision_encoder_attention_amd as vea
    c = st.case
    kc, vc, btd = paged_copy(torch, st, ps)

    def run():
        vea.attn_fwd_paged(st.q, kc, vc, btd, ps, st.cu_q, st.cu_k, c.causal, c.scale, st.out, st.lse,
                           piece_rows=c.piece_rows, max_seqlen_q=st.max_q, max_seqlen_k=st.max_k,
                           total_k=int(c.cu_seqlens_k[-1]), workspace=st.ws)

    warm_up(torch, run, max(1, warmup))
    tm = Timer(torch)
    for _ in range(steps):
        tm.run("paged", run)
    torch.cuda.synchronize()
    return tm.stats("paged")


def bench_sparse(torch, steps, warmup):
    """Sparse MQA on the full workload, first over a paged copy of the cache
    (64-row pages in shuffled places), then over the plain cache (the
    reported figure, timed last).  A 1 GiB fill between launches (untimed)
    evicts L2 and MALL."""
    import numpy as np
    import vision_encoder_attention_amd as vea
    from vision_encoder_attention_amd import runner as R
    from vision_encoder_attention_amd import workloads as W
    res = {}
    case = W.full_case("sparse_mqa")
    st = R.stage_sparse(case)
    scratch = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")
    by, fl = sparse_bytes(case), sparse_flops(case)

    def timed(name, fn):
        def fill_and_run():
            scratch.fill_(1)
            fn()
        warm_up(torch, fill_and_run, max(1, warmup))
        tm = Timer(torch)
        for _ in range(steps):
            scratch.fill_(1)
            tm.run(name, fn)
        torch.cuda.synchronize()
        return tm.stats(name)

    ps = 64
    rng = np.random.default_rng(64)
    n_pages = -(-case.kv_latent.shape[0] // ps)
    table = rng.permutation(n_pages + 8)[:n_pages].astype(np.int32)
    cache = np.zeros(((n_pages + 8) * ps, case.kv_latent.shape[1]), np.uint16)
    j = np.arange(case.kv_latent.shape[0])
    cache[table[j // ps] * ps + j % ps] = case.kv_latent
    kvc = R.bits_to_tensor(cache, "cuda")
    pt = torch.from_numpy(table).cuda()
    p = timed("paged", lambda: vea.sparse_mqa_paged_fwd(st.q, kvc, pt, ps, case.kv_latent.shape[0], st.idx,
                                                         case.k, case.scale, st.out, st.lse, workspace=st.ws))
    # the same index sets with each row independently permuted: the kernel sorts
    # every row first, so neither the time nor the bits may depend on the order
    prng = np.random.default_rng(65)
    perm = torch.from_numpy(np.stack([prng.permutation(row) for row in case.topk_idx]).astype(np.int32)).cuda()
    out_p, lse_p = torch.empty_like(st.out), torch.empty_like(st.lse)
    pm = timed("permuted", lambda: vea.sparse_mqa_fwd(st.q, st.kv, perm, case.k, case.scale, out_p, lse_p,
                                                      workspace=st.ws))
    t = timed("sparse", lambda: R.run_sparse(st))
    torch.cuda.synchronize()
    perm_equal = bool(torch.equal(out_p, st.out) and torch.equal(lse_p, st.lse))
    gbs = by / t["mean"] / 1e6
    res[case.name] = {"sparse_mqa_ms": _r(t["mean"]), "sparse_mqa_median_ms": _r(t["median"]),
                      "sparse_mqa_min_ms": _r(t["min"]), "gbs": round(gbs, 1),
                      "frac_hbm": _r(gbs / PEAK_HBM_GBS), "tflops": round(fl / t["mean"] / 1e9, 2),
                      "frac_bf16_peak": _r(fl / t["mean"] / 1e9 / PEAK_BF16_TFLOPS), "bytes": by, "flops": fl,
                      "roofline": roofline("hbm", "sparse_mqa_kernel<576,512,2048> + sparse_merge_kernel", gbs,
                                           PEAK_HBM_GBS, "GB/s", "sparse_mqa_counters.txt", by,
                                           mfma_frac=_r(fl / t["mean"] / 1e9 / PEAK_BF16_TFLOPS))}
    tr = res[case.name]["roofline"]["traffic"]
    if tr:
        res[case.name]["hbm_counter_gbs"] = round(tr / t["mean"] / 1e6, 1)
    res[case.name + "_paged64"] = {"sparse_mqa_ms": _r(p["mean"]), "sparse_mqa_median_ms": _r(p["median"]),
                                   "sparse_mqa_min_ms": _r(p["min"]), "gbs": round(by / p["mean"] / 1e6, 1),
                                   "frac_hbm": _r(by / p["mean"] / 1e6 / PEAK_HBM_GBS), "page_size": ps}
    res[case.name + "_rows_permuted"] = {"sparse_mqa_ms": _r(pm["mean"]), "sparse_mqa_median_ms": _r(pm["median"]),
                                         "sparse_mqa_min_ms": _r(pm["min"]),
                                         "frac_hbm": _r(by / pm["mean"] / 1e6 / PEAK_HBM_GBS),
                                         "bitwise_equal_to_unpermuted": perm_equal}
    del scratch, st, kvc, perm, out_p, lse_p
    torch.cuda.empty_cache()
    return res


def bench_indexer(torch, steps, warmup):
    """Top-k of the sparse indexer (the step before sparse MQA)."""
    import vision_encoder_attention_amd as vea
    from vision_encoder_attention_amd import workloads as W
    res = {}
    ic = W.indexer()
    x = torch.from_numpy(ic.logits).cuda()
    lens = torch.from_numpy(ic.row_lens).cuda()
    out = torch.empty((x.shape[0], ic.k), dtype=torch.int32, device="cuda")
    warm_up(torch, lambda: vea.topk_indices(x, ic.k, out, None, lens), max(1, warmup))
    tm = Timer(torch)
    for _ in range(steps):
        tm.run("topk", lambda: vea.topk_indices(x, ic.k, out, None, lens))
    torch.cuda.synchronize()
    t = tm.stats("topk")
    by = indexer_bytes(ic)
    res[ic.name] = {"topk_ms": _r(t["mean"]), "topk_median_ms": _r(t["median"]), "topk_min_ms": _r(t["min"]),
                    "gbs": round(by / t["mean"] / 1e6, 1), "frac_hbm": _r(by / t["mean"] / 1e6 / PEAK_HBM_GBS),
                    "bytes": by,
                    "note": "one workgroup per row sorts the row's keys in LDS; latency-bound, not HBM-bound"}
    return res


def bench_fp8(torch, steps, warmup):
    """FP8 (E4M3) attention on the vision image, the varlen batch and the 32K
    causal prefill: q, k, v quantised on the GPU (per (token, head), per head,
    per (head, channel)), then vea_attn_fwd_fp8; TFLOP/s against the dense
    FP8 MFMA peak, the bf16 kernel's time on the same shape beside it."""
    import vision_encoder_attention_amd as vea
    from vision_encoder_attention_amd import runner as R
    from vision_encoder_attention_amd import workloads as W
    res = {}
    for name in ("vision", "varlen_gqa", "long_causal"):
        case = W.full_case(name)
        st = R.stage_dense(case)
        if case.x_qkv is not None:
            R.run_rope(st)
        torch.cuda.synchronize()
        q = st.q if st.q.is_contiguous() else st.q.contiguous()
        k = st.k.contiguous()
        v = st.v.contiguous()

        def quant():
            return vea.quantize_fp8(q, 0), vea.quantize_fp8(k, 1), vea.quantize_fp8(v, 2)
        (q8, qs), (k8, ks), (v8, vs) = quant()
        out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((case.num_heads_q, case.total_q), dtype=torch.float32, device="cuda")

        def run():
            vea.attn_fwd_fp8(q8, qs, k8, ks, v8, vs, st.cu_q, st.cu_k, case.causal, case.scale, out, lse,
                             piece_rows=case.piece_rows, max_seqlen_q=st.max_q, max_seqlen_k=st.max_k)
        warm_up(torch, run, max(1, warmup))
        tm = Timer(torch)
        for _ in range(steps):
            tm.run("fp8", run)
            tm.run("quant", quant)
            tm.run("bf16", lambda: R.run_attn(st))
        torch.cuda.synchronize()
        fl = dense_flops(case)
        f = tm.stats("fp8")
        b_ms, _ = tm.ms("bf16")
        qn_ms, _ = tm.ms("quant")
        tf = fl / f["mean"] / 1e9
        res[case.name + "_fp8"] = {"attn_fwd_fp8_ms": _r(f["mean"]), "attn_fwd_fp8_median_ms": _r(f["median"]),
                                   "attn_fwd_fp8_min_ms": _r(f["min"]), "tflops": round(tf, 2),
                                   "frac_fp8_peak": _r(tf / PEAK_FP8_TFLOPS),
                                   "bf16_attn_fwd_ms": _r(b_ms), "quantize_qkv_ms": _r(qn_ms), "flops": fl,
                                   "roofline": roofline("mfma", "attn_fwd_fp8_kernel<%d,%s>" % (
                                       case.head_dim, "true" if case.causal else "false"), tf, PEAK_FP8_TFLOPS,
                                       "TFLOP/s", ("attn_fwd_fp8_hbm_counters.txt", FP8_PROFILE_ENTRY[name]))}
        del st, q, k, v, q8, k8, v8, out, lse
        torch.cuda.empty_cache()
    return res


def bench_proj(torch, steps, warmup):
    """Fused QKV projection + RoPE epilogue (the step before qkv_rope), on the
    vision image and the varlen batch; beside it the unfused form of the same
    step: the library GEMM (torch.matmul, hipBLASLt) followed by qkv_rope."""
    import vision_encoder_attention_amd as vea
    from vision_encoder_attention_amd import runner as R
    from vision_encoder_attention_amd import workloads as W
    res = {}
    for case, label in ((W.vision_proj(), "vision"), (W.varlen_proj(), "varlen")):
        st = R.stage_proj(case)
        R.run_rope_table(st)
        t, hid = case.x.shape
        n = (case.hq + 2 * case.hkv) * case.d
        y = torch.empty((t, n), dtype=torch.bfloat16, device="cuda")
        qr = torch.empty_like(st.q)
        kr = torch.empty_like(st.k)

        def unfused():
            torch.matmul(st.x, st.w, out=y)
            vea.qkv_rope(y, st.positions, case.theta, qr, kr)

        warm_up(torch, lambda: R.run_proj(st), max(1, warmup))
        warm_up(torch, unfused, 2)
        tm = Timer(torch)
        for _ in range(steps):
            tm.run("proj", lambda: R.run_proj(st))
            tm.run("table", lambda: R.run_rope_table(st))
            tm.run("unfused", unfused)
        torch.cuda.synchronize()
        fl = 2.0 * t * hid * n
        pr = tm.stats("proj")
        u_ms, _ = tm.ms("unfused")
        tb_ms, _ = tm.ms("table")
        tf = fl / pr["mean"] / 1e9
        res[case.name] = {"qkv_proj_rope_ms": _r(pr["mean"]), "qkv_proj_rope_median_ms": _r(pr["median"]),
                          "qkv_proj_rope_min_ms": _r(pr["min"]), "tflops": round(tf, 2),
                          "frac_bf16_peak": _r(tf / PEAK_BF16_TFLOPS), "flops": fl, "rope_table_ms": _r(tb_ms),
                          "unfused_matmul_plus_qkv_rope_ms": _r(u_ms),
                          "roofline": roofline("mfma", "qkv_proj_kernel", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                               ("qkv_proj_hbm_counters.txt", "%s %d x %d -> %d" % (label, t, hid, n)))}
        del st, y, qr, kr
        torch.cuda.empty_cache()
    return res


# workload labels of the FP8 counter summary, by workload
FP8_PROFILE_ENTRY = {"vision": "vision 8547 tokens, 16 heads, d 64",
                     "varlen_gqa": "varlen 32876 tokens, 32/8 heads, d 128, causal",
                     "long_causal": "32K causal, 16 heads, d 128"}


def committed_traffic(profile: str, entry=None):
    """HBM bytes per launch recorded in a committed counter summary under
    profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter
    reads for a plain copy of known size), or None when the kernel source has
    changed since the counters were taken.  A summary that covers several
    workloads is read at the entry whose workload label is `entry`."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("RESULT "):
                rec = json.loads(line[len("RESULT "):])
    from vision_encoder_attention_amd.profsum import source_digest
    if not rec or rec.get("source_digest") != source_digest(rec["sources"]):
        return None
    if "entries" in rec:                                 # one summary for several workloads
        hit = [e for e in rec["entries"] if e.get("workload") == entry]
        return hit[0]["hbm_bytes_per_launch"] if hit else None
    return rec.get("hbm_bytes_per_launch")


def host_info(workers):
    """The host facts reported with the oracle timings."""
    import platform
    import numpy as np
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = "%s %s (%s)" % (i.get("internal_api"), i.get("version"), i.get("architecture"))
                break
    except Exception:
        pass
    from oracle.pool import host_cores
    return {"cores_visible": host_cores(), "oracle_threads": workers, "cpu_model": model,
            "numpy": np.__version__, "blas": blas}


def cpu_oracle(workers):
    """The float64 oracle timed on the host cores, per workload, on the same
    seeded inputs the GPU ran, every workload whole (about 12 s on a 16-core
    host, about a minute on 8 cores).  Independent
    (sequence, head, row block) units run on ``workers`` threads, BLAS on one
    thread per worker.  Returns (headline baseline object, per-workload
    timings)."""
    import numpy as np
    import oracle
    from vision_encoder_attention_amd import workloads as W
    per = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # fp32 single head: the whole case, repeated for a stable figure
    c = W.single_head_f32()
    n_rep = 20
    dt = timed(lambda: [oracle.attention(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, False,
                                         float(np.float32(c.scale))) for _ in range(n_rep)]) / n_rep
    per[c.name] = {"oracle_ms": round(dt * 1e3, 3), "sample": "whole case", "gflops": round(dense_flops(c) / dt / 1e9, 2)}

    # vision: the whole step (RoPE of every token, attention of every head)
    c = W.vision()
    x64, v64 = W.bf16_bits_to_f64(c.x_qkv), W.bf16_bits_to_f64(c.v_from_x())
    box = {}

    def vision_step():
        q, k = oracle.qkv_rope(x64, c.positions, c.theta, c.num_heads_q, c.num_heads_kv, c.head_dim)
        box["t_rope"] = time.perf_counter()
        oracle.attention(q, k, v64, c.cu_seqlens_q, c.cu_seqlens_k, False, float(np.float32(c.scale)),
                         workers=workers)
    t0 = time.perf_counter()
    vision_s = timed(vision_step)
    rope_s = box["t_rope"] - t0
    vfl = dense_flops(c)
    per[c.name] = {"oracle_s": round(vision_s, 3), "qkv_rope_s": round(rope_s, 3), "sample": "whole step",
                   "gflops": round(vfl / (vision_s - rope_s) / 1e9, 2)}
    headline = {"value": round(vfl / vision_s / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
                "sample": "float64 oracle on the whole vision step: qkv_rope of all 8547 tokens + attention of all "
                          "16 heads x 8547 rows (%.4g attention flops in %.2f s on %d host threads)"
                          % (vfl, vision_s, workers)}
    del x64, v64

    # varlen GQA: RoPE of every token, then attention of every head
    c = W.varlen_gqa()
    x64, v64 = W.bf16_bits_to_f64(c.x_qkv), W.bf16_bits_to_f64(c.v_from_x())
    box = {}

    def varlen_step():
        q, k = oracle.qkv_rope(x64, c.positions, c.theta, c.num_heads_q, c.num_heads_kv, c.head_dim)
        box["t_rope"] = time.perf_counter()
        oracle.attention(q, k, v64, c.cu_seqlens_q, c.cu_seqlens_k, True, float(np.float32(c.scale)),
                         workers=workers)
    t0 = time.perf_counter()
    dt = timed(varlen_step)
    rope_s = box["t_rope"] - t0
    per[c.name] = {"oracle_s": round(dt, 3), "qkv_rope_s": round(rope_s, 3), "sample": "whole step",
                   "gflops": round(dense_flops(c) / (dt - rope_s) / 1e9, 2)}
    del x64, v64

    # 32K causal: every head
    c = W.long_causal()
    q, k, v = (W.bf16_bits_to_f64(a) for a in (c.q, c.k, c.v))
    dt = timed(lambda: oracle.attention(q, k, v, c.cu_seqlens_q, c.cu_seqlens_k, True, float(np.float32(c.scale)),
                                        workers=workers))
    per[c.name] = {"oracle_s": round(dt, 3), "sample": "whole workload", "gflops": round(dense_flops(c) / dt / 1e9, 2)}
    del q, k, v

    # sparse MQA: the whole workload
    c = W.sparse_mqa()
    q, kv = W.bf16_bits_to_f64(c.q), W.bf16_bits_to_f64(c.kv_latent)
    dt = timed(lambda: oracle.sparse_mqa(q, kv, c.topk_idx, c.d_v, float(np.float32(c.scale)), workers=workers))
    per[c.name] = {"oracle_s": round(dt, 3), "sample": "whole workload",
                   "gbs": round(sparse_bytes(c) / dt / 1e9, 3), "gflops": round(sparse_flops(c) / dt / 1e9, 2)}
    return headline, per


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--only", choices=WORKLOADS,
                    help="only run one workload (for profiling one kernel family); its JSON goes to stderr")
    ap.add_argument("--oracle-only", action="store_true", help="only time the CPU oracle (no GPU needed)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        err("bench.py measures one GPU: this library's path runs on a single MI355X "
            "(every workload here fits one GPU; multi-GPU sharding is described in DESIGN.md, not run). "
            "Use --gpus 1.")
        sys.exit(2)
    from oracle.pool import host_cores
    workers = max(1, min(16, host_cores()))
    if args.oracle_only:
        head, per = cpu_oracle(workers)
        err(json.dumps({"cpu_baseline": head, "per_workload": per, "host": host_info(workers)}))
        return

    import torch
    import vision_encoder_attention_amd as vea
    if not torch.cuda.is_available():
        err("no GPU visible")
        sys.exit(1)
    vea.load_library()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    err("device: %s, %d CUs" % (props.name, props.multi_processor_count))

    if args.calibrate_copy:
        n = 512 << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        err("copied %d bytes 3 times (expect FETCH_SIZE and WRITE_SIZE of %d KiB per copy)" % (n, n >> 10))
        return
    reserve_events(torch, 3 * max(args.steps, 20))
    gc.disable()                                         # collections run in warm_up, not while timing
    if args.only == "vision":
        case, tm, wall_ms, ent = bench_vision(torch, args)
        err(json.dumps({case.name: ent}))
        return
    if args.only:
        res = bench_other(torch, max(3, min(args.steps, 20)), args.warmup, only=args.only)
        err(json.dumps(res))
        return

    case, tm, wall_ms, vis = bench_vision(torch, args)
    fl = dense_flops(case)
    step = tm.stats("step")
    err("vision: step %.4f ms (wall), attn_fwd %.4f ms avg (%.1f TFLOP/s), qkv_rope %.4f ms warm, %.4f ms cold"
        % (wall_ms, vis["attn_fwd_ms"], vis["attn_tflops"], vis["qkv_rope_ms"], vis["qkv_rope_cold_ms"]))

    line = {
        "metric": "attention fwd TFLOP/s (qkv_rope + piecewise attn_fwd step), % of bf16 MFMA peak",
        "value": round(fl / wall_ms / 1e9, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup_done,
        "warmup_requested": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "ms_per_step_median": round(step["median"], 5),
        "ms_per_step_min": round(step["min"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "vision_encoder_8547tok_111x77grid_h16_d64_qb1462_2dRoPE",
                   "tokens": case.total_q, "heads": case.num_heads_q, "head_dim": case.head_dim,
                   "piece_rows": case.piece_rows, "causal": False, "flops_per_step": fl},
        "kernels": {k: v for k, v in vis.items() if k.startswith(("attn_fwd", "qkv_rope")) and k != "qkv_rope_roofline"},
        "roofline": vis["roofline"],
        "rooflines": {"qkv_rope": vis["qkv_rope_roofline"]},
    }
    if not args.no_extra:
        line["workloads"] = bench_other(torch, max(5, min(args.steps, 20)), args.warmup)
        for k, v in line["workloads"].items():
            err("%s: %s" % (k, v))
    gc.enable()
    if not args.no_cpu_baseline:
        head, per = cpu_oracle(workers)
        head["per_workload"] = per
        head["host"] = host_info(workers)
        line["cpu_baseline"] = head
        err("cpu_baseline: %s" % json.dumps(head))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
