"""Summaries of rocprofv3 output for the kernels of this library.

Two reports, each printed as text (the files under ``profiles/`` are these
reports, with the commands that produced the raw data):

* ``trace``: per-kernel call counts and durations from a
  ``rocprofv3 --kernel-trace --stats --output-format csv`` run, plus the
  average over each kernel's last N dispatches.  ``bench.py`` runs its timed
  launches after its warm-up ones, so the last N dispatches of a kernel are
  the timed window that the benchmark's HIP events cover.
* ``counters``: HBM bytes of one launch from a ``FETCH_SIZE`` run and a
  ``WRITE_SIZE`` run (KiB per dispatch), each scaled by what the same counter
  reads for a device-to-device copy of known size (``bench.py
  --calibrate-copy``), next to the launch's algorithmic bytes; optionally the
  MFMA counters of a third run.  The last line (``RESULT {...}``) is read
  back by ``bench.py``, which reports the traffic only while the kernel's
  sources still hash to the digest recorded there.

    python -m vision_encoder_attention_amd.profsum trace DIR [--last N] [--match TEXT ...]
    python -m vision_encoder_attention_amd.profsum counters --kernel TEXT --fetch DIR --write DIR
        --copy-fetch DIR --copy-write DIR --algorithmic-bytes B --sources FILE ... [--mfma DIR]
        [--extra DIR ...] [--also TEXT ...] [--last N]

``--also`` names kernels launched with the main one in the same call (a
merge kernel after a split); their bytes per dispatch are added to the
launch's traffic.  The MFMA and extra counters are the main kernel's.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 512 << 20          # size of bench.py --calibrate-copy


def _one(dir_, suffix):
    files = sorted(glob.glob(os.path.join(dir_, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, dir_))
    return files[0]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def source_digest(paths) -> str:
    """sha256 over the sources a kernel is built from.  "file#Name" stands for
    the part of a shared header the kernel uses: the text of its parameter
    struct Name plus the header's typedef and constexpr lines, so additions
    for other kernels do not invalidate a summary."""
    h = hashlib.sha256()
    for pth in paths:
        name = None
        if "#" in pth:
            pth, name = pth.split("#", 1)
        with open(os.path.join(ROOT, pth), "rb") as f:
            data = f.read()
        if name is not None:
            text = data.decode()
            m = re.search(r"^struct %s \{.*?^\};" % re.escape(name), text, re.S | re.M)
            if m is None:
                raise ValueError("struct %s not found in %s" % (name, pth))
            keep = [ln for ln in text.splitlines() if ln.startswith(("typedef", "constexpr"))]
            data = (m.group(0) + "\n" + "\n".join(keep)).encode()
        h.update(data)
    return h.hexdigest()[:16]


def trace_report(dir_, last=20, match=None):
    rows = _rows(_one(dir_, "_kernel_trace.csv"))
    per = {}
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    out = ["%-96s %6s %10s %10s %10s %10s %10s" % ("kernel", "calls", "avg_us", "min_us", "max_us",
                                                    "last%d_avg" % last, "last%d_med" % last)]
    order = sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1]))
    for name, ds in order:
        if match and not any(m in name for m in match):
            continue
        ds.sort()
        dur = [d for _, d in ds]
        tail = dur[-last:]
        out.append("%-96s %6d %10.2f %10.2f %10.2f %10.2f %10.2f" % (
            name[:96], len(dur), sum(dur) / len(dur), min(dur), max(dur), sum(tail) / len(tail),
            statistics.median(tail)))
    return "\n".join(out)


def _counter(dir_, counter, kernel):
    vals = []
    for r in _rows(_one(dir_, "_counter_collection.csv")):
        if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
            vals.append((int(r["Dispatch_Id"]), float(r["Counter_Value"]), r["Kernel_Name"]))
    vals.sort()
    return vals


def counters_report(kernel, fetch, write, copy_fetch, copy_write, algorithmic_bytes, sources, mfma=None, last=0,
                    extra=None, xcds=8, simds=1024, also=None):
    out = []
    f = _counter(fetch, "FETCH_SIZE", kernel)
    w = _counter(write, "WRITE_SIZE", kernel)
    if not f or not w:
        raise SystemExit("kernel %r not found in the counter runs" % kernel)
    full_name = f[0][2]
    more = []                                            # (name, fetch KiB, write KiB) per dispatch of the --also kernels
    for k in also or []:
        fa = _counter(fetch, "FETCH_SIZE", k)
        wa = _counter(write, "WRITE_SIZE", k)
        if not fa or not wa:
            raise SystemExit("kernel %r not found in the counter runs" % k)
        fva = [v for _, v, _ in fa][-last:] if last else [v for _, v, _ in fa]
        wva = [v for _, v, _ in wa][-last:] if last else [v for _, v, _ in wa]
        more.append((fa[0][2], statistics.mean(fva), statistics.mean(wva), len(fva)))
    cf = [v for _, v, _ in _counter(copy_fetch, "FETCH_SIZE", "copyBuffer")]
    cw = [v for _, v, _ in _counter(copy_write, "WRITE_SIZE", "copyBuffer")]
    fs = (COPY_BYTES >> 10) / statistics.median(cf)
    ws = (COPY_BYTES >> 10) / statistics.median(cw)
    fv = [v for _, v, _ in f][-last:] if last else [v for _, v, _ in f]
    wv = [v for _, v, _ in w][-last:] if last else [v for _, v, _ in w]
    rd = statistics.mean(fv) * 1024 * fs
    wr = statistics.mean(wv) * 1024 * ws
    out.append("kernel: %s" % full_name)
    out.append("  FETCH_SIZE per dispatch (KiB): mean %.0f, min %.0f, max %.0f over %d dispatches"
               % (statistics.mean(fv), min(fv), max(fv), len(fv)))
    out.append("  WRITE_SIZE per dispatch (KiB): mean %.0f, min %.0f, max %.0f over %d dispatches"
               % (statistics.mean(wv), min(wv), max(wv), len(wv)))
    for name, fm, wm, n in more:
        out.append("launched with it: %s" % name)
        out.append("  FETCH_SIZE per dispatch (KiB): mean %.0f over %d dispatches" % (fm, n))
        out.append("  WRITE_SIZE per dispatch (KiB): mean %.0f over %d dispatches" % (wm, n))
        rd += fm * 1024 * fs
        wr += wm * 1024 * ws
        full_name += " + " + name
    out.append("copy calibration (__amd_rocclr_copyBuffer, %d KiB read + %d KiB written):"
               % (COPY_BYTES >> 10, COPY_BYTES >> 10))
    out.append("  FETCH_SIZE %s -> scale %.4f" % ([round(x) for x in cf], fs))
    out.append("  WRITE_SIZE %s -> scale %.4f" % ([round(x) for x in cw], ws))
    out.append("")
    out.append("HBM bytes per launch: read %.4g + written %.4g = %.4g" % (rd, wr, rd + wr))
    out.append("algorithmic bytes per launch: %.4g  (ratio %.3f)" % (algorithmic_bytes, (rd + wr) / algorithmic_bytes))
    rec = {"kernel": full_name, "hbm_bytes_per_launch": int(round(rd + wr)), "read_bytes": int(round(rd)),
           "write_bytes": int(round(wr)), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "algorithmic_bytes": int(algorithmic_bytes), "sources": list(sources),
           "source_digest": source_digest(sources)}
    means = {}
    for run in ([mfma] if mfma else []) + list(extra or []):
        rows = [r for r in _rows(_one(run, "_counter_collection.csv")) if kernel in r["Kernel_Name"]]
        for n in sorted(set(r["Counter_Name"] for r in rows)):
            vs = [(int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows if r["Counter_Name"] == n]
            vs.sort()
            vv = [v for _, v in vs][-last:] if last else [v for _, v in vs]
            means[n] = statistics.mean(vv)
    if means:
        out.append("")
        out.append("counter means per dispatch (summed over the device's XCDs / SEs / SIMDs):")
        for n in sorted(means):
            out.append("  %-32s %.6g" % (n, means[n]))
        gui = means.get("GRBM_GUI_ACTIVE")
        cyc = gui / xcds if gui else None           # kernel cycles (GUI_ACTIVE is summed over the XCDs)
        for n in means:
            if n.startswith("SQ_INSTS_VALU_MFMA_MOPS_"):
                out.append("  %s x 512 = %.4g MFMA flops per launch" % (n, means[n] * 512))
                rec["mfma_flops_per_launch"] = means[n] * 512
        if cyc:
            out.append("  kernel cycles (GRBM_GUI_ACTIVE / %d XCDs): %.6g" % (xcds, cyc))
            rec["kernel_cycles"] = cyc
            if "SQ_VALU_MFMA_BUSY_CYCLES" in means:
                f = means["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)
                out.append("  MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (cycles x %d SIMDs) = %.3f" % (simds, f))
                rec["mfma_busy_frac"] = round(f, 4)
            if "SQ_ACTIVE_INST_VALU" in means and "SQ_WAVE_CYCLES" in means:
                out.append("  VALU-active share of wave cycles: SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES = %.3f"
                           % (means["SQ_ACTIVE_INST_VALU"] / means["SQ_WAVE_CYCLES"]))
            if "SQ_INSTS_VALU" in means:
                out.append("  VALU instructions per SIMD-cycle: SQ_INSTS_VALU / (cycles x %d SIMDs) = %.3f"
                           % (simds, means["SQ_INSTS_VALU"] / (cyc * simds)))
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in means:
                out.append("  MFMA co-execution: SQ_VALU_MFMA_COEXEC_CYCLES / (cycles x %d SIMDs) = %.3f"
                           % (simds, means["SQ_VALU_MFMA_COEXEC_CYCLES"] / (cyc * simds)))
        if "TCC_HIT_sum" in means and "TCC_MISS_sum" in means:
            req = means["TCC_HIT_sum"] + means["TCC_MISS_sum"]
            if req > 0:
                out.append("  L2 hit rate: TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) = %.3f" % (means["TCC_HIT_sum"] / req))
                rec["l2_hit_rate"] = round(means["TCC_HIT_sum"] / req, 4)
    out.append("")
    out.append("RESULT " + json.dumps(rec))
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--last", type=int, default=20)
    t.add_argument("--match", nargs="*")
    c = sub.add_parser("counters")
    c.add_argument("--kernel", required=True)
    for n in ("fetch", "write", "copy-fetch", "copy-write"):
        c.add_argument("--" + n, required=True)
    c.add_argument("--mfma")
    c.add_argument("--extra", nargs="*", help="further counter runs whose means are listed")
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("--algorithmic-bytes", type=float, required=True)
    c.add_argument("--sources", nargs="+", required=True)
    c.add_argument("--last", type=int, default=0)
    c.add_argument("--also", nargs="*", help="kernels launched with the main one whose bytes count with it")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_report(a.dir, a.last, a.match))
    else:
        print(counters_report(a.kernel, a.fetch, a.write, a.copy_fetch, a.copy_write, a.algorithmic_bytes, a.sources,
                              a.mfma, a.last, a.extra, a.xcds, a.simds, a.also))


if __name__ == "__main__":
    sys.exit(main())
