"""Summaries of rocprofv3 runs of bench.py for profiles/ (kernel trace, HBM bytes, MFMA busy).

    python -m mixture_experts_ffn_int32_amd.profsum WORKLOAD RUNDIR

RUNDIR holds the rocprofv3 output directories of these commands, each run from
the repository root (``export TMPDIR=/tmp``; WL is the workload name):

    prof_WL        rocprofv3 --kernel-trace --stats --output-format csv -d RUNDIR/prof_WL -o WL
                       -- python3 bench.py --workload WL --steps 3 --no-cpu-baseline --flush-mb 0
    pmc_WL_FETCH   rocprofv3 --pmc FETCH_SIZE --output-format csv -d RUNDIR/pmc_WL_FETCH -o pmc
                       -- python3 bench.py --workload WL --steps 2 --warmup 1 --no-cpu-baseline --flush-mb 0
    pmc_WL_WRITE   the same with WRITE_SIZE
    pmc_WL_MFMA    the same with SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY
                       SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE
    pmc_copy_FETCH, pmc_copy_WRITE
                   FETCH_SIZE and WRITE_SIZE over ``python3 bench.py --copy-calibration 1024``
                   (a plain 1 GiB device copy, five times): the scale of the byte counters

It writes profiles/step_kernels_WL_T.._H.._I.._E.._K...md (one row per kernel:
calls, average duration, algorithmic work and rate against the MI355X peak,
copy-calibrated HBM bytes per dispatch, MFMA-busy share and the clock the
kernel ran at) and records the bytes per stage in profiles/traffic.json, keyed
by a hash of the library sources, which bench.py reports as ``traffic`` while
the sources are unchanged.  Missing runs leave their columns empty.
"""

import csv
import glob
import hashlib
import json
import os
import re
import sys

from .roofline import stage_work

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SIMDS = 1024            # 256 CUs x 4 SIMDs
XCDS = 8                # GRBM_GUI_ACTIVE comes summed over the XCDs (one count each)
MFMA_CTRS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY",
             "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")


def source_sha():
    """sha256[:16] of the library sources (csrc/), the key of traffic.json."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _tiles(name):
    out = []
    for m in re.findall(r"Cfg<(\d+), (\d+)", name):
        t = "%sx%s" % m
        if t not in out:
            out.append(t)
    return "[" + "+".join(out) + "]" if out else ""


def stage_of(name):
    """(label, stage) of a kernel name: the label adds the tile shapes of a product; the
    stage is the library's name for the launch (what bench.py's stage events time)."""
    suf = _tiles(name)
    if "Gmm1Routed" in name:
        return "route+gmm1_swiglu[64x64]", "route+gmm1_swiglu"
    if "route_one" in name:
        return "route_one", "route"
    for r in ("route_hist", "route_scan", "route_scatter"):
        if r in name:
            return r, "route"
    if "combine_kernel<true" in name:
        return "combine", "combine"
    if "combine_kernel<false" in name:
        return "combine_dx", "combine_dx"
    if "expert_order" in name:
        return "expert_order", "expert_order"
    if "fused_forward" in name:
        return "fused_forward", "fused_forward"
    if "gemm_fp8_kernel" in name:
        if "ActGradF8<" in name:
            return "act_grad_fp8" + suf, "act_grad_fp8"
        if "InputGradF8<" in name:
            return "input_grad_fp8" + suf, "input_grad_fp8"
        m = re.search(r"F8Cfg<[^>]*>, (?:true|false), (\d)>", name)
        st = {"1": "gmm1_mx_swiglu", "2": "gmm1_group_swiglu"}.get(m.group(1) if m else "0", "gmm1_fp8_swiglu")
        return st + suf, st
    if "quant" in name:
        base = name.split("(")[0].split("::")[-1].split("<")[0]
        return base, base
    if "ActGrad<" in name and "Dw<" in name:
        return "act_grad+dw2" + suf, "act_grad+dw2"
    if "InputGrad<" in name and "Dw<" in name:
        return "input_grad+dw1" + suf, "input_grad+dw1"
    for key, st in (("Gmm1<", "gmm1_swiglu"), ("Gmm2<", "gmm2"), ("ActGrad<", "act_grad"), ("InputGrad<", "input_grad")):
        if key in name:
            return st + suf, st
    m = re.search(r"Dw<hmm::\(anonymous namespace\)::Cfg<[^>]*>, (true|false), (true|false)>", name)
    if m:
        st = "dw1" if m.group(1) == "true" else "dw2"
        return st + suf, st
    short = name.split("(")[0][-40:]
    return short, short


def _one(pattern):
    f = sorted(glob.glob(pattern, recursive=True))
    return f[0] if f else None


def kernel_stats(d):
    f = _one(os.path.join(d, "**", "*kernel_stats.csv"))
    return list(csv.DictReader(open(f))) if f else []


def overlapping(d):
    """Names of kernels whose dispatches overlap another kernel's in the trace (two streams)."""
    f = _one(os.path.join(d, "**", "*kernel_trace.csv"))
    if not f:
        return set()
    iv = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in csv.DictReader(open(f)))
    # consecutive launches on one stream may overlap by the few microseconds of a
    # kernel's end; count an overlap above 10 us and a tenth of the shorter kernel
    out, beg, end, last = set(), -1, -1, None
    for a, b, n in iv:
        ov = min(end, b) - a
        if ov > max(10000, 0.1 * min(b - a, end - beg)):
            out.update((n, last))
        if b > end:
            beg, end, last = a, b, n
    return out


def counters(d):
    """{kernel name: {counter: mean per dispatch}} and {kernel name: mean duration ns}."""
    f = _one(os.path.join(d, "**", "*counter_collection.csv"))
    if not f:
        return {}, {}
    acc, dur = {}, {}
    for r in csv.DictReader(open(f)):
        k = r["Kernel_Name"]
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        d_ns = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        dur.setdefault(k, {})[r["Dispatch_Id"]] = d_ns
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}
    return mean, {k: sum(v.values()) / len(v) for k, v in dur.items()}


def copy_scale(rundir, counter, kib_moved):
    """Bytes per counter KiB from the copy calibration: the copy kernel moves kib_moved KiB."""
    vals, _ = counters(os.path.join(rundir, "pmc_copy_" + counter.split("_")[0]))
    per = [c[counter] for c in vals.values() if counter in c]
    if not per:
        return None
    return kib_moved / max(per) * 1024.0


def summarise(wl, rundir):
    from .synth import WORKLOADS
    spec = WORKLOADS[wl]
    T, H, I, E, K = (spec[k] for k in "THIEK")
    stem = "%s_T%d_H%d_I%d_E%d_K%d" % (wl, T, H, I, E, K)
    sha = source_sha()
    fs = copy_scale(rundir, "FETCH_SIZE", 1 << 20)
    ws = copy_scale(rundir, "WRITE_SIZE", 1 << 20)
    fetch, _ = counters(os.path.join(rundir, "pmc_%s_FETCH" % wl))
    write, _ = counters(os.path.join(rundir, "pmc_%s_WRITE" % wl))
    mfma, mdur = counters(os.path.join(rundir, "pmc_%s_MFMA" % wl))
    bench = "python3 bench.py --workload %s" % wl
    cmd_trace = ("rocprofv3 --kernel-trace --stats --output-format csv -d %s/prof_%s -o %s -- %s --steps 3 "
                 "--no-cpu-baseline --flush-mb 0" % (rundir, wl, wl, bench))
    cmd_pmc = ("rocprofv3 --pmc <COUNTERS> --output-format csv -d %s/pmc_%s_<RUN> -o pmc -- %s --steps 2 --warmup 1 "
               "--no-cpu-baseline --flush-mb 0" % (rundir, wl, bench))
    out = ["# Kernels of one fwd+bwd step, %s workload: T=%d H=%d I=%d E=%d K=%d" % (wl, T, H, I, E, K), "",
           "Library source sha256[:16] of csrc/: `%s`." % sha, "",
           "Commands (repository root, `export TMPDIR=/tmp`), then "
           "`python -m mixture_experts_ffn_int32_amd.profsum %s %s`:" % (wl, rundir), "",
           "    " + cmd_trace,
           "    " + cmd_pmc.replace("<COUNTERS>", "FETCH_SIZE").replace("<RUN>", "FETCH"),
           "    " + cmd_pmc.replace("<COUNTERS>", "WRITE_SIZE").replace("<RUN>", "WRITE"),
           "    " + cmd_pmc.replace("<COUNTERS>", " ".join(MFMA_CTRS)).replace("<RUN>", "MFMA"),
           "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s/pmc_copy_FETCH -o pmc -- python3 bench.py "
           "--copy-calibration 1024  (and WRITE_SIZE into pmc_copy_WRITE)" % rundir, "",
           "Byte counters are scaled by what they read for a plain 1 GiB device copy: FETCH_SIZE x%s, WRITE_SIZE x%s "
           "bytes per KiB." % ("%.1f" % fs if fs else "n/a", "%.1f" % ws if ws else "n/a"),
           "Rate: algorithmic work (no tile padding; operands read once) / average duration, against the MI355X "
           "peak (bf16 2.5 PFLOP/s, fp8 5.0, HBM 8 TB/s).  GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's "
           "cycles are an eighth of it.  MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (XCD cycles x 1024 SIMDs).  "
           "Clock: XCD cycles / duration of the dispatch in the counter run (kernels of 100 us or more).  "
           "Dep. wait: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave time waiting on a dependency).  "
           "Executed / work: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / algorithmic flops (tile padding).", "",
           "| kernel | calls | avg us | % of GPU time | work | rate | of peak | HBM MB / dispatch | MFMA busy | "
           "clock GHz | dep. wait | executed / work |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    per = {}
    rows = kernel_stats(os.path.join(rundir, "prof_" + wl))
    # kernels per stage (a stage of several launches, such as the FP8 up-projection's
    # big-tile and small-tile launches, gets its rate in the per-stage table only)
    nk = {}
    for r in rows:
        nk[stage_of(r["Name"])[1]] = nk.get(stage_of(r["Name"])[1], 0) + 1
    calls = sorted(int(r["Calls"]) for r in rows)
    steps = max(set(calls), key=calls.count) if calls else 1  # the product kernels run once per step
    stage_ns = {}
    for r in rows:
        name = r["Name"]
        label, st = stage_of(name)
        stage_ns[st] = stage_ns.get(st, 0.0) + float(r["TotalDurationNs"])
        avg_us = float(r["AverageNs"]) / 1e3
        bound, work, unit, peak = stage_work(st, T, H, I, E, K)
        rate = frac = None
        if bound and not label.startswith("route_") and nk[st] == 1:
            rate = work / (avg_us * 1e-6) / (1e12 if bound == "mfma" else 1e9)
            frac = rate / peak
        f, w = fetch.get(name, {}).get("FETCH_SIZE"), write.get(name, {}).get("WRITE_SIZE")
        hbm = None
        if f is not None and w is not None and fs and ws:
            hbm = f * fs + w * ws
            e = per.setdefault(st, {"fetch_kib": 0.0, "write_kib": 0.0, "bytes": 0.0})
            e["fetch_kib"] += f
            e["write_kib"] += w
            e["bytes"] += hbm
        mc = mfma.get(name, {})
        busy = clock = wait = execd = None
        if mc.get("GRBM_GUI_ACTIVE"):
            xcd_cycles = mc["GRBM_GUI_ACTIVE"] / XCDS
            busy = mc.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (xcd_cycles * SIMDS)
            if mdur.get(name, 0) >= 100e3:
                clock = xcd_cycles / mdur[name]
        if mc.get("SQ_WAVE_CYCLES"):
            wait = mc.get("SQ_WAIT_INST_ANY", 0.0) / mc["SQ_WAVE_CYCLES"]
        if bound == "mfma" and mc.get("SQ_INSTS_VALU_MFMA_MOPS_BF16") and st in ("gmm1_swiglu", "gmm2", "act_grad",
                                                                                  "input_grad", "dw1", "dw2"):
            execd = mc["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / work
        out.append("| %s | %s | %.2f | %.2f | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            label, r["Calls"], avg_us, float(r["Percentage"]),
            ("%.4g %s" % (work / (1e12 if bound == "mfma" else 1e6), "TFLOP" if bound == "mfma" else "MB"))
            if bound else "",
            ("%.1f %s" % (rate, unit)) if rate else "", ("%.3f" % frac) if frac else "",
            ("%.1f" % (hbm / 1e6)) if hbm is not None else "", ("%.3f" % busy) if busy is not None else "",
            ("%.2f" % clock) if clock else "", ("%.2f" % wait) if wait is not None else "",
            ("%.3f" % execd) if execd else ""))
    ov = sorted({stage_of(n)[0] for n in overlapping(os.path.join(rundir, "prof_" + wl))})
    if ov:
        out += ["", "These kernels ran at the same time as another kernel in the traced steps (the backward's weight "
                "gradients on a second stream beside the dX chain), so their durations include the sharing: "
                + ", ".join(ov) + "."]
    multi = sorted(st for st, n in nk.items() if n > 1 and stage_work(st, T, H, I, E, K)[0])
    if multi:
        out += ["", "Stages of several launches (time per step = the launches' total duration / %d steps):" % steps,
                "", "| stage | launches per step | us per step | work | rate | of peak |", "|---|---|---|---|---|---|"]
        for st in multi:
            bound, work, unit, peak = stage_work(st, T, H, I, E, K)
            us = stage_ns[st] / steps / 1e3
            rate = work / (us * 1e-6) / (1e12 if bound == "mfma" else 1e9)
            out.append("| %s | %d | %.2f | %.4g %s | %.1f %s | %.3f |" % (
                st, nk[st], us, work / (1e12 if bound == "mfma" else 1e6), "TFLOP" if bound == "mfma" else "MB",
                rate, unit, rate / peak))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", "step_kernels_%s.md" % stem)
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    tj = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(tj))
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_sha") != sha:
        rec = {"source_sha": sha, "per_workload": {}}
    if per:
        rec["per_workload"][wl] = per
        with open(tj, "w") as fh:
            json.dump(rec, fh, indent=1)
    return path


if __name__ == "__main__":
    if len(sys.argv) != 3:
        print(__doc__, file=sys.stderr)
        sys.exit(2)
    print(summarise(sys.argv[1], sys.argv[2]))
