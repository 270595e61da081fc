"""Benchmark of the fused MoE-FFN forward + backward on one MI355X.

One step = hmm_forward + hmm_backward (routing, up-projection + SwiGLU,
down-projection, weighted combine; act_grad + SwiGLUGrad, input_grad,
combine(dX), d_topk_weights, W2Grad, W1Grad) over one batch of seeded
synthetic input already resident in HBM, through the C ABI of libhmm.

Prints ONE JSON line on stdout; details go to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload hotspot|skewed|sample|tiny|fp8|mx|group]

The default workload is hotspot (T=8192, H=7168, I=2048, E=32, K=8: the
largest bf16 workload of the list, one hot expert in every token).

Timing: W untimed warm-up steps (the first one's time is reported as
first_step_ms), then K steps between two synchronisations, timed with HIP
events on the stream the kernels run on -> ms_per_step and tokens/s.  A second
pass of K steps, with an event after each call, gives the forward and backward
times (fwd_ms, bwd_ms).  A third pass of K steps records HIP events around
every kernel launch (the library's stage timing) and gives each kernel's
average duration for the roofline figures (this pass runs the backward's
launches in series, so each kernel has the chip to itself; the timed steps use
the default, with the weight gradients on a second stream).  A fourth pass writes a 1 GiB
scratch buffer before every step (more than the 256 MB last-level cache holds)
and times the HBM-bound kernels again (flushed figures, beside the warm ones).
The CPU oracle (its pure mode, float32 sums: the plain per-token loop) is then
timed on a bounded sample of the same workload on the host's cores.
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mixture_experts_ffn_int32_amd.roofline import PEAK_BF16_TFLOPS, PEAK_FP8_TFLOPS, PEAK_HBM_GBS, stage_work  # noqa: E402,F401


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha():
    """sha256[:16] of the library sources (the key of the recorded traffic counters)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_ffn_int32_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 --pmc figures, or None if absent or stale."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != source_sha():
        return None
    ent = rec.get("per_workload", {}).get(workload, {}).get(kernel)
    return None if ent is None else int(round(ent["bytes"]))


class Runner:
    """Preallocated buffers and raw C-ABI calls for one workload."""

    def __init__(self, spec, seed, device, validate_ids=True, out_dtype="bf16", serial_backward=False):
        import torch
        from mixture_experts_ffn_int32_amd import _lib, synth
        self.torch = torch
        self.lib = _lib.load()
        self._lib = _lib
        self.spec = spec
        T, H, I, E, K = (spec[k] for k in "THIEK")
        self.dims = (T, H, I, E, K)
        t0 = time.time()
        inp = synth.make_inputs(spec, seed=seed)
        log("[bench] inputs generated in %.1fs" % (time.time() - t0))
        self.inp = inp

        def bf(bits):
            import numpy as np
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

        self.x = bf(inp["x"])
        self.dy = bf(inp["dY"])
        self.W1 = bf(inp["up_proj_weight"])
        self.W2 = bf(inp["down_proj_weight"])
        self.ids = torch.from_numpy(inp["topk_ids"]).to(device)
        self.w = torch.from_numpy(inp["topk_weights"]).to(device)
        flags = (_lib.HMM_FLAG_VALIDATE_IDS if validate_ids else 0) | (
            _lib.HMM_FLAG_SERIAL_BACKWARD if serial_backward else 0) | (
            _lib.HMM_FLAG_FP8_BACKWARD if spec.get("fp8_backward") else 0)
        gmm1 = {"bf16": _lib.HMM_BF16, "fp8": _lib.HMM_FP8_E4M3, "mx": _lib.HMM_MXFP8_E4M3,
                "group": _lib.HMM_FP8_E4M3_GROUP}[spec.get("gmm1", "bf16")]
        f32 = out_dtype == "f32"
        Is = spec.get("shared_I", 0)
        self.prob = _lib.Problem(T, H, I, E, K, _lib.HMM_F32 if f32 else _lib.HMM_BF16, gmm1, flags, Is)
        fws, sv, bws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        _lib.check(self.lib.hmm_forward_sizes(ctypes.byref(self.prob), ctypes.byref(fws), ctypes.byref(sv)))
        _lib.check(self.lib.hmm_backward_sizes(ctypes.byref(self.prob), ctypes.byref(bws)))
        u8 = torch.uint8
        odt = torch.float32 if f32 else torch.bfloat16
        if f32:
            self.dy = self.dy.float()
        self.y = torch.empty((T, H), dtype=odt, device=device)
        self.saved = torch.empty(sv.value, dtype=u8, device=device)
        self.fwork = torch.empty(fws.value, dtype=u8, device=device)
        self.bwork = torch.empty(bws.value, dtype=u8, device=device)
        self.dx = torch.empty((T, H), dtype=odt, device=device)
        self.dW1 = torch.empty((E, H, 2 * I), dtype=odt, device=device)
        self.dW2 = torch.empty((E, I, H), dtype=odt, device=device)
        self.dw = torch.empty((T, K), dtype=torch.float32, device=device)
        self.sizes = (fws.value, sv.value, bws.value)
        self.stream = torch.cuda.current_stream(device)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        st = ctypes.c_void_p(self.stream.cuda_stream)
        self.shared = bool(Is)
        if self.shared:  # the shared-expert entry points, with its weights and their gradients
            self.Ws1 = bf(inp["shared_up_proj_weight"])
            self.Ws2 = bf(inp["shared_down_proj_weight"])
            self.dWs1 = torch.empty((H, 2 * Is), dtype=odt, device=device)
            self.dWs2 = torch.empty((Is, H), dtype=odt, device=device)
            self.fargs = (ctypes.byref(self.prob), P(self.x), P(self.ids), P(self.w), P(self.W1), P(self.W2),
                          P(self.Ws1), P(self.Ws2), P(self.y), P(self.saved), sv.value, P(self.fwork), fws.value, st)
            self.bargs = (ctypes.byref(self.prob), P(self.dy), P(self.x), P(self.ids), P(self.w), P(self.W1),
                          P(self.W2), P(self.Ws1), P(self.Ws2), P(self.saved), sv.value, P(self.dx), P(self.dW1),
                          P(self.dW2), P(self.dWs1), P(self.dWs2), P(self.dw), P(self.bwork), bws.value, st)
            self.fwd, self.bwd = self.lib.hmm_forward_shared, self.lib.hmm_backward_shared
        else:
            self.fargs = (ctypes.byref(self.prob), P(self.x), P(self.ids), P(self.w), P(self.W1), P(self.W2),
                          P(self.y), P(self.saved), sv.value, P(self.fwork), fws.value, st)
            self.bargs = (ctypes.byref(self.prob), P(self.dy), P(self.x), P(self.ids), P(self.w), P(self.W1),
                          P(self.W2), P(self.saved), sv.value, P(self.dx), P(self.dW1), P(self.dW2), P(self.dw),
                          P(self.bwork), bws.value, st)
            self.fwd, self.bwd = self.lib.hmm_forward, self.lib.hmm_backward

    def step(self):
        self._lib.check(self.fwd(*self.fargs))
        self._lib.check(self.bwd(*self.bargs))

    def timed(self, n):
        torch = self.torch
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(n):
            self.step()
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def timed_flushed(self, n, flush_mb):
        """n steps, each preceded by a write of flush_mb MiB of scratch on the same stream
        (the stage events of the library time the kernels; the write is not a stage)."""
        torch = self.torch
        if getattr(self, "_scratch", None) is None or self._scratch.numel() != flush_mb << 18:
            self._scratch = torch.empty(flush_mb << 18, dtype=torch.float32, device=self.x.device)
        torch.cuda.synchronize()
        for i in range(n):
            self._scratch.fill_(float(i))
            self.step()
        torch.cuda.synchronize()

    def timed_split(self, n):
        """Average forward and backward times (ms) over n steps, an event after each call."""
        torch = self.torch
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n + 1)]
        ev[0].record(self.stream)
        for i in range(n):
            self._lib.check(self.fwd(*self.fargs))
            ev[2 * i + 1].record(self.stream)
            self._lib.check(self.bwd(*self.bargs))
            ev[2 * i + 2].record(self.stream)
        torch.cuda.synchronize()
        f = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)) / n
        b = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(n)) / n
        return f, b


def cpu_baseline(spec, seed, budget_s=12.0):
    """Time the oracle's pure mode with float32 sums (forward + full backward: the plain
    per-token loop over K experts, and each expert's weight gradients) on a bounded
    prefix of the workload's tokens."""
    import numpy as np
    from mixture_experts_ffn_int32_amd import synth
    from oracle.moe_ffn import MoEFFN
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    inp = synth.make_inputs(spec, seed=seed)
    T = spec["T"]

    def run(tp):
        d = dict(x=synth.bits_to_f32(inp["x"][:tp]), topk_ids=inp["topk_ids"][:tp],
                 topk_weights=inp["topk_weights"][:tp], up_proj_weight=synth.bits_to_f32(inp["up_proj_weight"]),
                 down_proj_weight=synth.bits_to_f32(inp["down_proj_weight"]), dY=synth.bits_to_f32(inp["dY"][:tp]))
        for k in ("shared_up_proj_weight", "shared_down_proj_weight"):
            if k in inp:
                d[k] = synth.bits_to_f32(inp[k])
        t0 = time.perf_counter()
        m = MoEFFN(**d, mode="pure", gmm1=spec.get("gmm1", "bf16"), acc="f32",
                   bwd="fp8" if spec.get("fp8_backward") else "bf16")
        m.forward()
        m.backward()
        if m.shared is not None:
            m.shared_backward_dev()
        return time.perf_counter() - t0

    tp = min(T, 8)
    el = run(tp)
    while el < budget_s / 4 and tp < T:
        tp = min(T, int(tp * max(2.0, min(8.0, budget_s / 2 / max(el, 1e-3)))))
        el = run(tp)
    # a workload the oracle finishes quickly: repeat whole passes up to at least 10 s of work
    passes = 1
    while tp == T and el < 10.0:
        el += run(tp)
        passes += 1
    return {"value": passes * tp / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": "first %d of %d tokens of the same workload x %d pass(es), oracle pure mode with float32 "
                      "sums, forward + full backward (numpy, %d BLAS threads), %.1f s" % (tp, T, passes, cores, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="hotspot")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-validate", action="store_true", help="skip the id check's device-to-host read-back")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"],
                    help="f32: the float32-output accuracy mode (hi/lo operand pairs)")
    ap.add_argument("--shared-I", type=int, default=0, metavar="IS",
                    help="add a shared expert of intermediate size IS (every token, weight 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial-backward", action="store_true",
                    help="keep every backward launch on one stream (HMM_FLAG_SERIAL_BACKWARD)")
    ap.add_argument("--cpu-budget", type=float, default=40.0,
                    help="the oracle sample grows until it takes about a quarter of this (seconds)")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="scratch written before each step of the flushed pass (0: no flushed pass)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times (scale for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_ffn_int32_amd import _lib, synth
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied %d MiB 5 times (reads %d KiB, writes %d KiB per copy)" % (n >> 20, n >> 10, n >> 10))
        return
    spec = dict(synth.WORKLOADS[args.workload])
    if args.shared_I:
        spec["shared_I"] = args.shared_I
    Is = spec.get("shared_I", 0)
    gmm1_kind = spec.get("gmm1", "bf16")
    T, H, I, E, K = (spec[k] for k in "THIEK")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    r = Runner(spec, args.seed, dev, validate_ids=not args.no_validate, out_dtype=args.out_dtype,
               serial_backward=args.serial_backward)
    log("[bench] workload %s T=%d H=%d I=%d E=%d K=%d shared_I=%d; workspace fwd %.1f MB, saved %.1f MB, bwd %.1f MB"
        % (args.workload, T, H, I, E, K, Is, r.sizes[0] / 1e6, r.sizes[1] / 1e6, r.sizes[2] / 1e6))

    first_ms = r.timed(1)
    for _ in range(max(0, args.warmup - 1)):
        r.step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    total_ms = r.timed(args.steps)
    wall = time.perf_counter() - wall0
    ms = total_ms / args.steps
    log("[bench] %d steps: %.4f ms/step (host wall %.4f ms/step), first step %.3f ms"
        % (args.steps, ms, wall * 1e3 / args.steps, first_ms))

    # forward and backward separately (an event between them in every step)
    fwd_ms, bwd_ms = r.timed_split(args.steps)
    log("[bench] forward %.4f ms, backward %.4f ms per step" % (fwd_ms, bwd_ms))

    # third pass: per-kernel device time from the library's stage events, with the
    # backward's launches in series (each kernel alone on the chip, so the stage
    # times add up and give each kernel's own rate)
    _lib.profile_read()
    _lib.profile_enable(True)
    flags0 = r.prob.flags
    r.prob.flags = flags0 | _lib.HMM_FLAG_SERIAL_BACKWARD
    prof_ms = r.timed(args.steps)
    r.prob.flags = flags0
    _lib.profile_enable(False)
    stages, dropped = _lib.profile_read()
    log("[bench] profiled pass %.4f ms/step; %d launches untimed" % (prof_ms / args.steps, dropped))
    S = T * K
    gemm_ms = 0.0
    gemm_ms_at_peak = 0.0          # time the products would take at their dtype's peak
    rows = []
    for name, (n, tot) in sorted(stages.items(), key=lambda kv: -kv[1][1]):
        avg = tot / max(n, 1)
        bound, work, unit, peak = stage_work(name, T, H, I, E, K, args.out_dtype == "f32", Is)
        rate = (work / (avg * 1e-3) / (1e12 if bound == "mfma" else 1e9)) if bound else None
        if bound == "mfma":
            gemm_ms += tot / args.steps
            gemm_ms_at_peak += work / (peak * 1e12) * 1e3 * n / args.steps
        rows.append((name, n, avg, bound, work, rate, unit, (rate / peak) if rate else None, peak))
        log("[bench]   %-16s launches %4d  avg %9.4f ms  %s" % (
            name, n, avg, ("%.1f %s (%.1f%% of peak)" % (rate, unit, 100 * rate / peak)) if rate else ""))
    dom = max((x for x in rows if x[3]), key=lambda x: x[2] * x[1])
    gemm_flops = 18 * S * H * I + 18 * T * H * Is
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else None
    roofline = {
        "kernel": dom[0],
        "bound": dom[3],
        "achieved": round(dom[5], 3),
        "peak": dom[8],
        "unit": dom[6],
        "frac": round(dom[7], 5),
        "algorithmic": dom[4],
        "traffic": recorded_traffic(args.workload, dom[0]),
    }

    # fourth pass: the HBM-bound kernels with the last-level cache flushed before every step
    hbm_rows = [x for x in rows if x[3] == "hbm"]
    flushed = {}
    if args.flush_mb > 0 and hbm_rows:
        _lib.profile_read()
        _lib.profile_enable(True)
        r.timed_flushed(args.steps, args.flush_mb)
        _lib.profile_enable(False)
        flushed, _ = _lib.profile_read()
    hbm = {}
    for name, n, avg, bound, work, rate, unit, frac, peak in hbm_rows:
        ent = {"bytes": work, "warm_ms": round(avg, 5), "warm_GBs": round(rate, 1), "warm_frac": round(frac, 4)}
        if name in flushed:
            fn, ftot = flushed[name]
            favg = ftot / max(fn, 1)
            frate = work / (favg * 1e-3) / 1e9
            ent.update({"flushed_ms": round(favg, 5), "flushed_GBs": round(frate, 1), "flushed_frac": round(frate / peak, 4)})
            log("[bench]   %-16s flushed avg %9.4f ms  %.1f GB/s (%.1f%% of peak)" % (name, favg, frate, 100 * frate / peak))
        hbm[name] = ent

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(spec, args.seed, args.cpu_budget)
        log("[bench] cpu baseline %.1f tokens/s (%s) in %.1fs" % (cpu["value"], cpu["sample"], time.time() - t0))

    out = {
        "metric": "MoE-FFN fwd+bwd tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), 1xMI355X",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "first_step_ms": round(first_ms, 4),
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "bf16+fp8", "mx": "bf16+mxfp8", "group": "bf16+fp8", "fp8bwd": "bf16+fp8"}.get(
            gmm1_kind, "bf16 hi/lo pairs, f32 outputs" if args.out_dtype == "f32" else "bf16"),
        "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "H": H, "I": I, "E": E, "K": K,
                   "routing": spec.get("routing"), "shared_I": Is, "seed": args.seed,
                   "gmm1": gmm1_kind, "fp8_backward": bool(spec.get("fp8_backward")),
                   "validate_ids": not args.no_validate, "serial_backward": args.serial_backward,
                   "out_dtype": args.out_dtype},
        "gemm_tflops": round(gemm_tflops, 3) if gemm_tflops else None,
        "gemm_frac_peak": round(gemm_ms_at_peak / gemm_ms, 5) if gemm_ms > 0 else None,
        "roofline": roofline,
        "stage_ms": {x[0]: round(x[2], 5) for x in rows},
        "hbm_kernels": hbm,
        "flush_mb": args.flush_mb,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
