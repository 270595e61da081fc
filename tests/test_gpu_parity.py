"""Forward and backward on the GPU against the FAITHFUL oracle.

Small problems are compared element by element on every output; they span
several 128x128 tiles, ragged tails, empty and hot experts, K = 1 and
duplicate ids.  The full-size workloads are compared on sampled tokens and
sampled weight-gradient columns the oracle evaluates one by one, in the same
launch configuration bench.py times.
"""

import numpy as np
import pytest

from _util import announce, assert_close, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN
from oracle.routing import route as oracle_route

pytestmark = pytest.mark.gpu


def run_gpu(g, tiles="auto", gmm1="bf16", fp8_backward=False):
    import torch
    from mixture_experts_ffn_int32_amd import backward_from_saved, forward_with_saved
    y, saved = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                  g["down_proj_weight"], tiles=tiles, gmm1_dtype=gmm1)
    dx, dW1, dW2, dw = backward_from_saved(g["dY"], g["x"], g["topk_ids"], g["topk_weights"],
                                           g["up_proj_weight"], g["down_proj_weight"], saved, tiles=tiles,
                                           gmm1_dtype=gmm1, fp8_backward=fp8_backward)
    torch.cuda.synchronize()
    return y, saved, dx, dW1, dW2, dw


SMALL = [
    # name, spec overrides
    ("tiny", dict()),
    ("ragged", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform")),
    ("hot", dict(T=257, H=192, I=128, E=5, K=2, routing="hot")),
    ("hotdup", dict(T=130, H=128, I=64, E=4, K=3, routing="hot_dup")),
    ("k1", dict(T=200, H=128, I=128, E=3, K=1, routing="uniform")),
    ("zipf", dict(T=411, H=256, I=128, E=16, K=4, routing="zipf", zipf_s=1.2, n_empty=5)),
    # expert sizes on the large tiling's boundaries: remainders of 1-64, 65-128
    # (small tiles, one or two table entries) and 129-255 rows (a partial big tile)
    # the most experts the routing takes, many of them empty or tied in size (the weight
    # gradients' longest-first expert order ranks all 1024; on 64x64 tiles the tables'
    # capacity exceeds the size above which the launches spread the real tiles over
    # the XCDs)
    ("e1024", dict(T=512, H=128, I=64, E=1024, K=8, routing="zipf", zipf_s=0.6, n_empty=200)),
    ("bounds", dict(T=2278, H=128, I=64, E=14, K=1, routing="counts",
                    counts=[0, 1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 320, 385, 228])),
]


@pytest.mark.parametrize("tiles", ["large", "narrow"])
@pytest.mark.parametrize("name,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_parity(name, over, tiles):
    spec = synth.spec_with("tiny", **over)
    inp = synth.make_inputs(spec, seed=11)
    announce("full parity %s %s tiles=%s" % (name, {k: spec[k] for k in "THIEK"}, tiles))
    g = gpu_inputs(inp, "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g, tiles)
    o = MoEFFN(**oracle_inputs(inp), mode="faithful")
    ry, ryd = o.forward_dev()
    assert_close(to_f64(y), ry, name + " y", ryd)
    (rdx, rdw, rdW1, rdW2), (ddx, ddw, ddW1, ddW2) = o.backward_dev()
    assert_close(to_f64(dx), rdx, name + " dx", ddx)
    assert_close(to_f64(dw), rdw, name + " d_topk_weights", ddw)
    assert_close(to_f64(dW1), rdW1, name + " d_up_proj_weight", ddW1)
    assert_close(to_f64(dW2), rdW2, name + " d_down_proj_weight", ddW2)
    # experts without tokens get exact zeros
    counts = np.bincount(inp["topk_ids"].reshape(-1), minlength=spec["E"])
    for e in np.flatnonzero(counts == 0):
        assert not to_f64(dW1[e]).any() and not to_f64(dW2[e]).any()


@pytest.mark.parametrize("tiles", ["large", "narrow"])
def test_saved_intermediates_match_oracle(tiles):
    from mixture_experts_ffn_int32_amd import saved_views
    spec = synth.spec_with("tiny", T=300, H=256, I=192, E=6, K=3)
    inp = synth.make_inputs(spec, seed=3)
    announce("saved intermediates tiles=%s" % tiles)
    g = gpu_inputs(inp, "cuda")
    y, saved, *_ = run_gpu(g, tiles)
    v = saved_views(saved, *(spec[k] for k in "THIEK"), tiles=tiles)
    ref_route = oracle_route(inp["topk_ids"], spec["E"])
    for k in ("counts", "offsets", "sorted_slot", "row_of_slot"):
        assert np.array_equal(v[k].cpu().numpy(), ref_route[k]), k
    o = MoEFFN(**oracle_inputs(inp), mode="faithful")
    (h, a, _), (hd, ad, _) = o.slot_intermediates_dev(ref_route["sorted_slot"])
    assert_close(to_f64(v["h"]), h, "h", hd)
    assert_close(to_f64(v["a"]), a, "a", ad)
    w = inp["topk_weights"].reshape(-1)[ref_route["sorted_slot"]].astype(np.float64)
    assert_close(to_f64(v["aw"]), w[:, None] * to_f64(v["a"]), "aw")


@pytest.mark.parametrize("Is", [0, 128])
def test_backward_side_stream_equals_serial(Is):
    """Large tiling: the weight gradients on the library's second stream give results
    bit-identical to the same launches in series on one stream (with and without a
    shared expert)."""
    import torch
    from mixture_experts_ffn_int32_amd import backward_from_saved, forward_with_saved
    spec = synth.spec_with("tiny", T=300, H=256, I=192, E=6, K=3, routing="uniform", shared_I=Is)
    g = gpu_inputs(synth.make_inputs(spec, seed=9), "cuda")
    sh = dict(shared_up_proj_weight=g.get("shared_up_proj_weight"), shared_down_proj_weight=g.get("shared_down_proj_weight"))
    announce("backward on two streams against one, shared_I=%d" % Is)
    y, saved = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                  g["down_proj_weight"], tiles="large", **sh)
    args = (g["dY"], g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"], saved)
    a = backward_from_saved(*args, tiles="large", serial=False, **sh)
    b = backward_from_saved(*args, tiles="large", serial=True, **sh)
    torch.cuda.synchronize()
    assert len(a) == len(b) == (6 if Is else 4)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_deterministic_and_t0():
    import torch
    spec = synth.spec_with("tiny", T=300, H=256, I=192, E=6, K=3)
    g = gpu_inputs(synth.make_inputs(spec, seed=4), "cuda")
    announce("determinism")
    from mixture_experts_ffn_int32_amd import saved_views
    r1 = run_gpu(g)
    r2 = run_gpu(g)
    for i in (0, 2, 3, 4, 5):                    # y, dx, dW1, dW2, d_topk_weights
        assert torch.equal(r1[i], r2[i])
    v1 = saved_views(r1[1], *(spec[k] for k in "THIEK"))
    v2 = saved_views(r2[1], *(spec[k] for k in "THIEK"))
    for k in v1:                                 # every array the forward records
        assert torch.equal(v1[k], v2[k]), k
    announce("T=0")
    spec0 = synth.spec_with(spec, T=0)
    g0 = gpu_inputs(synth.make_inputs(spec0, seed=4), "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g0)
    assert y.shape == (0, 256) and dx.shape == (0, 256) and dw.shape == (0, 3)
    assert not dW1.float().abs().sum().item() and not dW2.float().abs().sum().item()


def test_autograd_matches_raw_and_accumulates():
    import torch
    from mixture_experts_ffn_int32_amd import hyper_mega_moe
    spec = synth.spec_with("tiny", T=96, H=128, I=64, E=4, K=2)
    inp = synth.make_inputs(spec, seed=5)
    g = gpu_inputs(inp, "cuda")
    announce("autograd")
    x = g["x"].clone().requires_grad_(True)
    w = g["topk_weights"].clone().requires_grad_(True)
    W1 = g["up_proj_weight"].clone().requires_grad_(True)
    W2 = g["down_proj_weight"].clone().requires_grad_(True)
    ids64 = g["topk_ids"].long()                 # int64 ids are converted
    y = hyper_mega_moe(x, ids64, w, W1, W2)
    y.backward(g["dY"])
    y_raw, saved, dx, dW1, dW2, dw = run_gpu(g)
    assert torch.equal(y, y_raw) and torch.equal(x.grad, dx) and torch.equal(W1.grad, dW1)
    assert torch.equal(W2.grad, dW2) and torch.equal(w.grad, dw)
    # two forwards, then both backwards: gradients accumulate (sum of two single backwards)
    for p in (x, w, W1, W2):
        p.grad = None
    y1 = hyper_mega_moe(x, ids64, w, W1, W2)
    y2 = hyper_mega_moe(x, ids64, w, W1, W2)
    (y1.float() * g["dY"].float() + y2.float() * g["dY"].float()).sum().backward()
    assert torch.allclose(W2.grad.float(), 2 * dW2.float(), rtol=1e-2, atol=1e-2)
    assert torch.allclose(w.grad, 2 * dw, rtol=1e-5, atol=1e-5)


def test_bad_inputs_rejected_before_launch():
    import torch
    from mixture_experts_ffn_int32_amd import hyper_mega_moe
    spec = synth.spec_with("tiny", T=64, H=128, I=64, E=4, K=2)
    g = gpu_inputs(synth.make_inputs(spec, seed=6), "cuda")
    announce("bad inputs")
    with pytest.raises(ValueError):
        hyper_mega_moe(g["x"], g["topk_ids"], g["topk_weights"][:, :1], g["up_proj_weight"], g["down_proj_weight"])
    with pytest.raises(TypeError):
        hyper_mega_moe(g["x"].float(), g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    with pytest.raises(ValueError):
        hyper_mega_moe(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"][:, :, :100],
                       g["down_proj_weight"])
    bad = g["topk_ids"].clone()
    bad[5, 0] = 4
    with pytest.raises(ValueError):
        hyper_mega_moe(g["x"], bad, g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    # H not a multiple of 64: rejected by the library's host checks
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        hyper_mega_moe(x, g["topk_ids"][:4], g["topk_weights"][:4], torch.zeros((4, 96, 128), dtype=torch.bfloat16,
                       device="cuda"), torch.zeros((4, 64, 96), dtype=torch.bfloat16, device="cuda"))
    # a valid call right after the failures matches a fresh one
    y1 = hyper_mega_moe(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    y2 = hyper_mega_moe(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    assert torch.equal(y1, y2)


ROUTED = [
    # problems whose up-projection launch routes the ids itself (narrow tiles, S <= 4096,
    # E <= 256, at most 256 tiles of 64x64 in the launch), at its bounds: the most slots,
    # the most experts (and exactly 256 tiles), one expert, one slot, a slot count that
    # splits unevenly over the four waves
    ("max_slots", dict(T=512, H=128, I=64, E=8, K=8, routing="zipf", zipf_s=0.8, n_empty=0)),
    ("max_experts", dict(T=16, H=128, I=64, E=256, K=8, routing="uniform")),
    ("one_expert", dict(T=4096, H=128, I=64, E=1, K=1, routing="uniform")),
    ("one_slot", dict(T=1, H=128, I=64, E=3, K=1, routing="uniform")),
    ("uneven", dict(T=585, H=192, I=64, E=20, K=7, routing="zipf", zipf_s=1.1, n_empty=5)),
]


@pytest.mark.parametrize("name,over", ROUTED, ids=[r[0] for r in ROUTED])
def test_routed_up_projection_at_its_bounds(name, over):
    """The routing arrays of the launch that routes inside the up-projection match the
    oracle's bit for bit; h, a and y match it element by element."""
    from mixture_experts_ffn_int32_amd import forward_with_saved, saved_views
    spec = synth.spec_with("tiny", **over)
    inp = synth.make_inputs(spec, seed=23)
    announce("routed up-projection %s %s" % (name, {k: spec[k] for k in "THIEK"}))
    g = gpu_inputs(inp, "cuda")
    y, saved = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                  g["down_proj_weight"], tiles="narrow")
    v = saved_views(saved, *(spec[k] for k in "THIEK"), tiles="narrow")
    ref_route = oracle_route(inp["topk_ids"], spec["E"])
    for k in ("counts", "offsets", "sorted_slot", "row_of_slot"):
        assert np.array_equal(v[k].cpu().numpy(), ref_route[k]), k
    o = MoEFFN(**oracle_inputs(inp), mode="faithful")
    ry, ryd = o.forward_dev()
    assert_close(to_f64(y), ry, name + " y", ryd)
    (h, a, _), (hd, ad, _) = o.slot_intermediates_dev(ref_route["sorted_slot"])
    assert_close(to_f64(v["h"]), h, name + " h", hd)
    assert_close(to_f64(v["a"]), a, name + " a", ad)


def test_routed_up_projection_drops_out_of_range_ids():
    """Without the id check, slots whose id lies outside [0, E) get no row (row_of_slot
    -1) and the others keep the stable order; with it, the call fails."""
    from mixture_experts_ffn_int32_amd import _lib, forward_with_saved, saved_views
    spec = synth.spec_with("tiny", T=200, H=128, I=64, E=5, K=2, routing="uniform")
    inp = synth.make_inputs(spec, seed=29)
    ids = inp["topk_ids"].copy()
    ids[5, 0] = 5
    ids[77, 1] = -3
    inp["topk_ids"] = ids
    announce("routed up-projection with out-of-range ids")
    g = gpu_inputs(inp, "cuda")
    args = (g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    y, saved = forward_with_saved(*args, validate_ids=False, tiles="narrow")
    v = saved_views(saved, *(spec[k] for k in "THIEK"), tiles="narrow")
    flat = ids.reshape(-1)
    good = (flat >= 0) & (flat < spec["E"])
    order = np.flatnonzero(good)[np.argsort(flat[good], kind="stable")]
    assert np.array_equal(v["sorted_slot"].cpu().numpy()[:order.size], order)
    assert v["row_of_slot"].cpu().numpy()[~good].tolist() == [-1, -1]
    assert np.array_equal(v["counts"].cpu().numpy(), np.bincount(flat[good], minlength=spec["E"]))
    with pytest.raises(ValueError) as ei:
        forward_with_saved(*args, tiles="narrow")
    assert ei.value.status == _lib.HMM_ERR_EXPERT_ID_OUT_OF_RANGE


# ----------------------------------------------------------------------------- full-size workloads, sampled

def _sample_full(name, n_tok=6, icols_frac=(0.0, 0.37, 1.0)):
    import torch
    spec = synth.WORKLOADS[name]
    T, H, I, E, K = (spec[k] for k in "THIEK")
    gmm1 = spec.get("gmm1", "bf16")
    fp8bwd = bool(spec.get("fp8_backward"))
    inp = synth.make_inputs(spec, seed=0)
    announce("full-size sampled parity %s" % name)
    g = gpu_inputs(inp, "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g, gmm1=gmm1, fp8_backward=fp8bwd)
    from mixture_experts_ffn_int32_amd import saved_views
    v = saved_views(saved, T, H, I, E, K, gmm1_dtype=gmm1)
    ref_route = oracle_route(inp["topk_ids"], E)
    for k in ("counts", "offsets", "sorted_slot", "row_of_slot"):
        assert np.array_equal(v[k].cpu().numpy(), ref_route[k]), k
    o = MoEFFN(**oracle_inputs(inp), mode="faithful", gmm1=gmm1, bwd="fp8" if fp8bwd else "bf16")
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_tok, replace=False)]))
    ti = torch.from_numpy(toks).cuda()
    announce("oracle forward of %d tokens" % toks.size)
    ry, ryd = o.forward_dev(toks)
    assert_close(to_f64(y[ti]), ry, name + " y", ryd)
    announce("oracle backward of %d tokens" % toks.size)
    (rdx, rdw), (ddx, ddw) = o.backward_tokens_dev(toks)
    assert_close(to_f64(dx[ti]), rdx, name + " dx", ddx)
    assert_close(to_f64(dw[ti]), rdw, name + " d_topk_weights", ddw)
    counts = ref_route["counts"]
    nz = np.flatnonzero(counts)
    experts = {int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])]), int(rng.choice(nz))}
    experts |= set(np.flatnonzero(counts == 0)[:1].tolist())
    icols = np.unique([min(I - 1, int(f * I)) for f in icols_frac] + [int(rng.integers(I))])
    for e in sorted(experts):
        announce("oracle weight gradients of expert %d (%d rows)" % (e, counts[e]))
        (gcol, ucol, drow), (gd, ud, rd) = o.weight_grads_expert_dev(e, icols)
        assert_close(to_f64(dW1[e][:, icols]), gcol, "%s dW1[%d] gate cols" % (name, e), gd)
        assert_close(to_f64(dW1[e][:, icols + I]), ucol, "%s dW1[%d] up cols" % (name, e), ud)
        assert_close(to_f64(dW2[e][icols]), drow, "%s dW2[%d] rows" % (name, e), rd)
        if counts[e] == 0:
            assert not to_f64(dW1[e]).any() and not to_f64(dW2[e]).any()


@pytest.mark.slow
def test_full_size_sample_workload():
    """The pages' sample shape, checked in full (the oracle handles it in seconds)."""
    spec = synth.WORKLOADS["sample"]
    inp = synth.make_inputs(spec, seed=0)
    announce("full parity sample workload")
    g = gpu_inputs(inp, "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g)
    o = MoEFFN(**oracle_inputs(inp), mode="faithful")
    ry, ryd = o.forward_dev()
    assert_close(to_f64(y), ry, "sample y", ryd)
    (rdx, rdw, rdW1, rdW2), (ddx, ddw, ddW1, ddW2) = o.backward_dev()
    assert_close(to_f64(dx), rdx, "sample dx", ddx)
    assert_close(to_f64(dw), rdw, "sample d_topk_weights", ddw)
    assert_close(to_f64(dW1), rdW1, "sample dW1", ddW1)
    assert_close(to_f64(dW2), rdW2, "sample dW2", ddW2)


@pytest.mark.slow
def test_full_size_skewed_sampled():
    _sample_full("skewed")


@pytest.mark.slow
def test_full_size_hotspot_sampled():
    _sample_full("hotspot", n_tok=4)


@pytest.mark.slow
def test_full_size_fp8_sampled():
    """FP8 up-projection workload (T=16384, H=4096, I=1536, E=64, K=6)."""
    _sample_full("fp8", n_tok=4)


# ----------------------------------------------------------------------------- fused small-problem forward (opt-in)

FUSED = [
    ("sample-like", dict(T=1024, H=512, I=128, E=4, K=2, routing="uniform")),
    ("ragged", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform")),
    ("k1", dict(T=200, H=128, I=128, E=3, K=1, routing="uniform")),
    ("zipf-empty", dict(T=411, H=256, I=128, E=16, K=4, routing="zipf", zipf_s=1.2, n_empty=5)),
    ("max-slots", dict(T=1024, H=128, I=64, E=256, K=8, routing="uniform")),
]


@pytest.mark.parametrize("name,over", FUSED, ids=[f[0] for f in FUSED])
def test_fused_forward_equals_kernel_sequence(name, over):
    """The one-launch forward matches the FAITHFUL oracle (y, and the saved h and a
    element by element; the routing arrays bit-exactly), and gives bit-identical y
    and saved arrays to the kernel sequence."""
    import torch
    from mixture_experts_ffn_int32_amd import forward_with_saved, saved_views
    spec = synth.spec_with("tiny", **over)
    inp = synth.make_inputs(spec, seed=41)
    announce("fused forward %s %s" % (name, {k: spec[k] for k in "THIEK"}))
    g = gpu_inputs(inp, "cuda")
    args = (g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    y1, s1 = forward_with_saved(*args, tiles="narrow", fused=True)
    y0, s0 = forward_with_saved(*args, tiles="narrow", fused=False)
    torch.cuda.synchronize()
    v1 = saved_views(s1, *(spec[k] for k in "THIEK"), tiles="narrow")
    ref_route = oracle_route(inp["topk_ids"], spec["E"])
    for k in ("counts", "offsets", "sorted_slot", "row_of_slot"):
        assert np.array_equal(v1[k].cpu().numpy(), ref_route[k]), k
    announce("oracle forward and intermediates of %d slots" % ref_route["sorted_slot"].size)
    o = MoEFFN(**oracle_inputs(inp), mode="faithful")
    ry, ryd = o.forward_dev()
    assert_close(to_f64(y1), ry, "y", ryd)
    (h, a, _), (hd, ad, _) = o.slot_intermediates_dev(ref_route["sorted_slot"])
    assert_close(to_f64(v1["h"]), h, "h", hd)
    assert_close(to_f64(v1["a"]), a, "a", ad)
    assert torch.equal(y1, y0)
    v0 = saved_views(s0, *(spec[k] for k in "THIEK"), tiles="narrow")
    for k in v1:
        assert torch.equal(v1[k], v0[k]), k


def test_fused_forward_reports_a_wait_that_gives_up():
    """With the wait limit lowered from the host to one poll, the fused forward's waits
    give up (the routing item still runs; every workgroup ends normally): the call
    returns HMM_ERR_TIMEOUT.  The next call, at the default limit, is correct."""
    import ctypes
    import torch
    from mixture_experts_ffn_int32_amd import _lib, forward_with_saved
    spec = synth.spec_with("tiny", T=1024, H=512, I=128, E=4, K=2, routing="uniform")
    T, H, I, E, K = (spec[k] for k in "THIEK")
    lib = _lib.load()
    prob = _lib.Problem(T, H, I, E, K, _lib.HMM_BF16, _lib.HMM_BF16,
                        _lib.HMM_FLAG_VALIDATE_IDS | _lib.HMM_FLAG_FUSED_FORWARD | _lib.HMM_FLAG_TILES_NARROW, 0)
    ws, sv = ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(lib.hmm_forward_sizes(ctypes.byref(prob), ctypes.byref(ws), ctypes.byref(sv)))
    work = torch.zeros(ws.value, dtype=torch.uint8, device="cuda")
    saved = torch.empty(sv.value, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    g = gpu_inputs(synth.make_inputs(spec, seed=60), "cuda")

    def call():
        return lib.hmm_forward(ctypes.byref(prob), P(g["x"]), P(g["topk_ids"]), P(g["topk_weights"]),
                               P(g["up_proj_weight"]), P(g["down_proj_weight"]), P(y), P(saved), sv.value, P(work),
                               ws.value, stream)
    announce("fused forward with a one-poll wait limit")
    try:
        _lib.check(lib.hmm_set_fused_spin_limit(1))
        st = call()
    finally:
        _lib.check(lib.hmm_set_fused_spin_limit(0))
    assert st == _lib.HMM_ERR_TIMEOUT, lib.hmm_status_string(st)
    assert b"gave up" in lib.hmm_last_error_message()
    announce("fused forward after the failure, default limit")
    _lib.check(call())
    ref, _ = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                g["down_proj_weight"], tiles="narrow", fused=False)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


def test_fused_forward_reuses_its_workspace():
    """Raw calls on one workspace: counters from the previous call never leak into the next."""
    import ctypes
    import torch
    from mixture_experts_ffn_int32_amd import _lib, forward_with_saved
    spec = synth.spec_with("tiny", T=512, H=256, I=128, E=8, K=2, routing="uniform")
    T, H, I, E, K = (spec[k] for k in "THIEK")
    lib = _lib.load()
    prob = _lib.Problem(T, H, I, E, K, _lib.HMM_BF16, _lib.HMM_BF16,
                        _lib.HMM_FLAG_VALIDATE_IDS | _lib.HMM_FLAG_FUSED_FORWARD | _lib.HMM_FLAG_TILES_NARROW, 0)
    ws, sv = ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(lib.hmm_forward_sizes(ctypes.byref(prob), ctypes.byref(ws), ctypes.byref(sv)))
    work = torch.full((ws.value,), 0xA5, dtype=torch.uint8, device="cuda")   # garbage counters at the start
    saved = torch.empty(sv.value, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for seed in (50, 51, 52):
        g = gpu_inputs(synth.make_inputs(spec, seed=seed), "cuda")
        announce("fused forward, reused workspace, seed %d" % seed)
        _lib.check(lib.hmm_forward(ctypes.byref(prob), P(g["x"]), P(g["topk_ids"]), P(g["topk_weights"]),
                                   P(g["up_proj_weight"]), P(g["down_proj_weight"]), P(y), P(saved), sv.value,
                                   P(work), ws.value, stream))
        ref, _ = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                    g["down_proj_weight"], tiles="narrow", fused=False)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
