"""Helpers shared by the tests: tensor conversion, tolerance checks, case printing."""

import sys

import numpy as np

from mixture_experts_ffn_int32_amd import synth

# bf16 outputs and gradients against the FAITHFUL oracle: |gpu - ref| <= ATOL + RTOL |ref|
RTOL = 1e-2
ATOL = 1e-2


# pytest's capture manager (set by conftest): announce() writes past the
# capture, so a long test shows its progress while it runs
_capman = None


def announce(msg):
    """Name the case before a GPU step, flushed, so a crash log says what ran.

    The line goes to the real stdout even while pytest captures output, so a
    long test prints progress as it goes instead of only after it ends."""
    if _capman is not None:
        with _capman.global_and_fixture_disabled():
            print("[case] %s" % msg, flush=True)
    else:
        print("[case] %s" % msg, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def assert_close(got, ref, name, dev=0.0, rtol=RTOL, atol=ATOL):
    """|got - ref| <= atol + rtol |ref| + dev, elementwise.

    ``dev`` is the oracle's admissible deviation: nonzero only where a bf16
    rounding decision upstream is open (see oracle.moe_ffn)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref) + dev
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err, -1)), got.shape)
        raise AssertionError("%s: %d of %d entries outside |d| <= %g + %g|ref|; worst at %s: got %r ref %r"
                             % (name, int(bad.sum()), bad.size, atol, rtol, idx, got[idx], ref[idx]))


def gpu_inputs(inp, device):
    """Upload a synth.make_inputs() dict."""
    import torch
    out = {
        "x": bf16_tensor(inp["x"], device),
        "topk_ids": torch.from_numpy(inp["topk_ids"]).to(device),
        "topk_weights": torch.from_numpy(inp["topk_weights"]).to(device),
        "up_proj_weight": bf16_tensor(inp["up_proj_weight"], device),
        "down_proj_weight": bf16_tensor(inp["down_proj_weight"], device),
    }
    if "dY" in inp:
        out["dY"] = bf16_tensor(inp["dY"], device)
    for k in ("shared_up_proj_weight", "shared_down_proj_weight"):
        if k in inp:
            out[k] = bf16_tensor(inp[k], device)
    return out


def oracle_inputs(inp):
    """float32 views (exact bf16 values) for the oracle."""
    d = {
        "x": synth.bits_to_f32(inp["x"]),
        "topk_ids": inp["topk_ids"],
        "topk_weights": inp["topk_weights"],
        "up_proj_weight": synth.bits_to_f32(inp["up_proj_weight"]),
        "down_proj_weight": synth.bits_to_f32(inp["down_proj_weight"]),
    }
    if "dY" in inp:
        d["dY"] = synth.bits_to_f32(inp["dY"])
    for k in ("shared_up_proj_weight", "shared_down_proj_weight"):
        if k in inp:
            d[k] = synth.bits_to_f32(inp[k])
    return d
