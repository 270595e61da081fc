"""The no-allocation forward (hmm_forward_noalloc) against hmm_forward (collected last).

Both run the same kernels; the no-allocation variant takes its workspace from
the library's own device array.  Two calls in a row, the second on a smaller
problem (the array keeps the first call's contents), must give y and every
saved array bit-identical to hmm_forward's on the same inputs; y also matches
the FAITHFUL oracle.  The variant rejects what it does not take, before any
launch.
"""

import ctypes

import numpy as np
import pytest

from _util import announce, assert_close, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN

pytestmark = pytest.mark.gpu

CASES = [
    ("first", dict(T=1024, H=512, I=128, E=8, K=2, routing="uniform"), 71),
    ("second, smaller", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform"), 72),
]


def _forward(lib, _lib, prob, g, noalloc):
    import torch
    T, H = g["x"].shape
    ws, sv = ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(lib.hmm_forward_sizes(ctypes.byref(prob), ctypes.byref(ws), ctypes.byref(sv)))
    saved = torch.full((sv.value,), 0x5A, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (ctypes.byref(prob), P(g["x"]), P(g["topk_ids"]), P(g["topk_weights"]), P(g["up_proj_weight"]),
            P(g["down_proj_weight"]), P(y), P(saved), sv.value)
    if noalloc:
        _lib.check(lib.hmm_forward_noalloc(*args, stream))
    else:
        work = torch.empty(ws.value, dtype=torch.uint8, device="cuda")
        _lib.check(lib.hmm_forward(*args, P(work), ws.value, stream))
    torch.cuda.synchronize()
    return y, saved


def test_noalloc_forward_equals_hmm_forward_twice():
    import torch
    from mixture_experts_ffn_int32_amd import _lib, saved_views
    lib = _lib.load()
    for name, over, seed in CASES:
        spec = synth.spec_with("tiny", **over)
        T, H, I, E, K = (spec[k] for k in "THIEK")
        inp = synth.make_inputs(spec, seed=seed)
        g = gpu_inputs(inp, "cuda")
        prob = _lib.Problem(T, H, I, E, K, _lib.HMM_BF16, _lib.HMM_BF16, 0, 0)
        announce("no-allocation forward, %s call %s" % (name, {k: spec[k] for k in "THIEK"}))
        y1, s1 = _forward(lib, _lib, prob, g, noalloc=True)
        y0, s0 = _forward(lib, _lib, prob, g, noalloc=False)
        assert torch.equal(y1, y0), name
        v1, v0 = saved_views(s1, T, H, I, E, K), saved_views(s0, T, H, I, E, K)
        for k in v0:
            assert torch.equal(v1[k], v0[k]), (name, k)
        ry, ryd = MoEFFN(**oracle_inputs(inp), mode="faithful").forward_dev()
        assert_close(to_f64(y1), ry, "y (%s)" % name, ryd)


def test_noalloc_forward_rejects_what_it_does_not_take():
    import torch
    from mixture_experts_ffn_int32_amd import _lib
    lib = _lib.load()
    spec = synth.spec_with("tiny", T=64, H=128, I=64, E=4, K=2)
    g = gpu_inputs(synth.make_inputs(spec, seed=73), "cuda")
    y = torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")
    saved = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    announce("no-allocation forward: rejected inputs")

    def call(prob):
        return lib.hmm_forward_noalloc(ctypes.byref(prob), P(g["x"]), P(g["topk_ids"]), P(g["topk_weights"]),
                                       P(g["up_proj_weight"]), P(g["down_proj_weight"]), P(y), P(saved),
                                       saved.numel(), None)
    for flags in (_lib.HMM_FLAG_VALIDATE_IDS, _lib.HMM_FLAG_FUSED_FORWARD | _lib.HMM_FLAG_TILES_NARROW):
        assert call(_lib.Problem(64, 128, 64, 4, 2, _lib.HMM_BF16, _lib.HMM_BF16, flags, 0)) == _lib.HMM_ERR_UNSUPPORTED
    # a problem whose forward workspace exceeds the 64 MiB array (S*H*2 = 128 MiB)
    big = _lib.Problem(8192, 8192, 64, 4, 1, _lib.HMM_BF16, _lib.HMM_BF16, 0, 0)
    assert call(big) == _lib.HMM_ERR_WORKSPACE_TOO_SMALL
    assert b"no-allocation" in lib.hmm_last_error_message()
    torch.cuda.synchronize()
