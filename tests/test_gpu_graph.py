"""The forward and backward captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: every replay, on inputs copied into the captured buffers between replays (new
ids too: the grids are sized by upper bounds, the routing reads the ids on the device),
gives the same bits as the eager calls on those inputs.  The calls allocate nothing and
issue no memset, and without the id check's read-back they never wait on the host, so
the whole step can be captured; the backward's second stream joins the capture through
its fork and join events."""

import pytest

from _util import announce, gpu_inputs
from mixture_experts_ffn_int32_amd import synth

pytestmark = pytest.mark.gpu

CASES = [
    # name, spec overrides, tiling
    ("large", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform"), "large"),
    ("narrow", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform"), "narrow"),
    ("shared", dict(T=200, H=128, I=128, E=4, K=2, routing="uniform", shared_I=128), "large"),
    ("multiblock", dict(T=3000, H=128, I=64, E=16, K=4, routing="zipf", zipf_s=1.1, n_empty=3), "auto"),
]
KEYS = ("x", "topk_ids", "topk_weights", "up_proj_weight", "down_proj_weight", "dY",
        "shared_up_proj_weight", "shared_down_proj_weight")


def _step(g, tiles):
    from mixture_experts_ffn_int32_amd import backward_from_saved, forward_with_saved
    sh = {k: g[k] for k in ("shared_up_proj_weight", "shared_down_proj_weight") if k in g}
    y, saved = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                  g["down_proj_weight"], validate_ids=False, tiles=tiles, **sh)
    grads = backward_from_saved(g["dY"], g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                g["down_proj_weight"], saved, tiles=tiles, **sh)
    return (y,) + tuple(grads)


@pytest.mark.parametrize("name,over,tiles", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, over, tiles):
    import torch
    spec = synth.spec_with("tiny", **over)
    inputs = [gpu_inputs(synth.make_inputs(spec, seed=s), "cuda") for s in (21, 22)]
    announce("graph capture %s %s tiles=%s" % (name, {k: spec[k] for k in "THIEK"}, tiles))
    ref = [tuple(t.clone() for t in _step(g, tiles)) for g in inputs]
    torch.cuda.synchronize()
    static = {k: v.clone() for k, v in inputs[0].items()}
    # warm-up on a side stream (the library's lazy per-device state is made outside the capture)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(static, tiles)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _step(static, tiles)
    for it, which in enumerate((1, 0, 1)):
        for k in KEYS:
            if k in static:
                static[k].copy_(inputs[which][k])
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref[which]):
            assert torch.equal(a, b), (name, it)
        # eager work between the replays
        _step(inputs[1 - which], tiles)
        torch.cuda.synchronize()
