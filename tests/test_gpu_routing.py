"""GPU routing (histogram, offsets, stable permutation) against the oracle, bit for bit."""

import numpy as np
import pytest

from _util import announce
from mixture_experts_ffn_int32_amd import synth
from oracle.routing import route as oracle_route

pytestmark = pytest.mark.gpu


def _gpu_route(ids_np, E, validate=True):
    import torch
    from mixture_experts_ffn_int32_amd import route
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to("cuda")
    out = route(ids, E, validate_ids=validate)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _check(ids, E, label):
    announce("route %s T=%d K=%d E=%d" % (label, ids.shape[0], ids.shape[1], E))
    got = _gpu_route(ids, E)
    ref = oracle_route(ids, E)
    for k in ("counts", "offsets", "sorted_slot", "row_of_slot"):
        assert np.array_equal(got[k], ref[k]), (label, k)


@pytest.mark.parametrize("name", ["tiny", "sample", "skewed", "hotspot", "fp8"])
def test_route_workloads_bit_exact(name):
    spec = synth.WORKLOADS[name]
    ids, _, _ = synth.make_routing(spec, seed=0)
    _check(ids, spec["E"], name)


@pytest.mark.parametrize("T,K,E,seed", [
    (1, 1, 1, 0), (1, 16, 16, 1), (3, 2, 1024, 2), (1023, 3, 7, 3), (1025, 1, 2, 4),
    (4000, 8, 128, 5), (700, 5, 1000, 6), (333, 16, 16, 7),
])
def test_route_random_bit_exact(T, K, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)   # duplicates allowed
    _check(ids, E, "random%d" % seed)


def test_route_degenerate_cases():
    _check(np.full((2049, 4), 3, np.int32), 5, "all-one-expert")        # others empty
    ids = np.tile(np.arange(8, dtype=np.int32), (300, 1))               # K = E
    _check(ids, 8, "K=E")
    _check(np.zeros((0, 2), np.int32), 4, "T=0")


def test_route_rejects_out_of_range_ids():
    from mixture_experts_ffn_int32_amd import _lib
    ids = np.zeros((100, 2), np.int32)
    ids[57, 1] = 9
    announce("route out-of-range id")
    with pytest.raises(ValueError) as ei:
        _gpu_route(ids, 9)
    assert ei.value.status == _lib.HMM_ERR_EXPERT_ID_OUT_OF_RANGE
    ids[57, 1] = -1
    with pytest.raises(ValueError):
        _gpu_route(ids, 9)
    # without validation the bad slot is dropped and the rest is still exact
    got = _gpu_route(ids, 9, validate=False)
    flat = ids.reshape(-1)
    good = flat >= 0
    assert got["row_of_slot"][~good].tolist() == [-1]
    assert got["counts"].sum() == good.sum()
    # a valid call right after the failures is exact
    ids[57, 1] = 4
    _check(ids, 9, "after-failure")
