"""Seeded synthetic inputs for the MoE-FFN workloads.

This module only draws random numbers; it holds none of the method's
arithmetic, so both the HIP path and the CPU oracle may consume what it makes.
bfloat16 values are produced by torch's float32 -> bfloat16 conversion and
handed out as uint16 bit patterns (numpy has no bfloat16 dtype).

Recipe (every workload):
* one numpy PCG64 stream per tensor, spawned from SeedSequence(seed);
* x ~ N(0, 1), dY ~ N(0, 1);
* up_proj_weight [E,H,2I] ~ N(0, 1/H), down_proj_weight [E,I,H] ~ N(0, 1/I)
  (variance 1/fan_in; fan_in is the contracted dimension);
* topk_weights = softmax over K of N(0, 1) logits, float32;
* the K ids of a token are kept in the order they were drawn;
* with ``shared_I`` = Is > 0 in the spec, a shared expert: shared_up_proj_weight
  [H,2Is] ~ N(0, 1/H) and shared_down_proj_weight [Is,H] ~ N(0, 1/Is), from
  streams of their own (the other tensors do not change).

Routing structures:
* ``uniform``: K distinct experts per token, uniformly (the first K entries of
  a uniformly random permutation of the E experts);
* ``zipf``: K distinct experts per token drawn without replacement with
  probability proportional to rank**-s over the first E - n_empty experts of a
  seeded permutation of all experts, so that n_empty experts receive no
  token (successive sampling without replacement, done as Gumbel-top-K);
* ``hot``: one seeded hot expert sits in every token at a random position, the
  other K - 1 are distinct and uniform over the remaining experts
  (``hot_dup`` puts the hot expert in two positions of every token);
* ``counts``: K = 1 and expert e receives exactly ``counts[e]`` tokens, in a
  seeded random token order (T = sum of the counts), to place expert sizes on
  chosen tile boundaries.
"""

import math

import numpy as np
import torch

WORKLOADS = {
    # tiny case the oracle finishes in seconds
    "tiny": dict(T=128, H=128, I=64, E=4, K=2, routing="uniform"),
    # the usage guide's sample module shape
    "sample": dict(T=1024, H=512, I=128, E=4, K=2, routing="uniform"),
    # skewed Zipf routing with tail tokens and empty experts
    "skewed": dict(T=4000, H=2048, I=768, E=128, K=8, routing="zipf", zipf_s=1.2, n_empty=10),
    # large hidden size with one hot expert
    "hotspot": dict(T=8192, H=7168, I=2048, E=32, K=8, routing="hot"),
    # FP8 up-projection variant with 1% outlier token rows
    "fp8": dict(T=16384, H=4096, I=1536, E=64, K=6, routing="uniform",
                outlier_frac=0.01, outlier_scale=20.0, gmm1="fp8"),
    # the same shape with the MX (32-block) quantised up-projection
    "mx": dict(T=16384, H=4096, I=1536, E=64, K=6, routing="uniform",
               outlier_frac=0.01, outlier_scale=20.0, gmm1="mx"),
    # the FP8 workload with the FP8 backward as well (act_grad and input_grad on E4M3)
    "fp8bwd": dict(T=16384, H=4096, I=1536, E=64, K=6, routing="uniform",
                   outlier_frac=0.01, outlier_scale=20.0, gmm1="fp8", fp8_backward=True),
    # the same shape with the per-group (128 along H) quantised up-projection
    "group": dict(T=16384, H=4096, I=1536, E=64, K=6, routing="uniform",
                  outlier_frac=0.01, outlier_scale=20.0, gmm1="group"),
}


def to_bf16_bits(a):
    """float32 array -> uint16 bfloat16 bit patterns (torch's conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits):
    """uint16 bfloat16 bit patterns -> exact float32 values."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, std, chunk=1 << 24):
    """N(0, std^2) float32 array, drawn in chunks to bound temporaries."""
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for i in range(0, out.size, chunk):
        n = min(chunk, out.size - i)
        out[i:i + n] = rng.standard_normal(n, dtype=np.float32)
        if std != 1.0:
            out[i:i + n] *= np.float32(std)
    return out.reshape(shape)


def _bf16_normal(rng, shape, std):
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    chunk = 1 << 24
    for i in range(0, flat.size, chunk):
        n = min(chunk, flat.size - i)
        v = rng.standard_normal(n, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        flat[i:i + n] = to_bf16_bits(v)
    return out


def route_uniform(rng, T, E, K):
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1)[:, :K].astype(np.int32)


def route_zipf(rng, T, E, K, s, n_empty):
    support = E - n_empty
    if support < K:
        raise ValueError("Zipf support smaller than K")
    perm = rng.permutation(E)
    logp = -s * np.log(np.arange(1, support + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(rng.random((T, support))))
    order = np.argsort(-(logp[None, :] + gumbel), axis=1)[:, :K]
    return perm[:support][order].astype(np.int32)


def route_hot(rng, T, E, K, dup=False):
    hot = int(rng.integers(E))
    others = np.array([e for e in range(E) if e != hot])
    n_hot = 2 if dup else 1
    rest = others[np.argsort(rng.random((T, E - 1)), axis=1)[:, :K - n_hot]]
    ids = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        pos = rng.permutation(K)[:n_hot]
        mask = np.zeros(K, bool)
        mask[pos] = True
        ids[t, mask] = hot
        ids[t, ~mask] = rest[t]
    return ids, hot


def route_counts(rng, T, E, K, counts):
    counts = np.asarray(counts, np.int64)
    if K != 1 or counts.shape != (E,) or counts.sum() != T or (counts < 0).any():
        raise ValueError("counts routing needs K = 1 and E non-negative counts summing to T")
    return rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)).reshape(T, 1)


def softmax_weights(rng, T, K):
    z = rng.standard_normal((T, K))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def make_routing(spec, seed=0):
    """(topk_ids int32 [T,K], topk_weights float32 [T,K], info dict)."""
    T, E, K = spec["T"], spec["E"], spec["K"]
    ss = np.random.SeedSequence([seed, 1])
    r_ids, r_w = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(2)]
    info = {}
    kind = spec.get("routing", "uniform")
    if kind == "uniform":
        ids = route_uniform(r_ids, T, E, K)
    elif kind == "zipf":
        ids = route_zipf(r_ids, T, E, K, spec.get("zipf_s", 1.2), spec.get("n_empty", 10))
    elif kind in ("hot", "hot_dup"):
        ids, info["hot_expert"] = route_hot(r_ids, T, E, K, dup=(kind == "hot_dup"))
    elif kind == "counts":
        ids = route_counts(r_ids, T, E, K, spec["counts"])
    else:
        raise ValueError(kind)
    return ids, softmax_weights(r_w, T, K), info


def make_inputs(spec, seed=0, with_dy=True):
    """All inputs of one problem; bf16 tensors as uint16 bit arrays.

    Returns dict(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight,
    dY, info), plus shared_up_proj_weight and shared_down_proj_weight when the
    spec has shared_I > 0.
    """
    T, H, I, E = spec["T"], spec["H"], spec["I"], spec["E"]
    ss = np.random.SeedSequence([seed, 0])
    r_x, r_w1, r_w2, r_dy, r_out = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]
    xf = _normal(r_x, (T, H), 1.0)
    frac = spec.get("outlier_frac", 0.0)
    if frac > 0 and T > 0:
        n = int(math.ceil(frac * T))
        rows = r_out.choice(T, size=n, replace=False)
        xf[rows] *= np.float32(spec.get("outlier_scale", 1.0))
    ids, w, info = make_routing(spec, seed)
    out = {
        "x": to_bf16_bits(xf),
        "topk_ids": ids,
        "topk_weights": w,
        "up_proj_weight": _bf16_normal(r_w1, (E, H, 2 * I), 1.0 / math.sqrt(H)),
        "down_proj_weight": _bf16_normal(r_w2, (E, I, H), 1.0 / math.sqrt(I)),
        "info": info,
    }
    if with_dy:
        out["dY"] = _bf16_normal(r_dy, (T, H), 1.0)
    Is = spec.get("shared_I", 0)
    if Is:
        r_s1, r_s2 = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence([seed, 2]).spawn(2)]
        out["shared_up_proj_weight"] = _bf16_normal(r_s1, (H, 2 * Is), 1.0 / math.sqrt(H))
        out["shared_down_proj_weight"] = _bf16_normal(r_s2, (Is, H), 1.0 / math.sqrt(Is))
    return out


def spec_with(base, **kw):
    """Copy of a workload spec with some fields replaced."""
    s = dict(WORKLOADS[base] if isinstance(base, str) else base)
    s.update(kw)
    return s
