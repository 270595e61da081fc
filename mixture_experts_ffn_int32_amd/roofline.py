"""Algorithmic work and MI355X peaks of the library's stages (roofline figures).

Shared by bench.py (live figures from the stage events) and profsum (figures
from a rocprofv3 kernel trace).  Work counts what the method needs, not what a
kernel happens to move: FLOPs of the products over the routed rows (no tile
padding), and for the memory-bound kernels each operand read once and each
output written once (the per-slot and per-token sizes of the hot-path scope
table).
"""

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def stage_work(stage, T, H, I, E, K, f32=False, Is=0):
    """Algorithmic work of one launch of a stage: (bound, amount, unit, peak).

    The float32-output mode counts the same algorithmic flops (its hi/lo operand
    pairs make the MFMAs do about 1.9x that work) and float32 rows in the combines.
    Is > 0: a shared expert of that width (one more group of all T rows)."""
    S = T * K
    eb = 4 if f32 else 2
    if stage in ("gmm1_fp8_swiglu", "gmm1_mx_swiglu", "gmm1_group_swiglu"):
        return "mfma", 4 * S * H * I, "TFLOP/s", PEAK_FP8_TFLOPS
    if stage == "act_grad_fp8":     # FP8 backward: [S,H] x [H,I] on E4M3
        return "mfma", 2 * S * H * I, "TFLOP/s", PEAK_FP8_TFLOPS
    if stage == "input_grad_fp8":   # [S,2I] x [2I,H] on E4M3
        return "mfma", 4 * S * H * I, "TFLOP/s", PEAK_FP8_TFLOPS
    flops = {
        "gmm1_swiglu": 4 * S * H * I,   # [S,H] x [H,2I]
        "gmm2": 2 * S * I * H,          # [S,I] x [I,H]
        "act_grad": 2 * S * H * I,      # [S,H] x [H,I]
        "input_grad": 4 * S * I * H,    # [S,2I] x [2I,H]
        "dw2": 2 * S * I * H,           # [I,S] x [S,H]
        "dw1": 4 * S * H * I,           # [H,S] x [S,2I]
    }
    flops["act_grad+dw2"] = flops["act_grad"] + flops["dw2"]      # two products in one launch
    flops["input_grad+dw1"] = flops["input_grad"] + flops["dw1"]
    flops["route+gmm1_swiglu"] = flops["gmm1_swiglu"]  # small problems: the routing rides in the up-projection
    # a shared expert: the same products over T rows of width Is, in the routed launches ("<stage>+shared")
    shared = {k: v * T * Is // (S * I) for k, v in flops.items()}
    for k, v in shared.items():
        flops[k + "+shared"] = flops[k] + v
        flops["shared_" + k] = v                      # its own launches (float32-output mode)
    flops["shared_gmm1"] = shared["gmm1_swiglu"]
    if stage in flops:
        return "mfma", flops[stage], "TFLOP/s", PEAK_BF16_TFLOPS
    nbytes = {
        # read K gathered rows per token + row index + weight, write one row
        "combine": S * H * eb + S * 8 + T * H * eb + (T * H * eb if Is else 0),   # (+ shared rows)
        "combine_dx": S * H * eb + S * 4 + T * H * eb + (T * H * eb if Is else 0),  # (+ d_topk_weights partials)
        "shared_tables": T * 12,
        "split_dy": T * H * 4 + T * H * 4,              # float32 dY -> bf16 hi | lo
        # algorithmic: ids read once, sorted_slot + row_of_slot written (12 S bytes)
        "route": S * 12,
        "route_narrow": S * 12,   # the per-group product's 64-row tile table
        # FP8 quantisers: read the bf16 operand once, write its codes and descales
        "quant_x": T * H * 2 + T * H + T * 4,
        "quant_w1": E * H * 2 * I * 2 + E * H * 2 * I + E * 2 * I * 4,
        # MX quantisers: the bf16 operand once, its codes and one exponent byte per 32 elements
        "quant_x_mx": T * H * 2 + T * H + T * H // 32,
        "quant_w1_mx": E * H * 2 * I * 2 + E * H * 2 * I + E * 2 * I * H // 32,
        # per group of 128 along H: one float32 descale per token row / weight column
        "quant_x_group": T * H * 2 + T * H + T * (H // 128) * 4,
        "quant_w1_group": E * H * 2 * I * 2 + E * H * 2 * I + E * (H // 128) * 2 * I * 4,
        # FP8 backward's per-row quantisers: bf16 rows in, E4M3 codes and one descale per row out
        "quant_dy": T * H * 3 + T * 4,
        "quant_w2": E * I * H * 3 + E * I * 4,
        "quant_dh": S * 2 * I * 3 + S * 4,
        "quant_w1r": E * H * 2 * I * 3 + E * H * 4,
    }
    if stage in nbytes:
        return "hbm", nbytes[stage], "GB/s", PEAK_HBM_GBS
    return None, 0, None, None
