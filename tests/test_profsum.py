"""The profile summariser: kernel names to stages, overlap detection (CPU only)."""

import csv

from mixture_experts_ffn_int32_amd.profsum import overlapping, stage_of

NS = "hmm::(anonymous namespace)::"


def test_stage_names_of_the_library_kernels():
    cases = [
        ("void %sgemm_pair_kernel<%sGmm1<%sCfg<256, 256, 2, 4, 64>, false>, %sGmm1<%sCfg<64, 256, 2, 4, 64>, true> >"
         "(args)" % (NS, NS, NS, NS, NS), "gmm1_swiglu[256x256+64x256]", "gmm1_swiglu"),
        ("void %sgemm_kernel<%sDw<%sCfg<256, 256, 2, 4, 64>, true, false> >(args)" % (NS, NS, NS),
         "dw1[256x256]", "dw1"),
        ("void %sgemm_kernel<%sDw<%sCfg<256, 256, 2, 4, 64>, false, true> >(args)" % (NS, NS, NS),
         "dw2[256x256]", "dw2"),
        ("void %sgemm_fp8_kernel<%sGmm1F8K<%sF8Cfg<256, 256, 2, 4, 1>, false, 0> >(args)" % (NS, NS, NS),
         "gmm1_fp8_swiglu", "gmm1_fp8_swiglu"),
        ("void %sgemm_fp8_kernel<%sGmm1F8K<%sF8Cfg<64, 256, 2, 4, 2>, true, 2> >(args)" % (NS, NS, NS),
         "gmm1_group_swiglu", "gmm1_group_swiglu"),
        ("void %sgemm_fp8_kernel<%sActGradF8<%sF8Cfg<64, 256, 1, 4, 2>, true> >(args)" % (NS, NS, NS),
         "act_grad_fp8", "act_grad_fp8"),
        ("void %sgemm_fp8_kernel<%sInputGradF8<%sF8Cfg<256, 256, 2, 4, 1>, false> >(args)" % (NS, NS, NS),
         "input_grad_fp8", "input_grad_fp8"),
        ("void hmm::combine_kernel<true, unsigned short>(args)", "combine", "combine"),
        ("void hmm::combine_kernel<false, unsigned short>(args)", "combine_dx", "combine_dx"),
        ("hmm::route_scan(int const*, int)", "route_scan", "route"),
        ("void %sgemm_kernel<%sGmm1Routed>(args)" % (NS, NS), "route+gmm1_swiglu", "route+gmm1_swiglu"),
        ("hmm::expert_order(int const*, int, int*)", "expert_order", "expert_order"),
        ("hmm::quant_rows_fp8(unsigned short const*, long)", "quant_rows_fp8", "quant_rows_fp8"),
    ]
    for name, label, stage in cases:
        lab, st = stage_of(name)
        assert st == stage, (name, st)
        assert lab.startswith(label), (name, lab)


def _trace(tmp_path, rows):
    d = tmp_path / "prof_x"
    d.mkdir()
    with open(d / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(rows)
    return str(d)


def test_overlap_ignores_kernel_end_slack_and_finds_two_streams(tmp_path):
    # back to back on one stream, overlapping by 2 us at each boundary: no overlap
    d = _trace(tmp_path, [("a", 0, 100000), ("b", 98000, 300000), ("c", 298000, 400000)])
    assert overlapping(d) == set()
    # c runs beside b for 150 us (a second stream)
    (tmp_path / "prof_x" / "x_kernel_trace.csv").unlink()
    (tmp_path / "prof_x").rmdir()
    d = _trace(tmp_path, [("a", 0, 100000), ("b", 100000, 400000), ("c", 150000, 300000), ("d", 400500, 500000)])
    assert overlapping(d) == {"b", "c"}
