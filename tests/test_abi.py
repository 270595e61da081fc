"""The C ABI on the CPU: the library loads, exports every declared symbol, and its
host-side checks reject bad problems before any HIP call (no GPU is touched)."""

import ctypes
import os
import re

import pytest

from mixture_experts_ffn_int32_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hmm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_ffn_int32_amd import build
        build.build(verbose=False)
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hmm_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_status_strings(lib):
    assert lib.hmm_status_string(0) == b"HMM_OK"
    assert lib.hmm_status_string(7) == b"HMM_ERR_EXPERT_ID_OUT_OF_RANGE"
    assert b"gfx950" in lib.hmm_build_info()


def _prob(**kw):
    d = dict(T=1024, H=512, I=128, E=4, K=2, out_dtype=_lib.HMM_BF16, gmm1_dtype=_lib.HMM_BF16,
             flags=_lib.HMM_FLAG_VALIDATE_IDS, shared_I=0)
    d.update(kw)
    return _lib.Problem(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(H=500), _lib.HMM_ERR_BAD_SHAPE), (dict(I=32), _lib.HMM_ERR_BAD_SHAPE), (dict(K=0), _lib.HMM_ERR_BAD_SHAPE),
    (dict(K=17), _lib.HMM_ERR_BAD_SHAPE), (dict(E=0), _lib.HMM_ERR_BAD_SHAPE), (dict(E=1025), _lib.HMM_ERR_BAD_SHAPE),
    (dict(T=-1), _lib.HMM_ERR_BAD_SHAPE), (dict(T=1 << 28, K=16), _lib.HMM_ERR_BAD_SHAPE),
    (dict(out_dtype=7), _lib.HMM_ERR_BAD_DTYPE), (dict(gmm1_dtype=9), _lib.HMM_ERR_BAD_DTYPE),
    (dict(out_dtype=_lib.HMM_F32, gmm1_dtype=_lib.HMM_FP8_E4M3), _lib.HMM_ERR_UNSUPPORTED),
    (dict(gmm1_dtype=_lib.HMM_FP8_E4M3, H=192), _lib.HMM_ERR_BAD_SHAPE), (dict(flags=64), _lib.HMM_ERR_BAD_SHAPE),
    (dict(flags=_lib.HMM_FLAG_FP8_BACKWARD, out_dtype=_lib.HMM_F32), _lib.HMM_ERR_UNSUPPORTED),
    (dict(flags=_lib.HMM_FLAG_FP8_BACKWARD, H=192), _lib.HMM_ERR_BAD_SHAPE),
    (dict(gmm1_dtype=_lib.HMM_MXFP8_E4M3, H=192), _lib.HMM_ERR_BAD_SHAPE), (dict(gmm1_dtype=5), _lib.HMM_ERR_BAD_DTYPE),
    (dict(gmm1_dtype=_lib.HMM_FP8_E4M3_GROUP, H=192), _lib.HMM_ERR_BAD_SHAPE),
    (dict(gmm1_dtype=_lib.HMM_FP8_E4M3_GROUP, flags=_lib.HMM_FLAG_VALIDATE_IDS | _lib.HMM_FLAG_TILES_LARGE),
     _lib.HMM_OK),
    (dict(out_dtype=_lib.HMM_F32, gmm1_dtype=_lib.HMM_FP8_E4M3_GROUP), _lib.HMM_ERR_UNSUPPORTED),
    (dict(out_dtype=_lib.HMM_F32, gmm1_dtype=_lib.HMM_MXFP8_E4M3), _lib.HMM_ERR_UNSUPPORTED),
    (dict(shared_I=1), _lib.HMM_ERR_BAD_SHAPE), (dict(shared_I=32), _lib.HMM_ERR_BAD_SHAPE),
    (dict(shared_I=65600), _lib.HMM_ERR_BAD_SHAPE), (dict(flags=6), _lib.HMM_ERR_BAD_SHAPE),
])
def test_sizes_reject_bad_problems(lib, kw, status):
    ws, sv = ctypes.c_size_t(), ctypes.c_size_t()
    p = _prob(**kw)
    assert lib.hmm_forward_sizes(ctypes.byref(p), ctypes.byref(ws), ctypes.byref(sv)) == status
    assert lib.hmm_last_error_message()


def test_sizes_and_layout(lib):
    ws, sv, bws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    p = _prob()
    assert lib.hmm_forward_sizes(ctypes.byref(p), ctypes.byref(ws), ctypes.byref(sv)) == 0
    assert lib.hmm_backward_sizes(ctypes.byref(p), ctypes.byref(bws)) == 0
    L = _lib.SavedLayout()
    assert lib.hmm_saved_layout_of(ctypes.byref(p), ctypes.byref(L)) == 0
    S, I = 1024 * 2, 128
    assert L.total == sv.value
    offs = [L.counts, L.offsets, L.sorted_slot, L.row_of_slot, L.tok_of_row, L.tiles, L.h, L.a, L.aw, L.id_error]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L.a - L.h >= S * 2 * I * 2 and L.aw - L.a >= S * I * 2
    assert ws.value >= S * 512 * 2          # o [S, H] bf16
    assert bws.value >= S * (2 * I + 512) * 2


def test_null_and_misaligned_pointers_rejected_without_launch(lib):
    p = _prob()
    z = ctypes.c_void_p(0)
    st = lib.hmm_forward(ctypes.byref(p), z, z, z, z, z, z, z, 0, z, 0, z)
    assert st == _lib.HMM_ERR_NULL_POINTER
    bad = ctypes.c_void_p(0x1001)             # never dereferenced: the check fails first
    st = lib.hmm_forward(ctypes.byref(p), bad, bad, bad, bad, bad, bad, bad, 1 << 30, bad, 1 << 30, z)
    assert st == _lib.HMM_ERR_MISALIGNED
    ok = ctypes.c_void_p(0x1000)              # aligned, but the buffers are declared too small
    st = lib.hmm_forward(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, 16, ok, 16, z)
    assert st == _lib.HMM_ERR_WORKSPACE_TOO_SMALL


def test_profile_read_without_launches(lib):
    lib.hmm_profile_enable(1)
    buf = (_lib.StageTime * 8)()
    n, dropped = ctypes.c_int32(-1), ctypes.c_int32(-1)
    assert lib.hmm_profile_read(buf, 8, ctypes.byref(n), ctypes.byref(dropped)) == 0
    assert n.value == 0 and dropped.value == 0
    lib.hmm_profile_enable(0)


def test_f32_mode_sizes(lib):
    """The accuracy mode keeps h in float32 and a, aw as [hi | lo] pairs; its workspaces grow to match."""
    sizes = {}
    for out in (_lib.HMM_BF16, _lib.HMM_F32):
        p = _prob(out_dtype=out)
        ws, sv, bws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        assert lib.hmm_forward_sizes(ctypes.byref(p), ctypes.byref(ws), ctypes.byref(sv)) == 0
        assert lib.hmm_backward_sizes(ctypes.byref(p), ctypes.byref(bws)) == 0
        L = _lib.SavedLayout()
        assert lib.hmm_saved_layout_of(ctypes.byref(p), ctypes.byref(L)) == 0
        sizes[out] = (ws.value, sv.value, bws.value, L)
    S, H, I, T = 2048, 512, 128, 1024
    L = sizes[_lib.HMM_F32][3]
    assert L.a - L.h >= S * 2 * I * 4 and L.aw - L.a >= S * 2 * I * 2 and L.id_error - L.aw >= S * 2 * I * 2
    assert sizes[_lib.HMM_F32][0] >= S * H * 4                       # o in float32
    assert sizes[_lib.HMM_F32][2] >= T * 2 * H * 2 + S * 4 * I * 2 + S * H * 4
    assert all(sizes[_lib.HMM_F32][i] > sizes[_lib.HMM_BF16][i] for i in range(3))


def test_shared_expert_sizes_and_entry_points(lib):
    """A shared expert (shared_I = Is) adds its tables, h_s and a_s to ``saved`` and its
    output / dH / dX rows to the workspaces; the plain entry points refuse such a problem."""
    T, H, I, Is = 1024, 512, 128, 192
    base, shr = _prob(), _prob(shared_I=Is)
    got = {}
    for name, p in (("base", base), ("shared", shr)):
        ws, sv, bws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        assert lib.hmm_forward_sizes(ctypes.byref(p), ctypes.byref(ws), ctypes.byref(sv)) == 0
        assert lib.hmm_backward_sizes(ctypes.byref(p), ctypes.byref(bws)) == 0
        L = _lib.SavedLayout()
        assert lib.hmm_saved_layout_of(ctypes.byref(p), ctypes.byref(L)) == 0
        got[name] = (ws.value, sv.value, bws.value, L)
    Lb, Ls = got["base"][3], got["shared"][3]
    assert Lb.shared_h == Lb.shared_a == Lb.total                      # empty without a shared expert
    offs = [Ls.id_error, Ls.shared_offsets, Ls.shared_idx, Ls.shared_ones, Ls.shared_tiles, Ls.shared_h,
            Ls.shared_a, Ls.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert Ls.shared_ones - Ls.shared_idx >= T * 4 and Ls.shared_a - Ls.shared_h >= T * 2 * Is * 2
    assert Ls.total - Ls.shared_a >= T * Is * 2
    assert got["shared"][0] - got["base"][0] >= T * H * 2                     # shared output rows
    assert got["shared"][2] - got["base"][2] >= T * 2 * Is * 2 + T * H * 2      # shared dH and dX rows
    z = ctypes.c_void_p(0)
    ok = ctypes.c_void_p(0x1000)              # never dereferenced: every check fails first
    assert lib.hmm_forward(ctypes.byref(shr), ok, ok, ok, ok, ok, ok, ok, 1 << 40, ok, 1 << 40, z) == \
        _lib.HMM_ERR_BAD_SHAPE
    assert lib.hmm_backward(ctypes.byref(shr), ok, ok, ok, ok, ok, ok, ok, 1 << 40, ok, ok, ok, ok, ok, 1 << 40,
                            z) == _lib.HMM_ERR_BAD_SHAPE
    # the shared weights are required with shared_I > 0, ignored without
    assert lib.hmm_forward_shared(ctypes.byref(shr), ok, ok, ok, ok, ok, z, z, ok, ok, 1 << 40, ok, 1 << 40, z) == \
        _lib.HMM_ERR_NULL_POINTER
    assert b"shared_up_proj_weight" in lib.hmm_last_error_message()
    assert lib.hmm_backward_shared(ctypes.byref(shr), ok, ok, ok, ok, ok, ok, ok, ok, ok, 1 << 40, ok, ok, ok, z, z,
                                   ok, ok, 1 << 40, z) == _lib.HMM_ERR_NULL_POINTER
    assert lib.hmm_forward_shared(ctypes.byref(base), ok, ok, ok, ok, ok, z, z, ok, ok, 16, ok, 16, z) == \
        _lib.HMM_ERR_WORKSPACE_TOO_SMALL


def test_group_quantisers_reject_bad_shapes_and_pointers(lib):
    """Per-group quantisers: H must be a multiple of 128 (the group), N of 8; NULL
    pointers are rejected; T = 0 is a no-op.  All before any HIP call."""
    z = ctypes.c_void_p(0)
    ok = ctypes.c_void_p(0x1000)
    assert lib.hmm_quant_rows_group(ok, 4, 192, ok, ok, z) == _lib.HMM_ERR_BAD_SHAPE
    assert lib.hmm_quant_rows_group(ok, -1, 256, ok, ok, z) == _lib.HMM_ERR_BAD_SHAPE
    assert lib.hmm_quant_rows_group(z, 4, 256, ok, ok, z) == _lib.HMM_ERR_NULL_POINTER
    assert lib.hmm_quant_rows_group(ok, 4, 256, ok, z, z) == _lib.HMM_ERR_NULL_POINTER
    assert lib.hmm_quant_rows_group(z, 0, 256, z, z, z) == _lib.HMM_OK
    assert lib.hmm_quant_cols_group(ok, 2, 192, 64, ok, ok, z) == _lib.HMM_ERR_BAD_SHAPE
    assert lib.hmm_quant_cols_group(ok, 2, 256, 60, ok, ok, z) == _lib.HMM_ERR_BAD_SHAPE
    assert lib.hmm_quant_cols_group(ok, 2, 256, 64, z, ok, z) == _lib.HMM_ERR_NULL_POINTER
