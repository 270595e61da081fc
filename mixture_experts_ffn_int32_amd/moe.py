"""Python binding of libhmm: ``hyper_mega_moe`` and its autograd Function.

Argument marshalling only.  Every step of the path (routing, the grouped
products, SwiGLU and its gradient, the combines) runs in the HIP kernels behind
the C ABI of include/hmm.h; torch supplies device memory and the current HIP
stream.  (HyperMegaMoE RFC section 3.1: the public call takes exactly x,
topk_ids, topk_weights, up_proj_weight and down_proj_weight and returns y;
section 3.2: the backward returns one gradient per public argument, None for
topk_ids; section 3.3: offsets, tiling and buffers are internal.)  The
optional shared expert (section 6.1) is a keyword-only pair of weights.
"""

import ctypes

import torch

from . import _lib


def _problem(T, H, I, E, K, flags=_lib.HMM_FLAG_VALIDATE_IDS, out_dtype=_lib.HMM_BF16, gmm1_dtype=_lib.HMM_BF16,
             shared_I=0):
    return _lib.Problem(int(T), int(H), int(I), int(E), int(K), out_dtype, gmm1_dtype, flags, int(shared_I))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if (t is not None and t.numel() > 0) else 0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_inputs(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight):
    """Shape/dtype/device checks of the public arguments (RFC section 4.2)."""
    for name, t in (("x", x), ("topk_ids", topk_ids), ("topk_weights", topk_weights),
                    ("up_proj_weight", up_proj_weight), ("down_proj_weight", down_proj_weight)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be on a HIP device (got %s)" % (name, t.device))
        if t.device != x.device:
            raise ValueError("%s is on %s, x on %s" % (name, t.device, x.device))
    if x.dtype != torch.bfloat16 or up_proj_weight.dtype != torch.bfloat16 or down_proj_weight.dtype != torch.bfloat16:
        raise TypeError("x, up_proj_weight and down_proj_weight must be bfloat16")
    if topk_ids.dtype not in (torch.int32, torch.int64):
        raise TypeError("topk_ids must be int32 or int64")
    if not topk_weights.is_floating_point():
        raise TypeError("topk_weights must be floating point")
    if x.dim() != 2 or topk_ids.dim() != 2 or up_proj_weight.dim() != 3 or down_proj_weight.dim() != 3:
        raise ValueError("expected x [T,H], topk_ids [T,K], up_proj_weight [E,H,2I], down_proj_weight [E,I,H]")
    T, H = x.shape
    E, H1, I2 = up_proj_weight.shape
    I = I2 // 2
    if topk_weights.shape != topk_ids.shape or topk_ids.shape[0] != T:
        raise ValueError("topk_ids and topk_weights must both be [T, K] with T = x.shape[0]")
    if H1 != H or I2 != 2 * I or tuple(down_proj_weight.shape) != (E, I, H):
        raise ValueError("up_proj_weight must be [E,H,2I] and down_proj_weight [E,I,H] (got %s, %s, H=%d)"
                         % (tuple(up_proj_weight.shape), tuple(down_proj_weight.shape), H))
    return T, H, I, E, topk_ids.shape[1]


def _check_shared(x, shared_up_proj_weight, shared_down_proj_weight):
    """Shared-expert weights: both or neither; bf16 [H,2Is] and [Is,H] on x's device.  Returns Is (0: none)."""
    if shared_up_proj_weight is None and shared_down_proj_weight is None:
        return 0
    if shared_up_proj_weight is None or shared_down_proj_weight is None:
        raise ValueError("shared_up_proj_weight and shared_down_proj_weight go together")
    for name, t in (("shared_up_proj_weight", shared_up_proj_weight),
                    ("shared_down_proj_weight", shared_down_proj_weight)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.device != x.device:
            raise ValueError("%s is on %s, x on %s" % (name, t.device, x.device))
        if t.dtype != torch.bfloat16:
            raise TypeError("%s must be bfloat16" % name)
    H = x.shape[1]
    if shared_up_proj_weight.dim() != 2 or shared_down_proj_weight.dim() != 2:
        raise ValueError("expected shared_up_proj_weight [H,2Is] and shared_down_proj_weight [Is,H]")
    Is = shared_down_proj_weight.shape[0]
    if tuple(shared_up_proj_weight.shape) != (H, 2 * Is) or tuple(shared_down_proj_weight.shape) != (Is, H):
        raise ValueError("shared_up_proj_weight must be [H,2Is] and shared_down_proj_weight [Is,H] (got %s, %s, H=%d)"
                         % (tuple(shared_up_proj_weight.shape), tuple(shared_down_proj_weight.shape), H))
    return Is


GMM1_DTYPES = {"bf16": _lib.HMM_BF16, "fp8": _lib.HMM_FP8_E4M3, "mx": _lib.HMM_MXFP8_E4M3,
               "group": _lib.HMM_FP8_E4M3_GROUP}


def _gmm1_code(gmm1_dtype):
    if gmm1_dtype not in GMM1_DTYPES:
        raise ValueError("gmm1_dtype must be one of %s (got %r)" % (sorted(GMM1_DTYPES), gmm1_dtype))
    return GMM1_DTYPES[gmm1_dtype]


OUT_DTYPES = {"bf16": _lib.HMM_BF16, "f32": _lib.HMM_F32}


def _out_code(out_dtype):
    """'bf16' / torch.bfloat16 (default) or 'f32' / torch.float32 (the accuracy mode)."""
    if out_dtype in (torch.bfloat16, "bf16"):
        return _lib.HMM_BF16
    if out_dtype in (torch.float32, "f32"):
        return _lib.HMM_F32
    raise ValueError("out_dtype must be torch.bfloat16 or torch.float32 (got %r)" % (out_dtype,))


def _contig(t, dtype=None):
    if dtype is not None and t.dtype != dtype:
        t = t.to(dtype)
    return t.contiguous()


def _forward_raw(x, ids, w, W1, W2, T, H, I, E, K, flags, gmm1=_lib.HMM_BF16, out=_lib.HMM_BF16, Ws1=None, Ws2=None):
    lib = _lib.load()
    Is = 0 if Ws2 is None else Ws2.shape[0]
    prob = _problem(T, H, I, E, K, flags, out_dtype=out, gmm1_dtype=gmm1, shared_I=Is)
    ws, sv = ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(lib.hmm_forward_sizes(ctypes.byref(prob), ctypes.byref(ws), ctypes.byref(sv)))
    dev = x.device
    odt = torch.float32 if out == _lib.HMM_F32 else torch.bfloat16
    y = torch.empty((T, H), dtype=odt, device=dev)
    saved = torch.empty(sv.value, dtype=torch.uint8, device=dev)
    work = torch.empty(ws.value, dtype=torch.uint8, device=dev)
    if Is:
        _lib.check(lib.hmm_forward_shared(ctypes.byref(prob), _ptr(x), _ptr(ids), _ptr(w), _ptr(W1), _ptr(W2),
                                          _ptr(Ws1), _ptr(Ws2), _ptr(y), _ptr(saved), sv.value, _ptr(work), ws.value,
                                          _stream(dev)))
    else:
        _lib.check(lib.hmm_forward(ctypes.byref(prob), _ptr(x), _ptr(ids), _ptr(w), _ptr(W1), _ptr(W2), _ptr(y),
                                   _ptr(saved), sv.value, _ptr(work), ws.value, _stream(dev)))
    return y, saved


def _backward_raw(dy, x, ids, w, W1, W2, saved, T, H, I, E, K, flags, gmm1=_lib.HMM_BF16, out=_lib.HMM_BF16,
                  Ws1=None, Ws2=None):
    """(dx, dW1, dW2, d_topk_weights), and (dWs1, dWs2) after them with a shared expert."""
    lib = _lib.load()
    Is = 0 if Ws2 is None else Ws2.shape[0]
    prob = _problem(T, H, I, E, K, flags, out_dtype=out, gmm1_dtype=gmm1, shared_I=Is)
    ws = ctypes.c_size_t()
    _lib.check(lib.hmm_backward_sizes(ctypes.byref(prob), ctypes.byref(ws)))
    dev = x.device
    odt = torch.float32 if out == _lib.HMM_F32 else torch.bfloat16
    dx = torch.empty((T, H), dtype=odt, device=dev)
    dW1 = torch.empty((E, H, 2 * I), dtype=odt, device=dev)
    dW2 = torch.empty((E, I, H), dtype=odt, device=dev)
    dw = torch.empty((T, K), dtype=torch.float32, device=dev)
    work = torch.empty(ws.value, dtype=torch.uint8, device=dev)
    if Is:
        dWs1 = torch.empty((H, 2 * Is), dtype=odt, device=dev)
        dWs2 = torch.empty((Is, H), dtype=odt, device=dev)
        _lib.check(lib.hmm_backward_shared(ctypes.byref(prob), _ptr(dy), _ptr(x), _ptr(ids), _ptr(w), _ptr(W1),
                                           _ptr(W2), _ptr(Ws1), _ptr(Ws2), _ptr(saved), saved.numel(), _ptr(dx),
                                           _ptr(dW1), _ptr(dW2), _ptr(dWs1), _ptr(dWs2), _ptr(dw), _ptr(work),
                                           ws.value, _stream(dev)))
        return dx, dW1, dW2, dw, dWs1, dWs2
    _lib.check(lib.hmm_backward(ctypes.byref(prob), _ptr(dy), _ptr(x), _ptr(ids), _ptr(w), _ptr(W1), _ptr(W2),
                                _ptr(saved), saved.numel(), _ptr(dx), _ptr(dW1), _ptr(dW2), _ptr(dw),
                                _ptr(work), ws.value, _stream(dev)))
    return dx, dW1, dW2, dw


class HyperMegaMoEFunction(torch.autograd.Function):
    """Forward calls hmm_forward and keeps the saved buffer; backward calls hmm_backward."""

    @staticmethod
    def forward(ctx, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, flags, gmm1, out,
                shared_up_proj_weight=None, shared_down_proj_weight=None):
        T, H, I, E, K = _check_inputs(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight)
        Is = _check_shared(x, shared_up_proj_weight, shared_down_proj_weight)
        x_ = _contig(x)
        ids = _contig(topk_ids, torch.int32)
        w = _contig(topk_weights, torch.float32)
        W1 = _contig(up_proj_weight)
        W2 = _contig(down_proj_weight)
        Ws1 = _contig(shared_up_proj_weight) if Is else None
        Ws2 = _contig(shared_down_proj_weight) if Is else None
        with torch.cuda.device(x.device):
            y, saved = _forward_raw(x_, ids, w, W1, W2, T, H, I, E, K, flags, gmm1, out, Ws1, Ws2)
        ctx.save_for_backward(x_, ids, w, W1, W2, saved, Ws1, Ws2)
        ctx.dims = (T, H, I, E, K, flags, gmm1, out)
        ctx.w_dtype = topk_weights.dtype
        return y

    @staticmethod
    def backward(ctx, dy):
        x_, ids, w, W1, W2, saved, Ws1, Ws2 = ctx.saved_tensors
        T, H, I, E, K, flags, gmm1, out = ctx.dims
        dy = _contig(dy, torch.float32 if out == _lib.HMM_F32 else torch.bfloat16)
        with torch.cuda.device(x_.device):
            g = _backward_raw(dy, x_, ids, w, W1, W2, saved, T, H, I, E, K, flags, gmm1, out, Ws1, Ws2)
        dx, dW1, dW2, dw = g[:4]
        dWs1, dWs2 = g[4:] if Ws1 is not None else (None, None)
        return dx, None, dw.to(ctx.w_dtype), dW1, dW2, None, None, None, dWs1, dWs2


def hyper_mega_moe(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, *, validate_ids=True,
                   gmm1_dtype="bf16", out_dtype=torch.bfloat16, shared_up_proj_weight=None,
                   shared_down_proj_weight=None, fp8_backward=False):
    """y [T,H] = sum_k topk_weights[t,k] * SwiGLU-FFN_{topk_ids[t,k]}(x[t]), on the GPU.

    x bf16 [T,H]; topk_ids int32/int64 [T,K] (0 <= id < E); topk_weights float [T,K];
    up_proj_weight bf16 [E,H,2I] (gate columns first, then up); down_proj_weight
    bf16 [E,I,H].  Differentiable in x, topk_weights and both weights.
    ``validate_ids`` checks the ids on the device before the matrix products
    (one small device-to-host read-back) and raises ValueError if one is out
    of range.  ``gmm1_dtype="fp8"`` runs the up-projection in FP8 E4M3: each
    token row and each (expert, column) of up_proj_weight is quantised with a
    dynamic per-row / per-column scale (H must then be a multiple of 128); the
    rest of the forward and the whole backward stay bf16.  ``gmm1_dtype="mx"``
    uses MX quantisation instead (one power-of-two scale per 32 elements along
    H, for tokens and for each weight column); ``gmm1_dtype="group"`` uses
    per-group quantisation (one float scale per 128 elements along H for tokens,
    per 128-row block for each weight column; its up-projection runs on
    64-row tiles).  ``out_dtype=torch.float32``
    is the accuracy mode: y (and dx and the weight gradients of the raw backward)
    are float32 and every intermediate is kept to about 16 significant bits
    (bf16 hi + lo pairs), for agreement with an unrounded computation to 1e-3;
    it costs about twice the MFMA work.  Under autograd, gradients are cast to
    the dtype of their inputs (bf16 weights get bf16 gradients).
    ``shared_up_proj_weight`` bf16 [H,2Is] and ``shared_down_proj_weight`` bf16
    [Is,H] add a shared expert: every token also goes through that SwiGLU FFN,
    and its output is added to y with weight 1 (after the routed terms); both
    get gradients.  Its up-projection stays bf16 under ``gmm1_dtype="fp8"``.
    ``fp8_backward=True`` runs the backward's act_grad and input_grad products on
    FP8 E4M3 (per-row dynamic scales of dY, dH and the weight rows; H a multiple
    of 128, bf16 outputs); the weight gradients stay bf16.
    """
    flags = (_lib.HMM_FLAG_VALIDATE_IDS if validate_ids else 0) | (_lib.HMM_FLAG_FP8_BACKWARD if fp8_backward else 0)
    return HyperMegaMoEFunction.apply(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, flags,
                                      _gmm1_code(gmm1_dtype), _out_code(out_dtype), shared_up_proj_weight,
                                      shared_down_proj_weight)


# ----------------------------------------------------------------------------- stage entry points (tests, tools)

def route(topk_ids, E, validate_ids=True):
    """Routing alone: dict(counts[E], offsets[E+1], sorted_slot[S], row_of_slot[S]) int32 tensors."""
    if topk_ids.device.type != "cuda":
        raise ValueError("topk_ids must be on a HIP device")
    ids = _contig(topk_ids, torch.int32)
    T, K = ids.shape
    lib = _lib.load()
    prob = _problem(T, 64, 64, E, K, _lib.HMM_FLAG_VALIDATE_IDS if validate_ids else 0)
    ws = ctypes.c_size_t()
    _lib.check(lib.hmm_route_workspace_size(ctypes.byref(prob), ctypes.byref(ws)))
    dev = ids.device
    out = {
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "sorted_slot": torch.empty(T * K, dtype=torch.int32, device=dev),
        "row_of_slot": torch.empty(T * K, dtype=torch.int32, device=dev),
    }
    work = torch.empty(ws.value, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _lib.check(lib.hmm_route(ctypes.byref(prob), _ptr(ids), _ptr(out["counts"]), _ptr(out["offsets"]),
                                 _ptr(out["sorted_slot"]), _ptr(out["row_of_slot"]), _ptr(work), ws.value,
                                 _stream(dev)))
    return out


def quantize_rows_fp8(x):
    """Per-token FP8 E4M3 quantisation of x bf16 [T,H]: (codes uint8 [T,H], descale float32 [T])."""
    if x.device.type != "cuda" or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a bf16 [T,H] tensor on a HIP device")
    x = _contig(x)
    T, H = x.shape
    q = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    ds = torch.empty(T, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _lib.check(_lib.load().hmm_quant_rows_fp8(_ptr(x), T, H, _ptr(q), _ptr(ds), _stream(x.device)))
    return q, ds


def quantize_cols_fp8(w):
    """Per-(expert, column) FP8 E4M3 quantisation of w bf16 [E,H,N]: (codes uint8 [E,H,N], descale float32 [E,N])."""
    if w.device.type != "cuda" or w.dtype != torch.bfloat16 or w.dim() != 3:
        raise ValueError("w must be a bf16 [E,H,N] tensor on a HIP device")
    w = _contig(w)
    E, H, N = w.shape
    lib = _lib.load()
    ws = ctypes.c_size_t()
    _lib.check(lib.hmm_quant_cols_workspace_size(E, H, N, ctypes.byref(ws)))
    q = torch.empty((E, H, N), dtype=torch.uint8, device=w.device)
    ds = torch.empty((E, N), dtype=torch.float32, device=w.device)
    work = torch.empty(ws.value, dtype=torch.uint8, device=w.device)
    with torch.cuda.device(w.device):
        _lib.check(lib.hmm_quant_cols_fp8(_ptr(w), E, H, N, _ptr(q), _ptr(ds), _ptr(work), ws.value,
                                          _stream(w.device)))
    return q, ds


def quantize_rows_mx(x):
    """MX quantisation of x bf16 [T,H] (blocks of 32): (codes uint8 [T,H], E8M0 exponents uint8 [T,H/32])."""
    if x.device.type != "cuda" or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a bf16 [T,H] tensor on a HIP device")
    x = _contig(x)
    T, H = x.shape
    q = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    s = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _lib.check(_lib.load().hmm_quant_rows_mx(_ptr(x), T, H, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def quantize_cols_mx(w):
    """MX quantisation of w bf16 [E,H,N] in blocks of 32 rows per column:
    (codes uint8 [E,H,N], E8M0 exponents uint8 [E,N,H/32])."""
    if w.device.type != "cuda" or w.dtype != torch.bfloat16 or w.dim() != 3:
        raise ValueError("w must be a bf16 [E,H,N] tensor on a HIP device")
    w = _contig(w)
    E, H, N = w.shape
    q = torch.empty((E, H, N), dtype=torch.uint8, device=w.device)
    s = torch.empty((E, N, H // 32), dtype=torch.uint8, device=w.device)
    with torch.cuda.device(w.device):
        _lib.check(_lib.load().hmm_quant_cols_mx(_ptr(w), E, H, N, _ptr(q), _ptr(s), _stream(w.device)))
    return q, s


def quantize_rows_group(x):
    """Per-group quantisation of x bf16 [T,H] (groups of 128 along H):
    (codes uint8 [T,H], float32 descales [T,H/128])."""
    if x.device.type != "cuda" or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a bf16 [T,H] tensor on a HIP device")
    x = _contig(x)
    T, H = x.shape
    q = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    d = torch.empty((T, H // 128), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _lib.check(_lib.load().hmm_quant_rows_group(_ptr(x), T, H, _ptr(q), _ptr(d), _stream(x.device)))
    return q, d


def quantize_cols_group(w):
    """Per-group quantisation of w bf16 [E,H,N] in blocks of 128 rows per column:
    (codes uint8 [E,H,N], float32 descales [E,H/128,N])."""
    if w.device.type != "cuda" or w.dtype != torch.bfloat16 or w.dim() != 3:
        raise ValueError("w must be a bf16 [E,H,N] tensor on a HIP device")
    w = _contig(w)
    E, H, N = w.shape
    q = torch.empty((E, H, N), dtype=torch.uint8, device=w.device)
    d = torch.empty((E, H // 128, N), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        _lib.check(_lib.load().hmm_quant_cols_group(_ptr(w), E, H, N, _ptr(q), _ptr(d), _stream(w.device)))
    return q, d


def saved_views(saved, T, H, I, E, K, tiles="auto", out_dtype="bf16", shared_I=0, gmm1_dtype="bf16"):
    """Typed views of the arrays a forward recorded in its saved buffer.

    In the float32-output mode h is float32 [S, 2I] and a, aw are bf16 [S, 2I]
    pairs (hi in the first I columns, lo in the last I).  With a shared expert
    (shared_I = Is > 0) also shared_h [T, 2Is] and shared_a [T, Is] (same rules).
    gmm1_dtype is the forward's: the per-group mode always runs on narrow tiles, whose
    tables have another size."""
    lib = _lib.load()
    out = _out_code(out_dtype)
    prob = _problem(T, H, I, E, K, _lib.TILE_FLAGS[tiles], out_dtype=out, shared_I=shared_I,
                    gmm1_dtype=GMM1_DTYPES[gmm1_dtype])
    L = _lib.SavedLayout()
    _lib.check(lib.hmm_saved_layout_of(ctypes.byref(prob), ctypes.byref(L)))
    S = T * K
    f32 = out == _lib.HMM_F32

    def view(off, n, dtype, shape):
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return saved[off:off + nbytes].view(dtype).view(shape)

    views = {
        "counts": view(L.counts, E, torch.int32, (E,)),
        "offsets": view(L.offsets, E + 1, torch.int32, (E + 1,)),
        "sorted_slot": view(L.sorted_slot, S, torch.int32, (S,)),
        "row_of_slot": view(L.row_of_slot, S, torch.int32, (S,)),
        "tok_of_row": view(L.tok_of_row, S, torch.int32, (S,)),
        "h": view(L.h, S * 2 * I, torch.float32 if f32 else torch.bfloat16, (S, 2 * I)),
        "a": view(L.a, S * I * (2 if f32 else 1), torch.bfloat16, (S, 2 * I if f32 else I)),
        "aw": view(L.aw, S * I * (2 if f32 else 1), torch.bfloat16, (S, 2 * I if f32 else I)),
        "id_error": view(L.id_error, 1, torch.int32, (1,)),
    }
    if shared_I:
        Is = shared_I
        views.update({
            "shared_offsets": view(L.shared_offsets, 2, torch.int32, (2,)),
            "shared_idx": view(L.shared_idx, T, torch.int32, (T,)),
            "shared_ones": view(L.shared_ones, T, torch.float32, (T,)),
            "shared_h": view(L.shared_h, T * 2 * Is, torch.float32 if f32 else torch.bfloat16, (T, 2 * Is)),
            "shared_a": view(L.shared_a, T * Is * (2 if f32 else 1), torch.bfloat16, (T, 2 * Is if f32 else Is)),
        })
    return views


def forward_with_saved(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, validate_ids=True,
                       tiles="auto", gmm1_dtype="bf16", out_dtype="bf16", fused=False, shared_up_proj_weight=None,
                       shared_down_proj_weight=None):
    """Forward without autograd; returns (y, saved buffer) for stage-level checks.

    ``tiles`` forces the tiling of the grouped products ("auto", "large" or
    "narrow"); the matching backward_from_saved call must use the same value.
    ``fused=True`` runs a small problem's forward as one persistent launch
    (same results; slower on MI355X today, see include/hmm.h).
    """
    T, H, I, E, K = _check_inputs(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight)
    Is = _check_shared(x, shared_up_proj_weight, shared_down_proj_weight)
    flags = (_lib.HMM_FLAG_VALIDATE_IDS if validate_ids else 0) | _lib.TILE_FLAGS[tiles]
    if fused:
        flags |= _lib.HMM_FLAG_FUSED_FORWARD
    with torch.cuda.device(x.device):
        return _forward_raw(_contig(x), _contig(topk_ids, torch.int32), _contig(topk_weights, torch.float32),
                            _contig(up_proj_weight), _contig(down_proj_weight), T, H, I, E, K, flags,
                            _gmm1_code(gmm1_dtype), _out_code(out_dtype),
                            _contig(shared_up_proj_weight) if Is else None,
                            _contig(shared_down_proj_weight) if Is else None)


def backward_from_saved(dy, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, saved, tiles="auto",
                        gmm1_dtype="bf16", out_dtype="bf16", shared_up_proj_weight=None,
                        shared_down_proj_weight=None, serial=False, fp8_backward=False):
    """Backward without autograd; returns (dx, d_up_proj_weight, d_down_proj_weight, d_topk_weights),
    then (d_shared_up_proj_weight, d_shared_down_proj_weight) with a shared expert.

    With out_dtype float32, dy is taken in float32 and dx and the weight gradients are float32.
    ``serial=True`` keeps every launch on the current stream (HMM_FLAG_SERIAL_BACKWARD);
    ``fp8_backward=True`` runs act_grad and input_grad on E4M3 (HMM_FLAG_FP8_BACKWARD)."""
    T, H, I, E, K = _check_inputs(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight)
    Is = _check_shared(x, shared_up_proj_weight, shared_down_proj_weight)
    out = _out_code(out_dtype)
    dyt = torch.float32 if out == _lib.HMM_F32 else torch.bfloat16
    with torch.cuda.device(x.device):
        return _backward_raw(_contig(dy, dyt), _contig(x), _contig(topk_ids, torch.int32),
                             _contig(topk_weights, torch.float32), _contig(up_proj_weight),
                             _contig(down_proj_weight), saved, T, H, I, E, K,
                             _lib.TILE_FLAGS[tiles] | (_lib.HMM_FLAG_SERIAL_BACKWARD if serial else 0)
                             | (_lib.HMM_FLAG_FP8_BACKWARD if fp8_backward else 0),
                             _gmm1_code(gmm1_dtype), out, _contig(shared_up_proj_weight) if Is else None,
                             _contig(shared_down_proj_weight) if Is else None)
