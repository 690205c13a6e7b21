"""RIB window attention with the CLA gate on MI355X (gfx950).

A thin ctypes binding over ``librib.so`` (the hand-written HIP kernels behind
the C ABI in ``include/rib.h``).  The binding only marshals arguments: it
checks devices, dtypes, shapes and contiguity, allocates outputs with torch and
passes raw device pointers plus torch's current HIP stream.  Every step of the
computation runs in the library's kernels; there is no fallback path, and the
calls raise if the library is missing.

    qp, kp = encode(window, L, hidden, R, weights)          # once per window size
    o = window_attn(qc, kc, v, g, qp, kp, heads, window)    # per layer call
    o, lse = window_attn_train(qc, kc, v, g, qp, kp, heads, window)   # training forward
    grads = window_attn_backward(qc, kc, v, g, qp, kp, o, lse, dout, heads, window)
    dweights = encode_backward(window, L, hidden, R, weights, grads[4], grads[5])

Method: "Rank-Factorized Implicit Neural Bias: Scaling Super-Resolution
Transformer with FlashAttention" (gist.science summaries, part A/B;
omica.com.cn explainer, sections 2.2, 2.3 and 5.2).
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librib.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "rib.h")

RIB_OK, RIB_ERR_INVALID_ARG, RIB_ERR_UNSUPPORTED, RIB_ERR_HIP = 0, 1, 2, 3
RIB_F32, RIB_BF16 = 0, 1

_lib = None


class RibError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"rib status {status}: {message}")
        self.status = status


class AttnCall(ctypes.Structure):
    """rib_attn_call: one call of rib_window_attn_multi."""
    _fields_ = [("qc", ctypes.c_void_p), ("kc", ctypes.c_void_p), ("v", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("qp", ctypes.c_void_p), ("kp", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("W", ctypes.c_int), ("heads", ctypes.c_int),
                ("dh", ctypes.c_int), ("R", ctypes.c_int), ("window", ctypes.c_int)]


def lib(path: str | None = None):
    """Load librib.so (built in-tree by ``build.py``); raise if it is not there."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build the HIP library first "
                           "(python super_resolution_transformer_amd/build.py)")
    L = ctypes.CDLL(p)
    vp, i = ctypes.c_void_p, ctypes.c_int
    L.rib_encode.argtypes = [i, i, i, i, vp, vp, vp, vp]
    L.rib_encode.restype = i
    L.rib_window_attn.argtypes = [vp] * 7 + [i] * 8 + [vp]
    L.rib_window_attn.restype = i
    L.rib_window_attn_heads.argtypes = [vp] * 7 + [i] * 8 + [vp]
    L.rib_window_attn_heads.restype = i
    L.rib_cla_gate.argtypes = [vp] * 6 + [i] * 5 + [vp]
    L.rib_cla_gate.restype = i
    sz = ctypes.c_size_t
    L.rib_window_attn_backward_workspace.argtypes = [i] * 8
    L.rib_window_attn_backward_workspace.restype = sz
    L.rib_window_attn_train.argtypes = [vp] * 8 + [i] * 8 + [vp]
    L.rib_window_attn_train.restype = i
    L.rib_window_attn_backward.argtypes = [vp] * 16 + [sz] + [i] * 8 + [vp]
    L.rib_window_attn_backward.restype = i
    L.rib_window_attn_heads_backward.argtypes = [vp] * 16 + [sz] + [i] * 8 + [vp]
    L.rib_window_attn_heads_backward.restype = i
    L.rib_window_attn_heads_train.argtypes = [vp] * 8 + [i] * 8 + [vp]
    L.rib_window_attn_heads_train.restype = i
    L.rib_encode_backward_workspace.argtypes = [i] * 4
    L.rib_encode_backward_workspace.restype = sz
    L.rib_encode_backward.argtypes = [i] * 4 + [vp] * 5 + [sz, vp]
    L.rib_encode_backward.restype = i
    L.rib_encode_backward_noalloc.argtypes = [i] * 4 + [vp] * 5
    L.rib_encode_backward_noalloc.restype = i
    L.rib_ln_qkv.argtypes = [vp] * 9 + [i] * 4 + [ctypes.c_float, i, vp]
    L.rib_ln_qkv.restype = i
    L.rib_window_attn_lnq.argtypes = [vp] * 11 + [i] * 7 + [ctypes.c_float, i, vp]
    L.rib_window_attn_lnq.restype = i
    L.rib_encode3d.argtypes = [i] * 5 + [vp] * 4
    L.rib_encode3d.restype = i
    L.rib_window_attn3d.argtypes = [vp] * 7 + [i] * 10 + [vp]
    L.rib_window_attn3d.restype = i
    L.rib_window_attn_multi.argtypes = [i, ctypes.POINTER(AttnCall), i, vp]
    L.rib_window_attn_multi.restype = i
    L.rib_attn_supported.argtypes = [i, i, i, i]
    L.rib_attn_supported.restype = i
    L.rib_last_error.argtypes = []
    L.rib_last_error.restype = ctypes.c_char_p
    L.rib_abi_version.argtypes = []
    L.rib_abi_version.restype = i
    if path is None:
        _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/rib.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rib_\w+)\s*\(", text, flags=re.M)


def _check(status: int) -> None:
    if status != RIB_OK:
        raise RibError(status, lib().rib_last_error().decode())


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def weight_count(L: int, hidden: int, R: int) -> int:
    """Length of the packed weight vector W_h | b_h | Wp_q | Wp_k."""
    return (2 + 4 * L) * hidden + hidden + 2 * hidden * R


def encode(window: int, L: int, hidden: int, R: int, weights):
    """Positional factors (Qp, Kp), each float32 [window*window, R], on the weights' device."""
    import torch
    if not (weights.is_cuda and weights.dtype == torch.float32 and weights.is_contiguous()):
        raise ValueError("weights must be a contiguous float32 GPU tensor")
    if weights.numel() != weight_count(L, hidden, R):
        raise ValueError("packed weight vector has the wrong length")
    qp = torch.empty((window * window, R), dtype=torch.float32, device=weights.device)
    kp = torch.empty_like(qp)
    encode_into(window, L, hidden, R, weights, qp, kp)
    return qp, kp


def encode_into(window, L, hidden, R, weights, qp, kp) -> None:
    _check(lib().rib_encode(window, L, hidden, R, _ptr(weights), _ptr(qp), _ptr(kp), _stream(weights)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return RIB_F32
    if t.dtype == torch.bfloat16:
        return RIB_BF16
    raise ValueError("feature maps must be float32 or bfloat16")


def window_attn(qc, kc, v, g, qp, kp, heads: int, window: int):
    """O = (softmax([Qc/sqrt(dh), Qp/sqrt(R)] [Kc, Kp]^T) V) * sigmoid(G) per window and head.

    qc, kc, v, g: [B, H, W, heads*dh] contiguous GPU tensors (float32 or bfloat16);
    qp, kp: float32 [window*window, R] from ``encode``.  Returns O like qc.
    """
    import torch
    o = torch.empty_like(qc)
    window_attn_into(qc, kc, v, g, qp, kp, heads, window, o)
    return o


def window_attn_into(qc, kc, v, g, qp, kp, heads: int, window: int, o) -> None:
    import torch
    ts = (qc, kc, v, g, o)
    if any(t.dim() != 4 for t in ts) or any(t.shape != qc.shape for t in ts):
        raise ValueError("qc, kc, v, g, o must all be [B, H, W, C]")
    if any(t.dtype != qc.dtype for t in ts):
        raise ValueError("qc, kc, v, g, o must share one dtype")
    if not all(t.is_cuda and t.is_contiguous() for t in ts + (qp, kp)):
        raise ValueError("all tensors must be contiguous GPU tensors")
    if qp.dtype != torch.float32 or kp.dtype != torch.float32 or qp.shape != kp.shape or qp.dim() not in (2, 3):
        raise ValueError("qp, kp must be float32 [window*window, R] or per-head [heads, window*window, R]")
    per_head = qp.dim() == 3
    if qp.shape[-2] != window * window or (per_head and qp.shape[0] != heads):
        raise ValueError("qp, kp must have window*window rows (and one table per head)")
    B, H, W, C = qc.shape
    if heads < 1 or C % heads:
        raise ValueError("channel count must be a multiple of heads")
    dh, R = C // heads, qp.shape[-1]
    fn = lib().rib_window_attn_heads if per_head else lib().rib_window_attn
    _check(fn(_ptr(qc), _ptr(kc), _ptr(v), _ptr(g), _ptr(qp), _ptr(kp), _ptr(o),
              B, H, W, heads, dh, R, window, _dtype_code(qc), _stream(qc)))


def window_attn_multi(calls):
    """Several independent window_attn calls in as few launches as possible.

    calls: list of (qc, kc, v, g, qp, kp, heads, window), all of one dtype; window sizes and
    shapes may differ.  Returns the list of outputs, each equal to window_attn's."""
    import torch
    outs = [torch.empty_like(c[0]) for c in calls]
    window_attn_multi_into(calls, outs)
    return outs


def window_attn_multi_into(calls, outs) -> None:
    import torch
    if len(calls) != len(outs) or not calls:
        raise ValueError("need one output per call and at least one call")
    arr = (AttnCall * len(calls))()
    dtype = calls[0][0].dtype
    for k, ((qc, kc, v, g, qp, kp, heads, window), o) in enumerate(zip(calls, outs)):
        ts = (qc, kc, v, g, o)
        if any(t.dim() != 4 or t.shape != qc.shape or t.dtype != dtype for t in ts):
            raise ValueError("each call's qc, kc, v, g, o must be [B, H, W, C] of the batch's dtype")
        if not all(t.is_cuda and t.is_contiguous() for t in ts + (qp, kp)):
            raise ValueError("all tensors must be contiguous GPU tensors")
        if qp.dtype != torch.float32 or kp.dtype != torch.float32 or qp.shape != kp.shape or qp.dim() != 2:
            raise ValueError("qp, kp must be float32 [window*window, R]")
        if qp.shape[0] != window * window:
            raise ValueError("qp, kp must have window*window rows")
        B, H, W, C = qc.shape
        if heads < 1 or C % heads:
            raise ValueError("channel count must be a multiple of heads")
        arr[k] = AttnCall(_ptr(qc), _ptr(kc), _ptr(v), _ptr(g), _ptr(qp), _ptr(kp), _ptr(o),
                          B, H, W, heads, C // heads, qp.shape[1], window)
    _check(lib().rib_window_attn_multi(len(calls), arr, _dtype_code(calls[0][0]), _stream(calls[0][0])))


def window_attn_train(qc, kc, v, g, qp, kp, heads: int, window: int):
    """window_attn plus the row log-sum-exp the backward needs: returns (o, lse), lse float32
    [B, H, W, heads] (natural log)."""
    import torch
    B, H, W, C = qc.shape
    o = torch.empty_like(qc)
    lse = torch.empty((B, H, W, max(heads, 1)), dtype=torch.float32, device=qc.device)
    window_attn_train_into(qc, kc, v, g, qp, kp, heads, window, o, lse)
    return o, lse


def window_attn_train_into(qc, kc, v, g, qp, kp, heads: int, window: int, o, lse) -> None:
    import torch
    ts = (qc, kc, v, g, o)
    if any(t.dim() != 4 or t.shape != qc.shape or t.dtype != qc.dtype for t in ts):
        raise ValueError("qc, kc, v, g, o must all be [B, H, W, C] of one dtype")
    if not all(t.is_cuda and t.is_contiguous() for t in ts + (qp, kp, lse)):
        raise ValueError("all tensors must be contiguous GPU tensors")
    if qp.dtype != torch.float32 or kp.dtype != torch.float32 or qp.shape != kp.shape or qp.dim() not in (2, 3):
        raise ValueError("qp, kp must be float32 [window*window, R] or per-head [heads, window*window, R]")
    per_head = qp.dim() == 3
    if qp.shape[-2] != window * window or (per_head and qp.shape[0] != heads):
        raise ValueError("qp, kp must have window*window rows (and one table per head)")
    B, H, W, C = qc.shape
    if heads < 1 or C % heads:
        raise ValueError("channel count must be a multiple of heads")
    if lse.shape != (B, H, W, heads) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, W, heads]")
    fn = lib().rib_window_attn_heads_train if per_head else lib().rib_window_attn_train
    _check(fn(_ptr(qc), _ptr(kc), _ptr(v), _ptr(g), _ptr(qp), _ptr(kp), _ptr(o), _ptr(lse),
              B, H, W, heads, C // heads, qp.shape[-1], window, _dtype_code(qc), _stream(qc)))


def cla_gate(x, dw_w, dw_b, pw_w, pw_b):
    """G = PWConv1x1(DWConv3x3(X)) (the CLA gating map) for an NHWC map x; returns a new tensor."""
    import torch
    g = torch.empty_like(x)
    cla_gate_into(x, dw_w, dw_b, pw_w, pw_b, g)
    return g


def cla_gate_into(x, dw_w, dw_b, pw_w, pw_b, g) -> None:
    import torch
    if x.dim() != 4 or g.shape != x.shape or g.dtype != x.dtype:
        raise ValueError("x and g must be [B, H, W, C] of one dtype")
    B, H, W, C = x.shape
    ws = (dw_w, dw_b, pw_w, pw_b)
    if any(t.dtype != torch.float32 for t in ws):
        raise ValueError("gate weights must be float32")
    if dw_w.shape != (C, 3, 3) or dw_b.shape != (C,) or pw_w.shape != (C, C) or pw_b.shape != (C,):
        raise ValueError("gate weights must be dw_w [C,3,3], dw_b [C], pw_w [C,C], pw_b [C]")
    if not all(t.is_cuda and t.is_contiguous() for t in ws + (x, g)):
        raise ValueError("all tensors must be contiguous GPU tensors")
    _check(lib().rib_cla_gate(_ptr(x), _ptr(dw_w), _ptr(dw_b), _ptr(pw_w), _ptr(pw_b), _ptr(g), B, H, W, C,
                              _dtype_code(x), _stream(x)))


def window_attn_backward(qc, kc, v, g, qp, kp, o, lse, dout, heads: int, window: int):
    """Gradients (dqc, dkc, dv, dg, dqp, dkp) of window_attn for the upstream gradient dout.

    (o, lse) come from window_attn_train on the same inputs.  With one shared pair qp, kp
    [window*window, R], dqp and dkp have that shape and sum over every image, window and
    head; with one pair per head [heads, window*window, R], dqp[h], dkp[h] sum over head h's
    images and windows.  The workspace is a temporary torch buffer.
    """
    import torch
    outs = [torch.empty_like(qc) for _ in range(4)]
    dqp, dkp = torch.empty_like(qp), torch.empty_like(kp)
    work = torch.empty(max(backward_workspace_bytes(qc, qp, heads, window), 16), dtype=torch.uint8,
                       device=qc.device)
    window_attn_backward_into(qc, kc, v, g, qp, kp, o, lse, dout, heads, window, *outs, dqp, dkp, work)
    return (*outs, dqp, dkp)


def backward_workspace_bytes(qc, qp, heads: int, window: int) -> int:
    """Bytes of device workspace window_attn_backward_into needs for maps like qc."""
    B, H, W, C = qc.shape
    return lib().rib_window_attn_backward_workspace(B, H, W, heads, C // heads, qp.shape[-1], window,
                                                    _dtype_code(qc))


def window_attn_backward_into(qc, kc, v, g, qp, kp, o, lse, dout, heads: int, window: int,
                              dqc, dkc, dv, dg, dqp, dkp, work) -> None:
    """window_attn_backward into caller buffers; work is a uint8 device buffer of at least
    backward_workspace_bytes() bytes."""
    import torch
    ts = (qc, kc, v, g, o, dout, dqc, dkc, dv, dg)
    if any(t.dim() != 4 or t.shape != qc.shape or t.dtype != qc.dtype for t in ts):
        raise ValueError("qc, kc, v, g, o, dout and the map gradients must all be [B, H, W, C] of one dtype")
    if not all(t.is_cuda and t.is_contiguous() for t in ts + (qp, kp, dqp, dkp, work)):
        raise ValueError("all tensors must be contiguous GPU tensors")
    if qp.dtype != torch.float32 or kp.dtype != torch.float32 or qp.shape != kp.shape or qp.dim() not in (2, 3):
        raise ValueError("qp, kp must be float32 [window*window, R] or per-head [heads, window*window, R]")
    per_head = qp.dim() == 3
    if qp.shape[-2] != window * window or dqp.shape != qp.shape or dkp.shape != qp.shape:
        raise ValueError("qp, kp, dqp, dkp must have window*window rows of R, and one shape")
    B, H, W, C = qc.shape
    if heads < 1 or C % heads or (per_head and qp.shape[0] != heads):
        raise ValueError("channel count must be a multiple of heads (and per-head tables one per head)")
    if lse.shape != (B, H, W, heads) or lse.dtype != torch.float32 or not (lse.is_cuda and lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 GPU tensor [B, H, W, heads]")
    dh, R = C // heads, qp.shape[-1]
    code = _dtype_code(qc)
    nbytes = work.numel() * work.element_size()
    fn = lib().rib_window_attn_heads_backward if per_head else lib().rib_window_attn_backward
    _check(fn(*[_ptr(t) for t in ts[:4]], _ptr(qp), _ptr(kp), _ptr(o), _ptr(lse),
              _ptr(dout), _ptr(dqc), _ptr(dkc), _ptr(dv), _ptr(dg), _ptr(dqp),
              _ptr(dkp), _ptr(work), nbytes, B, H, W, heads, dh, R, window, code, _stream(qc)))


def encode_backward(window: int, L: int, hidden: int, R: int, weights, dqp, dkp):
    """Gradient of the packed encoder weights for upstream (dqp, dkp); float32 like weights."""
    import torch
    dw = torch.empty_like(weights)
    work = torch.empty(max(lib().rib_encode_backward_workspace(window, L, hidden, R), 16), dtype=torch.uint8,
                       device=weights.device)
    encode_backward_into(window, L, hidden, R, weights, dqp, dkp, dw, work)
    return dw


def encode_backward_into(window: int, L: int, hidden: int, R: int, weights, dqp, dkp, dw, work) -> None:
    import torch
    ts = (weights, dqp, dkp, dw)
    if not all(t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 for t in ts):
        raise ValueError("weights, dqp, dkp, dw must be contiguous float32 GPU tensors")
    if weights.numel() != weight_count(L, hidden, R) or dw.numel() != weights.numel():
        raise ValueError("packed weight vector has the wrong length")
    if dqp.shape != (window * window, R) or dkp.shape != (window * window, R):
        raise ValueError("dqp, dkp must be [window*window, R]")
    if not (work.is_cuda and work.is_contiguous()):
        raise ValueError("work must be a contiguous GPU buffer")
    _check(lib().rib_encode_backward(window, L, hidden, R, _ptr(weights), _ptr(dqp), _ptr(dkp), _ptr(dw),
                                     _ptr(work), work.numel() * work.element_size(), _stream(weights)))


def encode_backward_noalloc_into(window: int, L: int, hidden: int, R: int, weights, dqp, dkp, dw) -> None:
    """encode_backward_into without a workspace argument: the library's fixed per-device array
    takes the partial gradients (no device allocation; calls that overlap on one device race)."""
    import torch
    ts = (weights, dqp, dkp, dw)
    if not all(t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 for t in ts):
        raise ValueError("weights, dqp, dkp, dw must be contiguous float32 GPU tensors")
    if weights.numel() != weight_count(L, hidden, R) or dw.numel() != weights.numel():
        raise ValueError("packed weight vector has the wrong length")
    if dqp.shape != (window * window, R) or dkp.shape != (window * window, R):
        raise ValueError("dqp, dkp must be [window*window, R]")
    _check(lib().rib_encode_backward_noalloc(window, L, hidden, R, _ptr(weights), _ptr(dqp), _ptr(dkp), _ptr(dw),
                                             _stream(weights)))


def ln_qkv(x, gamma, beta, w, bias, eps: float = 1e-5, with_xn: bool = False):
    """(q, k, v[, xn]) = LayerNorm(x) W + bias split into Q | K | V, for an NHWC map x
    (w float32 [C, 3C], gamma/beta [C], bias [3C])."""
    import torch
    outs = [torch.empty_like(x) for _ in range(4 if with_xn else 3)]
    ln_qkv_into(x, gamma, beta, w, bias, *outs[:3], outs[3] if with_xn else None, eps)
    return tuple(outs)


def ln_qkv_into(x, gamma, beta, w, bias, q, k, v, xn=None, eps: float = 1e-5) -> None:
    import torch
    if x.dim() != 4:
        raise ValueError("x must be [B, H, W, C]")
    B, H, W, C = x.shape
    maps = [t for t in (q, k, v, xn) if t is not None]
    if any(t.shape != x.shape or t.dtype != x.dtype for t in maps):
        raise ValueError("q, k, v (and xn) must match x in shape and dtype")
    ws = (gamma, beta, w, bias)
    if any(t.dtype != torch.float32 for t in ws):
        raise ValueError("gamma, beta, w, bias must be float32")
    if gamma.shape != (C,) or beta.shape != (C,) or w.shape != (C, 3 * C) or bias.shape != (3 * C,):
        raise ValueError("gamma, beta [C], w [C, 3C], bias [3C] expected")
    if not all(t.is_cuda and t.is_contiguous() for t in ws + (x, *maps)):
        raise ValueError("all tensors must be contiguous GPU tensors")
    _check(lib().rib_ln_qkv(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(w), _ptr(bias),
                            _ptr(q) if q is not None else None, _ptr(k), _ptr(v),
                            _ptr(xn) if xn is not None else None, B, H, W, C, float(eps), _dtype_code(x), _stream(x)))


def window_attn_lnq(x, gamma, beta, w, bias, kc, v, g, qp, kp, heads: int, window: int, eps: float = 1e-5):
    """window_attn with Qc = LayerNorm(x) W_q + b_q computed inside the attention (the Q columns of
    rib_ln_qkv's w and bias); kc, v from ln_qkv_into(..., q=None, ...).  bf16 only."""
    import torch
    o = torch.empty_like(kc)
    window_attn_lnq_into(x, gamma, beta, w, bias, kc, v, g, qp, kp, heads, window, o, eps)
    return o


def window_attn_lnq_into(x, gamma, beta, w, bias, kc, v, g, qp, kp, heads: int, window: int, o,
                         eps: float = 1e-5) -> None:
    import torch
    ts = (x, kc, v, g, o)
    if any(t.dim() != 4 for t in ts) or any(t.shape != x.shape for t in ts):
        raise ValueError("x, kc, v, g, o must all be [B, H, W, C]")
    if any(t.dtype != torch.bfloat16 for t in ts):
        raise ValueError("x, kc, v, g, o must be bfloat16")
    B, H, W, C = x.shape
    ps = (gamma, beta, w, bias)
    if any(t.dtype != torch.float32 for t in ps) or gamma.shape != (C,) or beta.shape != (C,) \
            or w.shape != (C, 3 * C) or bias.shape != (3 * C,):
        raise ValueError("gamma, beta float32 [C], w [C, 3C], bias [3C] expected")
    if not all(t.is_cuda and t.is_contiguous() for t in ts + ps + (qp, kp)):
        raise ValueError("all tensors must be contiguous GPU tensors")
    if qp.dtype != torch.float32 or kp.dtype != torch.float32 or qp.shape != kp.shape or qp.dim() != 2 \
            or qp.shape[0] != window * window:
        raise ValueError("qp, kp must be float32 [window*window, R]")
    if heads < 1 or C % heads:
        raise ValueError("channel count must be a multiple of heads")
    _check(lib().rib_window_attn_lnq(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(w), _ptr(bias), _ptr(kc), _ptr(v),
                                     _ptr(g), _ptr(qp), _ptr(kp), _ptr(o), B, H, W, heads, C // heads, qp.shape[1],
                                     window, float(eps), _dtype_code(x), _stream(x)))


def weight_count3d(L: int, hidden: int, R: int) -> int:
    """Length of the packed space-time encoder weights W_h [3+6L][hidden] | b_h | Wp_q | Wp_k."""
    return (3 + 6 * L) * hidden + hidden + 2 * hidden * R


def encode3d(frames: int, window: int, L: int, hidden: int, R: int, weights):
    """Positional factors of frames x window x window space-time windows: float32 [frames*window^2, R] each."""
    import torch
    if not (weights.is_cuda and weights.dtype == torch.float32 and weights.is_contiguous()):
        raise ValueError("weights must be a contiguous float32 GPU tensor")
    if weights.numel() != weight_count3d(L, hidden, R):
        raise ValueError("packed weight vector has the wrong length")
    qp = torch.empty((frames * window * window, R), dtype=torch.float32, device=weights.device)
    kp = torch.empty_like(qp)
    _check(lib().rib_encode3d(frames, window, L, hidden, R, _ptr(weights), _ptr(qp), _ptr(kp), _stream(weights)))
    return qp, kp


def window_attn3d(qc, kc, v, g, qp, kp, heads: int, frames: int, window: int):
    """Window attention over [B, T, H, W, heads*dh] video maps with frames x window x window windows."""
    import torch
    ts = (qc, kc, v, g)
    if any(t.dim() != 5 or t.shape != qc.shape or t.dtype != qc.dtype for t in ts):
        raise ValueError("qc, kc, v, g must all be [B, T, H, W, C] of one dtype")
    if not all(t.is_cuda and t.is_contiguous() for t in ts + (qp, kp)):
        raise ValueError("all tensors must be contiguous GPU tensors")
    if qp.dtype != torch.float32 or kp.shape != qp.shape or qp.dim() != 2 or qp.shape[0] != frames * window * window:
        raise ValueError("qp, kp must be float32 [frames*window*window, R]")
    B, T, H, W, C = qc.shape
    if heads < 1 or C % heads:
        raise ValueError("channel count must be a multiple of heads")
    o = torch.empty_like(qc)
    _check(lib().rib_window_attn3d(_ptr(qc), _ptr(kc), _ptr(v), _ptr(g), _ptr(qp), _ptr(kp), _ptr(o), B, T, H, W,
                                   heads, C // heads, qp.shape[1], frames, window, _dtype_code(qc), _stream(qc)))
    return o


def supported(dh: int, R: int, window: int, dtype) -> bool:
    """Whether rib_window_attn has a compiled variant for this shape and dtype."""
    code = _dtype_code_from(dtype)
    return lib().rib_attn_supported(dh, R, window, code) == RIB_OK


def _dtype_code_from(dtype) -> int:
    import torch
    return {torch.float32: RIB_F32, torch.bfloat16: RIB_BF16}[dtype]
