"""CPU oracle for RIB window attention with the CLA gate -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library and its Python binding never touch it.

The arithmetic lives in ``rib_oracle.c`` (plain fp64 C, OpenMP over
image x window x head units); this module only builds it with gcc, loads it
with ctypes and marshals numpy arrays.  ``brute.py`` is a second, independent
pure-Python implementation for tiny cases.

Method: "Rank-Factorized Implicit Neural Bias: Scaling Super-Resolution
Transformer with FlashAttention" (gist.science summaries, methodology part A;
omica.com.cn explainer, sections 2.2 and 2.3).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rib_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def compile_oracle(src: str, out: str) -> str:
    """gcc with IEEE semantics: no fast-math, no FMA contraction."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        compile_oracle(_SRC, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _configure(L):
    L.rib_oracle_threads.restype = ctypes.c_int
    L.rib_oracle_encode.argtypes = [ctypes.c_int] * 4 + [_D, _D, _D]
    L.rib_oracle_encode.restype = ctypes.c_int
    L.rib_oracle_attn_units.argtypes = [_D] * 6 + [ctypes.c_int] * 7 + [ctypes.c_long] * 2 + [_D]
    L.rib_oracle_attn_units.restype = ctypes.c_int
    L.rib_oracle_attn_units_heads.argtypes = [_D] * 6 + [ctypes.c_int] * 7 + [ctypes.c_long] * 2 + [_D]
    L.rib_oracle_attn_units_heads.restype = ctypes.c_int
    L.rib_oracle_attn_rows.argtypes = [_D] * 6 + [ctypes.c_int] * 8 + [_I] * 3 + [_D]
    L.rib_oracle_attn_rows.restype = ctypes.c_int
    L.rib_oracle_window_debug.argtypes = ([_D] * 6 + [ctypes.c_int] * 11 + [_D] * 3 + [_I] * 3)
    L.rib_oracle_window_debug.restype = ctypes.c_int
    L.rib_oracle_cla_gate.argtypes = [_D] * 5 + [ctypes.c_int] * 4 + [_D]
    L.rib_oracle_cla_gate.restype = ctypes.c_int
    L.rib_oracle_ln_qkv.argtypes = [_D] * 5 + [ctypes.c_int] * 4 + [ctypes.c_double] + [_D] * 4
    L.rib_oracle_ln_qkv.restype = ctypes.c_int
    L.rib_oracle_encode3d.argtypes = [ctypes.c_int] * 5 + [_D] * 3
    L.rib_oracle_encode3d.restype = ctypes.c_int
    L.rib_oracle_attn3d.argtypes = [_D] * 6 + [ctypes.c_int] * 9 + [_D]
    L.rib_oracle_attn3d.restype = ctypes.c_int
    L.rib_oracle_attn_lse.argtypes = [_D] * 4 + [ctypes.c_int] * 7 + [_D]
    L.rib_oracle_attn_lse.restype = ctypes.c_int
    L.rib_oracle_attn_backward.argtypes = [_D] * 7 + [ctypes.c_int] * 7 + [_D] * 6
    L.rib_oracle_attn_backward.restype = ctypes.c_int
    L.rib_oracle_attn_backward_heads.argtypes = [_D] * 7 + [ctypes.c_int] * 7 + [_D] * 6
    L.rib_oracle_attn_backward_heads.restype = ctypes.c_int
    L.rib_oracle_attn_lse_heads.argtypes = [_D] * 4 + [ctypes.c_int] * 7 + [_D]
    L.rib_oracle_attn_lse_heads.restype = ctypes.c_int
    L.rib_oracle_encode_backward.argtypes = [ctypes.c_int] * 4 + [_D] * 4
    L.rib_oracle_encode_backward.restype = ctypes.c_int
    return L


class using:
    """Context manager: route this module's calls to another build of the oracle
    (the mutation tests load deliberately broken copies to prove the pins bite)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def threads() -> int:
    """OpenMP threads the oracle runs with (all host cores unless OMP_NUM_THREADS says otherwise)."""
    return int(lib().rib_oracle_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def weight_count(L: int, hidden: int, R: int) -> int:
    """Length of the packed weight vector W_h | b_h | Wp_q | Wp_k."""
    return (2 + 4 * L) * hidden + hidden + 2 * hidden * R


def encode(window: int, L: int, hidden: int, R: int, weights) -> tuple[np.ndarray, np.ndarray]:
    """Qp, Kp as [window*window, R] float64 (coordinate encoder + implicit field)."""
    w = _f64(weights).reshape(-1)
    if w.size != weight_count(L, hidden, R):
        raise ValueError("packed weight vector has the wrong length")
    n = window * window
    qp = np.zeros((n, R), np.float64)
    kp = np.zeros((n, R), np.float64)
    if lib().rib_oracle_encode(window, L, hidden, R, _p(w), _p(qp), _p(kp)) != 0:
        raise ValueError("oracle encode rejected its arguments")
    return qp, kp


def _shape_args(qc, heads, dh):
    B, H, W, C = qc.shape
    if C != heads * dh:
        raise ValueError("channel count must equal heads*dh")
    return B, H, W


def units(B: int, H: int, W: int, heads: int, window: int) -> int:
    """Number of (image, window, head) units of a problem."""
    return B * (-(-H // window)) * (-(-W // window)) * heads


def window_attn(qc, kc, v, g, qp, kp, heads: int, window: int, unit_range=None) -> np.ndarray:
    """O = (softmax(Qc Kc^T/sqrt(dh) + Qp Kp^T/sqrt(R)) V) * sigmoid(G), NHWC float64.

    ``qp``/``kp`` are one shared [window*window, R] pair, or per-head tables
    [heads, window*window, R].  ``unit_range=(begin, end)`` restricts the work
    to those (image, window, head) units; outputs of the other units are left
    at zero.
    """
    qc, kc, v, g = (_f64(a) for a in (qc, kc, v, g))
    qp, kp = _f64(qp), _f64(kp)
    dh = qc.shape[-1] // heads
    B, H, W = _shape_args(qc, heads, dh)
    R = qp.shape[-1]
    per_head = qp.ndim == 3
    if per_head and (qp.shape[0] != heads or kp.shape != qp.shape):
        raise ValueError("per-head tables must be [heads, window*window, R]")
    o = np.zeros(qc.shape, np.float64)
    ub, ue = (0, -1) if unit_range is None else unit_range
    fn = lib().rib_oracle_attn_units_heads if per_head else lib().rib_oracle_attn_units
    rc = fn(_p(qc), _p(kc), _p(v), _p(g), _p(qp), _p(kp), B, H, W, heads, dh, R, window, ub, ue, _p(o))
    if rc != 0:
        raise ValueError("oracle attention rejected its arguments")
    return o


def window_attn_rows(qc, kc, v, g, qp, kp, heads: int, window: int, tok_b, tok_y, tok_x) -> np.ndarray:
    """Output rows [n, heads*dh] for the query tokens (tok_b[k], tok_y[k], tok_x[k])."""
    qc, kc, v, g = (_f64(a) for a in (qc, kc, v, g))
    qp, kp = _f64(qp), _f64(kp)
    dh = qc.shape[-1] // heads
    B, H, W = _shape_args(qc, heads, dh)
    R = qp.shape[-1]
    tb, ty, tx = (np.ascontiguousarray(np.asarray(t, dtype=np.int32)) for t in (tok_b, tok_y, tok_x))
    nq = tb.size
    out = np.zeros((nq, heads * dh), np.float64)
    rc = lib().rib_oracle_attn_rows(_p(qc), _p(kc), _p(v), _p(g), _p(qp), _p(kp), B, H, W, heads, dh,
                                    R, window, nq, tb.ctypes.data_as(_I), ty.ctypes.data_as(_I),
                                    tx.ctypes.data_as(_I), _p(out))
    if rc != 0:
        raise ValueError("oracle row attention rejected its arguments")
    return out


def window_debug(qc, kc, v, g, qp, kp, heads: int, window: int, b: int, wy: int, wx: int, h: int):
    """(Sc, Bm, P, tokens) for one (image, window, head): content score, explicit bias, softmax.

    ``tokens`` is an int array [nt, 3] of (y, x, n) in map scan order.
    """
    qc, kc, v, g = (_f64(a) for a in (qc, kc, v, g))
    qp, kp = _f64(qp), _f64(kp)
    dh = qc.shape[-1] // heads
    B, H, W = _shape_args(qc, heads, dh)
    R = qp.shape[-1]
    cap = window * window
    Sc = np.zeros(cap * cap, np.float64)
    Bm = np.zeros(cap * cap, np.float64)
    P = np.zeros(cap * cap, np.float64)
    ty = np.zeros(cap, np.int32)
    tx = np.zeros(cap, np.int32)
    tn = np.zeros(cap, np.int32)
    nt = lib().rib_oracle_window_debug(_p(qc), _p(kc), _p(v), _p(g), _p(qp), _p(kp), B, H, W, heads,
                                       dh, R, window, b, wy, wx, h, _p(Sc), _p(Bm), _p(P),
                                       ty.ctypes.data_as(_I), tx.ctypes.data_as(_I),
                                       tn.ctypes.data_as(_I))
    if nt < 0:
        raise ValueError("oracle debug view rejected its arguments")
    m = nt * nt
    toks = np.stack([ty[:nt], tx[:nt], tn[:nt]], axis=1)
    return (Sc[:m].reshape(nt, nt), Bm[:m].reshape(nt, nt), P[:m].reshape(nt, nt), toks)


def cla_gate(x, dw_w, dw_b, pw_w, pw_b) -> np.ndarray:
    """G = PWConv1x1(DWConv3x3(X)) in NHWC float64 (zero padding, stride 1).

    dw_w: [C, 3, 3], dw_b: [C], pw_w: [C_in, C_out] (y = x W), pw_b: [C].
    """
    x = _f64(x)
    B, H, W, C = x.shape
    dw_w, dw_b, pw_w, pw_b = _f64(dw_w), _f64(dw_b), _f64(pw_w), _f64(pw_b)
    if dw_w.shape != (C, 3, 3) or dw_b.shape != (C,) or pw_w.shape != (C, C) or pw_b.shape != (C,):
        raise ValueError("gate weights do not match the channel count")
    g = np.zeros(x.shape, np.float64)
    if lib().rib_oracle_cla_gate(_p(x), _p(dw_w), _p(dw_b), _p(pw_w), _p(pw_b), B, H, W, C, _p(g)) != 0:
        raise ValueError("oracle gate rejected its arguments")
    return g


def window_lse(qc, kc, qp, kp, heads: int, window: int) -> np.ndarray:
    """Row log-sum-exp of the scores, [B, H, W, heads] float64.  qp, kp: one shared pair
    [window*window, R] or one pair per head [heads, window*window, R]."""
    qc, kc, qp, kp = _f64(qc), _f64(kc), _f64(qp), _f64(kp)
    dh = qc.shape[-1] // heads
    B, H, W = _shape_args(qc, heads, dh)
    out = np.zeros((B, H, W, heads), np.float64)
    fn = lib().rib_oracle_attn_lse_heads if qp.ndim == 3 else lib().rib_oracle_attn_lse
    if qp.ndim == 3 and qp.shape[0] != heads:
        raise ValueError("per-head tables need one pair per head")
    if fn(_p(qc), _p(kc), _p(qp), _p(kp), B, H, W, heads, dh, qp.shape[-1], window, _p(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def window_attn_backward(qc, kc, v, g, qp, kp, dout, heads: int, window: int):
    """Gradients (dqc, dkc, dv, dg, dqp, dkp) of O = (softmax(S) V) * sigmoid(G) for the
    upstream gradient dout (NHWC float64).  With one shared pair qp, kp [window*window, R],
    dqp/dkp have that shape and sum over all windows, heads and images; with one pair per
    head [heads, window*window, R], dqp[h]/dkp[h] sum over the windows and images of head h."""
    qc, kc, v, g, dout = (_f64(a) for a in (qc, kc, v, g, dout))
    qp, kp = _f64(qp), _f64(kp)
    dh = qc.shape[-1] // heads
    B, H, W = _shape_args(qc, heads, dh)
    R = qp.shape[-1]
    if qp.ndim == 3 and qp.shape[0] != heads:
        raise ValueError("per-head tables need one pair per head")
    outs = [np.zeros(qc.shape, np.float64) for _ in range(4)]
    dqp = np.zeros(qp.shape, np.float64)
    dkp = np.zeros(kp.shape, np.float64)
    fn = lib().rib_oracle_attn_backward_heads if qp.ndim == 3 else lib().rib_oracle_attn_backward
    rc = fn(_p(qc), _p(kc), _p(v), _p(g), _p(qp), _p(kp), _p(dout), B, H, W, heads,
            dh, R, window, *[_p(a) for a in outs], _p(dqp), _p(dkp))
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments")
    return (*outs, dqp, dkp)


def encode_backward(window: int, L: int, hidden: int, R: int, weights, dqp, dkp) -> np.ndarray:
    """Gradient of the packed weights W_h | b_h | Wp_q | Wp_k for upstream dqp, dkp."""
    w = _f64(weights).reshape(-1)
    if w.size != weight_count(L, hidden, R):
        raise ValueError("packed weight vector has the wrong length")
    dqp, dkp = _f64(dqp), _f64(dkp)
    dw = np.zeros_like(w)
    if lib().rib_oracle_encode_backward(window, L, hidden, R, _p(w), _p(dqp), _p(dkp), _p(dw)) != 0:
        raise ValueError("oracle encode backward rejected its arguments")
    return dw


def ln_qkv(x, gamma, beta, w, bias, eps: float = 1e-5, with_xn: bool = False):
    """(q, k, v[, xn]) of the block's input projection: LayerNorm over channels, then x W + bias
    with w [C][3C] (columns Q | K | V); NHWC float64."""
    x = _f64(x)
    B, H, W, C = x.shape
    gamma, beta, w, bias = (_f64(a) for a in (gamma, beta, w, bias))
    if gamma.shape != (C,) or beta.shape != (C,) or w.shape != (C, 3 * C) or bias.shape != (3 * C,):
        raise ValueError("gamma, beta [C], w [C, 3C], bias [3C] expected")
    q, k, v = (np.zeros(x.shape, np.float64) for _ in range(3))
    xn = np.zeros(x.shape, np.float64) if with_xn else None
    rc = lib().rib_oracle_ln_qkv(_p(x), _p(gamma), _p(beta), _p(w), _p(bias), B, H, W, C, float(eps),
                                 _p(q), _p(k), _p(v), _p(xn) if with_xn else None)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return (q, k, v, xn) if with_xn else (q, k, v)


def weight_count3d(L: int, hidden: int, R: int) -> int:
    """Packed weights of the space-time encoder: W_h [3+6L][hidden] | b_h | Wp_q | Wp_k."""
    return (3 + 6 * L) * hidden + hidden + 2 * hidden * R


def encode3d(wt: int, ws: int, L: int, hidden: int, R: int, weights) -> tuple[np.ndarray, np.ndarray]:
    """Qp, Kp as [wt*ws*ws, R] float64 for wt x ws x ws space-time windows."""
    w = _f64(weights).reshape(-1)
    if w.size != weight_count3d(L, hidden, R):
        raise ValueError("packed weight vector has the wrong length")
    n = wt * ws * ws
    qp = np.zeros((n, R), np.float64)
    kp = np.zeros((n, R), np.float64)
    if lib().rib_oracle_encode3d(wt, ws, L, hidden, R, _p(w), _p(qp), _p(kp)) != 0:
        raise ValueError("oracle encode3d rejected its arguments")
    return qp, kp


def window_attn3d(qc, kc, v, g, qp, kp, heads: int, wt: int, ws: int) -> np.ndarray:
    """Attention over wt x ws x ws windows of [B, T, H, W, C] video maps (float64)."""
    qc, kc, v, g = (_f64(a) for a in (qc, kc, v, g))
    qp, kp = _f64(qp), _f64(kp)
    B, T, H, W, C = qc.shape
    if C % heads:
        raise ValueError("channel count must be a multiple of heads")
    o = np.zeros(qc.shape, np.float64)
    rc = lib().rib_oracle_attn3d(_p(qc), _p(kc), _p(v), _p(g), _p(qp), _p(kp), B, T, H, W, heads, C // heads,
                                 qp.shape[-1], wt, ws, _p(o))
    if rc != 0:
        raise ValueError("oracle attn3d rejected its arguments")
    return o
