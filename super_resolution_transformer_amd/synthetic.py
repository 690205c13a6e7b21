"""Seeded synthetic inputs for RIB window attention.

This module holds none of the method's arithmetic: it draws random tensors of
the shapes the pages describe and rounds them to bf16 when asked.  Both the
GPU path's tests and the CPU oracle read the arrays it returns, so the two
always see bit-identical inputs.

Workloads (shapes from the omica.com.cn explainer: width D=180 with 6 heads,
section 3.1; SST-lite D=48 / 3 heads / R=16, section 5.1; L=10 frequency
bands, section 2.2; cyclic windows 16/32/64, section 3.2; 96x96 windows and
training patches, gist.science summaries part 3; 1280x720 and 640x360 inputs,
explainer sections 2.1 and 5.1):

  tiny-fp32         1 x 64x64,   C=48  (3 x 16), window 16, fp32
  sst-lite-bf16     1 x 180x320, C=48  (3 x 16), windows 16, 32, 64
  sst-infer-bf16    1 x 180x320, C=180 (6 x 30), window 64
  sst-train-bf16   32 x 96x96,   C=180 (6 x 30), window 96
  large-input-bf16  1 x 360x640, C=180 (6 x 30), window 96

Every config uses R=16, L=10 and a hidden width of 64.  Feature maps are
N(0,1); the coordinate-MLP weights are N(0, 1/fan_in) with fan_in = 2+4L for
W_h and b_h and fan_in = hidden for the two rank heads.  Draw order: Qc, Kc,
V, G, then W_h, b_h, Wp_q, Wp_k, from numpy's PCG64 with the config's seed.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    H: int
    W: int
    heads: int
    dh: int
    windows: tuple
    R: int = 16
    L: int = 10
    hidden: int = 64
    seed: int = 0

    @property
    def C(self) -> int:
        return self.heads * self.dh


CONFIGS = {
    1: Config("tiny-fp32", "f32", 1, 64, 64, 3, 16, (16,), seed=0),
    2: Config("sst-lite-bf16", "bf16", 1, 180, 320, 3, 16, (16, 32, 64), seed=1),
    3: Config("sst-infer-bf16", "bf16", 1, 180, 320, 6, 30, (64,), seed=2),
    4: Config("sst-train-bf16", "bf16", 32, 96, 96, 6, 30, (96,), seed=3),
    5: Config("large-input-bf16", "bf16", 1, 360, 640, 6, 30, (96,), seed=4),
}


def round_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 values to bf16, nearest-even.  Returns (uint16 bits, float32 values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    bias = ((b >> 16) & 1) + np.uint32(0x7FFF)
    r = ((b + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return (r >> 16).astype(np.uint16), r.view(np.float32)


def weight_count(L: int, hidden: int, R: int) -> int:
    return (2 + 4 * L) * hidden + hidden + 2 * hidden * R


@dataclass
class Problem:
    """One set of inputs.  ``*_f32`` hold the exact values (bf16-representable
    when dtype is bf16); ``*_bits`` hold the bf16 bit patterns (bf16 only)."""
    B: int
    H: int
    W: int
    heads: int
    dh: int
    R: int
    L: int
    hidden: int
    dtype: str
    qc: np.ndarray
    kc: np.ndarray
    v: np.ndarray
    g: np.ndarray
    weights: np.ndarray          # packed float32: W_h | b_h | Wp_q | Wp_k
    bits: dict = field(default_factory=dict)

    @property
    def C(self) -> int:
        return self.heads * self.dh


def draw_weights(rng: np.random.Generator, L: int, hidden: int, R: int) -> np.ndarray:
    F = 2 + 4 * L
    wh = rng.standard_normal((F, hidden)) / np.sqrt(F)
    bh = rng.standard_normal(hidden) / np.sqrt(F)
    wq = rng.standard_normal((hidden, R)) / np.sqrt(hidden)
    wk = rng.standard_normal((hidden, R)) / np.sqrt(hidden)
    return np.concatenate([wh.ravel(), bh, wq.ravel(), wk.ravel()]).astype(np.float32)


def make_problem(B: int, H: int, W: int, heads: int, dh: int, R: int = 16, L: int = 10,
                 hidden: int = 64, dtype: str = "bf16", seed: int = 0) -> Problem:
    rng = np.random.default_rng(seed)
    shape = (B, H, W, heads * dh)
    arrs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(4)]
    weights = draw_weights(rng, L, hidden, R)
    bits = {}
    if dtype == "bf16":
        names = ("qc", "kc", "v", "g")
        for i, nm in enumerate(names):
            bits[nm], arrs[i] = round_bf16(arrs[i])
    elif dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return Problem(B, H, W, heads, dh, R, L, hidden, dtype, *arrs, weights=weights, bits=bits)


def make_spike_problem(B: int, H: int, W: int, heads: int, dh: int, R: int, ws: int, a: float, b: float,
                       dtype: str = "bf16", seed: int = 0) -> Problem:
    """A problem whose scores jump far above the first key tile's maximum.

    Every head slice of the queries with (y + x) even is replaced by a * e_0; in
    every window two keys at in-window (row, column) positions (ws // 3, 7) and
    (2 * ws // 3, ws // 2 + 1), where they exist, get b * e_0.  For those
    queries the two keys score a * b / sqrt(dh) (plus the positional bias),
    far above every other key, so the softmax is dominated by keys that are
    not in the first tile.  a and b should be exact in bf16."""
    p = make_problem(B, H, W, heads, dh, R, dtype=dtype, seed=seed)
    qc, kc = p.qc.copy(), p.kc.copy()
    yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    even = (yy + xx) % 2 == 0
    spike = np.zeros((H, W), bool)
    for (iy, ix) in ((ws // 3, 7), (2 * ws // 3, ws // 2 + 1)):
        if iy < ws and ix < ws:
            spike |= ((yy % ws) == iy) & ((xx % ws) == ix)
    e0 = np.zeros(dh, np.float32)
    e0[0] = 1.0
    for h in range(heads):
        sl = slice(h * dh, (h + 1) * dh)
        qc[:, even, sl] = a * e0
        kc[:, spike, sl] = b * e0
    p.qc, p.kc = qc, kc
    if dtype == "bf16":
        p.bits["qc"], p.qc = round_bf16(qc)
        p.bits["kc"], p.kc = round_bf16(kc)
    return p


def make_low_score_problem(B: int, H: int, W: int, heads: int, dh: int, R: int, a: float,
                           dtype: str = "bf16", seed: int = 0, rows: str = "all") -> Problem:
    """A problem whose scores lie far below zero for the queries of the chosen map rows.

    Per head, with u a random unit vector: keys kc = u + 0.05 z and, on the rows chosen by
    ``rows`` ("all", "even" or "odd" y), queries qc = -a u + 0.25 z' (z, z' ~ N(0, 1) per
    element), so each of their scores is about -a / sqrt(dh) (natural units; times log2(e) in
    base 2), spread by a few percent of that, plus the positional bias.  Queries on the other
    rows keep make_problem's N(0, 1) values (scores near 0)."""
    p = make_problem(B, H, W, heads, dh, R, dtype=dtype, seed=seed)
    rng = np.random.default_rng(seed + 7)
    qc = p.qc.copy()
    kc = np.empty_like(qc)
    sel = {"all": np.ones(H, bool), "even": np.arange(H) % 2 == 0, "odd": np.arange(H) % 2 == 1}[rows]
    for h in range(heads):
        u = rng.standard_normal(dh)
        u /= np.linalg.norm(u)
        sl = slice(h * dh, (h + 1) * dh)
        kc[..., sl] = u + 0.05 * rng.standard_normal((B, H, W, dh))
        low = -a * u + 0.25 * rng.standard_normal((B, H, W, dh))
        qc[:, sel, :, sl] = low[:, sel]
    p.qc, p.kc = qc, kc
    if dtype == "bf16":
        p.bits["qc"], p.qc = round_bf16(qc)
        p.bits["kc"], p.kc = round_bf16(kc)
    return p


def config_problem(idx: int, batch: int | None = None) -> Problem:
    """Inputs of one of the five workloads (``batch`` overrides B, e.g. for a CPU sample)."""
    c = CONFIGS[idx]
    return make_problem(c.B if batch is None else batch, c.H, c.W, c.heads, c.dh, c.R, c.L,
                        c.hidden, c.dtype, c.seed)


@dataclass
class GateProblem:
    """Input map X [B,H,W,C] and the CLA gate producer's weights (float32)."""
    x: np.ndarray                 # exact values (bf16-representable when dtype is bf16)
    dw_w: np.ndarray              # [C, 3, 3]
    dw_b: np.ndarray              # [C]
    pw_w: np.ndarray              # [C_in, C_out]
    pw_b: np.ndarray              # [C]
    dtype: str
    x_bits: np.ndarray | None = None


def make_gate_problem(B: int, H: int, W: int, C: int, dtype: str = "bf16", seed: int = 0) -> GateProblem:
    """X ~ N(0,1); depth-wise weights and bias ~ N(0, 1/9), point-wise ~ N(0, 1/C) (fan-in)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, W, C), dtype=np.float32)
    dw_w = (rng.standard_normal((C, 3, 3)) / 3.0).astype(np.float32)
    dw_b = (rng.standard_normal(C) / 3.0).astype(np.float32)
    pw_w = (rng.standard_normal((C, C)) / np.sqrt(C)).astype(np.float32)
    pw_b = (rng.standard_normal(C) / np.sqrt(C)).astype(np.float32)
    bits = None
    if dtype == "bf16":
        bits, x = round_bf16(x)
    elif dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return GateProblem(x, dw_w, dw_b, pw_w, pw_b, dtype, bits)


def make_upstream_grad(shape, dtype: str = "bf16", seed: int = 0) -> tuple[np.ndarray, np.ndarray | None]:
    """Upstream gradient dO for the backward: N(0, 1) entries (scale is immaterial, the backward is
    linear in dO).  Returns (exact float32 values, bf16 bits or None)."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        bits, x = round_bf16(x)
        return x, bits
    return x, None


@dataclass
class LnQkvProblem:
    """Inputs of the block's input projection (LayerNorm, then X W + b into Q | K | V)."""
    x: np.ndarray                 # [B, H, W, C] exact values (bf16-representable when dtype is bf16)
    gamma: np.ndarray             # [C]
    beta: np.ndarray              # [C]
    w: np.ndarray                 # [C, 3C]  (y = x W; columns Q | K | V)
    bias: np.ndarray              # [3C]
    dtype: str
    x_bits: np.ndarray | None = None


def make_ln_qkv_problem(B: int, H: int, W: int, C: int, dtype: str = "bf16", seed: int = 0) -> LnQkvProblem:
    """Block input with a per-token offset and scale (so the normalisation has work to do):
    x = a_t + s_t * z, a_t ~ N(0, 1), s_t = exp(N(0, 0.5^2)), z ~ N(0, 1); LayerNorm affine
    gamma = 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2); projection W ~ N(0, 1/C), bias ~ N(0, 0.1^2)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((B, H, W, 1))
    s = np.exp(0.5 * rng.standard_normal((B, H, W, 1)))
    x = (a + s * rng.standard_normal((B, H, W, C))).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C)).astype(np.float32)
    w = (rng.standard_normal((C, 3 * C)) / np.sqrt(C)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(3 * C)).astype(np.float32)
    bits = None
    if dtype == "bf16":
        bits, x = round_bf16(x)
    elif dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return LnQkvProblem(x, gamma, beta, w, bias, dtype, bits)
