"""Brute-force RIB window attention in plain Python loops -- TEST INFRASTRUCTURE.

A second implementation of the same definition, written independently of
``rib_oracle.c`` (different traversal: it groups query tokens by window with a
dictionary and builds every score as content + bias term by term).  It is only
meant for tiny windows (2x2, 4x4) where its O(n^2 * C) Python loops finish in
well under a second.

Definition followed: the coordinate encoder and implicit neural field of the
omica.com.cn explainer (section 2.2), the content + bias score that the
channel concatenation reproduces (gist.science summaries, methodology part A),
and the gated output O = (softmax(S) V) * sigmoid(G) (explainer section 2.3).
"""
from __future__ import annotations

import math

import numpy as np


def coords(window: int) -> list[float]:
    """In-window coordinates: k -> -1 + 2k/(window-1), rounded once to float32."""
    return [float(np.float32(np.float32(2 * k - (window - 1)) / np.float32(window - 1)))
            for k in range(window)]


def features(cy: float, cx: float, L: int) -> list[float]:
    """[cy, cx] then, for each frequency 2^i: sin y, sin x, cos y, cos x."""
    out = [cy, cx]
    for i in range(L):
        f = 2.0 ** i
        out += [math.sin(f * cy), math.sin(f * cx), math.cos(f * cy), math.cos(f * cx)]
    return out


def encode(window: int, L: int, hidden: int, R: int, weights) -> tuple[list, list]:
    w = [float(x) for x in np.asarray(weights, dtype=np.float64).reshape(-1)]
    F = 2 + 4 * L
    pos = 0
    Wh = [[w[pos + f * hidden + j] for j in range(hidden)] for f in range(F)]
    pos += F * hidden
    bh = w[pos:pos + hidden]
    pos += hidden
    Wq = [[w[pos + j * R + r] for r in range(R)] for j in range(hidden)]
    pos += hidden * R
    Wk = [[w[pos + j * R + r] for r in range(R)] for j in range(hidden)]
    c = coords(window)
    qp, kp = [], []
    for iy in range(window):
        for ix in range(window):
            feat = features(c[iy], c[ix], L)
            h = []
            for j in range(hidden):
                z = bh[j] + sum(feat[f] * Wh[f][j] for f in range(F))
                h.append(max(z, 0.0))
            qp.append([sum(h[j] * Wq[j][r] for j in range(hidden)) for r in range(R)])
            kp.append([sum(h[j] * Wk[j][r] for j in range(hidden)) for r in range(R)])
    return qp, kp


def window_attn(qc, kc, v, g, qp, kp, heads: int, window: int) -> np.ndarray:
    """qp/kp: one shared list of rows, or a list of per-head lists (tables[h][n][r])."""
    qc, kc, v, g = (np.asarray(a, dtype=np.float64) for a in (qc, kc, v, g))
    B, H, W, C = qc.shape
    dh = C // heads
    per_head = np.asarray(qp).ndim == 3
    R = np.asarray(qp).shape[-1]
    groups: dict[tuple, list] = {}
    for b in range(B):
        for y in range(H):
            for x in range(W):
                groups.setdefault((b, y // window, x // window), []).append((y, x))
    out = np.zeros_like(qc)
    for (b, _, _), toks in groups.items():
        for h in range(heads):
            lo = h * dh
            tq = qp[h] if per_head else qp
            tk = kp[h] if per_head else kp
            for (yi, xi) in toks:
                ni = (yi % window) * window + (xi % window)
                scores = []
                for (yj, xj) in toks:
                    nj = (yj % window) * window + (xj % window)
                    content = 0.0
                    for d in range(dh):
                        content += qc[b, yi, xi, lo + d] * kc[b, yj, xj, lo + d]
                    bias = 0.0
                    for r in range(R):
                        bias += tq[ni][r] * tk[nj][r]
                    scores.append(content / math.sqrt(dh) + bias / math.sqrt(R))
                top = max(scores)
                e = [math.exp(s - top) for s in scores]
                z = sum(e)
                for d in range(dh):
                    acc = 0.0
                    for k, (yj, xj) in enumerate(toks):
                        acc += e[k] / z * v[b, yj, xj, lo + d]
                    gate = 1.0 / (1.0 + math.exp(-g[b, yi, xi, lo + d]))
                    out[b, yi, xi, lo + d] = acc * gate
    return out
