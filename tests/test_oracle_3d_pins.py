"""Pins of the oracle's space-time variant (explainer section 6: for video, the coordinate MLP takes
spatio-temporal coordinates and the attention windows become 3-D).

Held against the pinned 2-D oracle (single-frame windows are 2-D windows), an attention written
here with torch's softmax over gathered windows (content score plus the positional bias looked up
by in-window index), window locality, and an encoder written here in numpy; planted mistakes in
the oracle source must each fail a pin."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute


def video(B, T, H, W, C, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, T, H, W, C)) for _ in range(4)]


def weights3d(L, hidden, R, seed):
    return np.random.default_rng(seed).standard_normal(oracle.weight_count3d(L, hidden, R)) * 0.5


def np_encode3d(wt, ws, L, hidden, R, w):
    """The space-time encoder in numpy: coordinates as brute.coords (float32 grid; 0 for one frame)."""
    F = 3 + 6 * L
    Wh = w[:F * hidden].reshape(F, hidden)
    bh = w[F * hidden:F * hidden + hidden]
    o = F * hidden + hidden
    Wq = w[o:o + hidden * R].reshape(hidden, R)
    Wk = w[o + hidden * R:].reshape(hidden, R)
    ct = [0.0] if wt == 1 else brute.coords(wt)
    cs = brute.coords(ws)
    rows = []
    for it in range(wt):
        for iy in range(ws):
            for ix in range(ws):
                c = (ct[it], cs[iy], cs[ix])
                f = list(c)
                for i in range(L):
                    f += [math.sin(2.0 ** i * a) for a in c] + [math.cos(2.0 ** i * a) for a in c]
                rows.append(f)
    h = np.maximum(np.array(rows) @ Wh + bh, 0.0)
    return h @ Wq, h @ Wk


@pytest.mark.parametrize("wt,ws,L", [(2, 4, 2), (1, 3, 3), (3, 2, 0)])
def test_encoder3d_matches_numpy(wt, ws, L):
    hidden, R = 6, 4
    w = weights3d(L, hidden, R, wt + ws + L)
    got = oracle.encode3d(wt, ws, L, hidden, R, w)
    want = np_encode3d(wt, ws, L, hidden, R, w)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_encoder3d_single_frame_time_features():
    """wt = 1: c_t = 0, so sin(2^i c_t) = 0 and cos(2^i c_t) = 1 for every position.  A hidden unit that
    reads only c_t or sin(c_t) is 0 (after ReLU of 0); one that reads only cos(c_t) is 1 everywhere."""
    L, hidden, R, ws = 2, 3, 3, 4
    F = 3 + 6 * L
    Wh = np.zeros((F, hidden))
    Wh[0, 0] = 1.0       # c_t
    Wh[3, 1] = 1.0       # sin(c_t)
    Wh[6, 2] = 1.0       # cos(c_t)
    Wq = np.eye(hidden, R)
    w = np.concatenate([Wh.ravel(), np.zeros(hidden), Wq.ravel(), Wq.ravel()])
    qp, kp = oracle.encode3d(1, ws, L, hidden, R, w)
    np.testing.assert_array_equal(qp[:, 0], 0.0)
    np.testing.assert_array_equal(qp[:, 1], 0.0)
    np.testing.assert_array_equal(qp[:, 2], 1.0)


@pytest.mark.parametrize("T,H,W,ws", [(3, 9, 6, 4), (2, 5, 7, 2)])
def test_single_frame_windows_are_2d_windows(T, H, W, ws):
    """wt = 1: every frame is attended on its own with 2-D windows; the 3-D tables of a one-frame window
    are indexed exactly like the 2-D ones."""
    heads, dh, R = 2, 3, 4
    qc, kc, v, g = video(2, T, H, W, heads * dh, 3)
    qp, kp = oracle.encode3d(1, ws, 2, 5, R, weights3d(2, 5, R, 4))
    got = oracle.window_attn3d(qc, kc, v, g, qp, kp, heads, 1, ws)
    for t in range(T):
        want = oracle.window_attn(qc[:, t], kc[:, t], v[:, t], g[:, t], qp, kp, heads, ws)
        np.testing.assert_allclose(got[:, t], want, rtol=1e-12, atol=1e-13)


def torch_attn3d(qc, kc, v, g, qp, kp, heads, wt, ws):
    """Gather each space-time window's real tokens, then softmax(QcKc^T/sqrt(dh) + Qp Kp^T/sqrt(R)) V."""
    import torch
    B, T, H, W, C = qc.shape
    dh, R = C // heads, qp.shape[-1]
    out = np.zeros_like(qc)
    for b in range(B):
        for t0 in range(0, T, wt):
            for y0 in range(0, H, ws):
                for x0 in range(0, W, ws):
                    toks = [(t, y, x) for t in range(t0, min(T, t0 + wt)) for y in range(y0, min(H, y0 + ws))
                            for x in range(x0, min(W, x0 + ws))]
                    idx = tuple(np.array(a) for a in zip(*toks))
                    n = np.array([((t - t0) * ws + (y - y0)) * ws + (x - x0) for t, y, x in toks])
                    bias = torch.from_numpy(qp[n] @ kp[n].T / math.sqrt(R))
                    for h in range(heads):
                        sl = slice(h * dh, (h + 1) * dh)
                        q = torch.from_numpy(qc[b][idx][:, sl])
                        k = torch.from_numpy(kc[b][idx][:, sl])
                        vv = torch.from_numpy(v[b][idx][:, sl])
                        p = torch.softmax(q @ k.T / math.sqrt(dh) + bias, dim=-1)
                        o = (p @ vv).numpy() / (1.0 + np.exp(-g[b][idx][:, sl]))
                        for m, (t, y, x) in enumerate(toks):
                            out[b, t, y, x, sl] = o[m]
    return out


@pytest.mark.parametrize("T,H,W,wt,ws", [(5, 6, 7, 2, 4), (4, 4, 4, 4, 2), (3, 3, 5, 2, 3)])
def test_attn3d_matches_torch(T, H, W, wt, ws):
    heads, dh, R = 2, 3, 4
    qc, kc, v, g = video(1, T, H, W, heads * dh, T + H)
    qp, kp = oracle.encode3d(wt, ws, 1, 4, R, weights3d(1, 4, R, 7))
    got = oracle.window_attn3d(qc, kc, v, g, qp, kp, heads, wt, ws)
    want = torch_attn3d(qc, kc, v, g, qp, kp, heads, wt, ws)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_attn3d_locality():
    """Changing one token changes the outputs of its own space-time window only."""
    T, H, W, wt, ws = 5, 7, 6, 2, 4
    heads, dh, R = 1, 4, 3
    qc, kc, v, g = video(1, T, H, W, heads * dh, 9)
    qp, kp = oracle.encode3d(wt, ws, 1, 4, R, weights3d(1, 4, R, 10))
    base = oracle.window_attn3d(qc, kc, v, g, qp, kp, heads, wt, ws)
    kc2, v2 = kc.copy(), v.copy()
    kc2[0, 2, 5, 1] += 1.0
    v2[0, 2, 5, 1] += 1.0
    moved = oracle.window_attn3d(qc, kc2, v2, g, qp, kp, heads, wt, ws)
    changed = np.abs(moved - base).max(axis=-1)[0] > 0
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    inside = (t // wt == 2 // wt) & (y // ws == 5 // ws) & (x // ws == 1 // ws)
    assert changed[inside].all() and not changed[~inside].any()


MUTATIONS = {
    "row and column swapped in n": ("tn[nt] = ((t % wt) * ws + y % ws) * ws + x % ws;",
                                    "tn[nt] = ((t % wt) * ws + x % ws) * ws + y % ws;"),
    "frame window shifted": ("if (t / wt != wtw) continue;", "if ((t + 1) / wt != wtw) continue;"),
    "encoder index order": ("const int n = (it * ws + iy) * ws + ix;", "const int n = (iy * wt + it) * ws + ix;"),
    "single-frame time coordinate": ("return wt == 1 ? 0.0 : coord_value(k, wt);", "return coord_value(k, wt + 1);"),
    "sin t and sin y swapped": ("out[f++] = sin(freq * ct);\n    out[f++] = sin(freq * cy);",
                                "out[f++] = sin(freq * cy);\n    out[f++] = sin(freq * ct);"),
}

PINS = [
    lambda: test_encoder3d_matches_numpy(2, 4, 2),
    test_encoder3d_single_frame_time_features,
    lambda: test_single_frame_windows_are_2d_windows(3, 9, 6, 4),
    lambda: test_attn3d_matches_torch(5, 6, 7, 2, 4),
    test_attn3d_locality,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "rib_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor missing: {old}"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = oracle.compile_oracle(str(mut), str(tmp_path / "libmut.so"))
    caught = 0
    with oracle.using(so):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught += 1
    assert caught > 0, f"no pin caught the planted mistake '{name}'"
