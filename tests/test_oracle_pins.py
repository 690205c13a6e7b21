"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
closed forms, textbook constants, invariants, a library routine (PyTorch's
scaled_dot_product_attention on the CPU in float64) or an independent
brute-force implementation (oracle/brute.py).  The mutation test at the end
compiles deliberately broken copies of the oracle and shows that each planted
mistake fails at least one pin.

Pages: "Rank-Factorized Implicit Neural Bias" (gist.science summaries part A:
the concatenation identity; part B: the gate) and the omica.com.cn explainer
(section 2.2: coordinate encoder, implicit field, attention rewrite; section
2.3: O = (softmax(S) V) * sigmoid(G), G from a depth-wise 3x3 and a point-wise
1x1 convolution).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from super_resolution_transformer_amd import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


# ---------------------------------------------------------------- helpers
def pack(Wh, bh, Wq, Wk):
    return np.concatenate([Wh.ravel(), bh.ravel(), Wq.ravel(), Wk.ravel()]).astype(np.float64)


def coords32(ws):
    """Coordinates as float32 values (reading: endpoints included, float tensor)."""
    return [float(np.float32(np.float32(2 * k - (ws - 1)) / np.float32(ws - 1))) for k in range(ws)]


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def small_problem(B=2, H=9, W=6, heads=2, dh=3, R=4, L=2, hidden=5, seed=11):
    p = synthetic.make_problem(B, H, W, heads, dh, R, L, hidden, dtype="f32", seed=seed)
    return p


def window_pad_view(x, ws):
    """[B,H,W,C] -> [B, nWy, nWx, ws*ws, C] windows with NaN padding (written for the tests)."""
    B, H, W, C = x.shape
    Hp, Wp = -(-H // ws) * ws, -(-W // ws) * ws
    xp = np.full((B, Hp, Wp, C), np.nan)
    xp[:, :H, :W] = x
    xp = xp.reshape(B, Hp // ws, ws, Wp // ws, ws, C).transpose(0, 1, 3, 2, 4, 5)
    return xp.reshape(B, Hp // ws, Wp // ws, ws * ws, C)


# ---------------------------------------------------------------- page facts
def test_golden_page_facts_match_workloads():
    facts = json.load(open(GOLDEN))
    c = synthetic.CONFIGS
    assert all(cfg.L == facts["L"]["value"] for cfg in c.values())
    assert all(cfg.R == facts["R"]["value"] for cfg in c.values())
    assert c[3].C == facts["D_full"]["value"] and c[2].C == facts["D_lite"]["value"]
    assert c[2].heads == facts["heads_lite"]["value"]
    assert tuple(c[2].windows) == tuple(sorted(set(facts["cyclic_windows"]["value"])))
    assert c[4].windows == (facts["max_window"]["value"],) and (c[4].H, c[4].W) == tuple(facts["train_patch"]["value"])
    H720, W1280 = facts["output_1280x720"]["value"]
    assert (c[3].H, c[3].W) == (H720 // 4, W1280 // 4)       # x4 super-resolution input
    assert (c[5].H, c[5].W) == tuple(facts["input_640x360"]["value"])
    assert round(c[5].H * c[5].W / 1000) == facts["tokens_640x360_thousands"]["value"]


# ---------------------------------------------------------------- pin 1: encoder
@pytest.mark.parametrize("ws,expect", [
    (2, [-1.0, 1.0]),
    (3, [-1.0, 0.0, 1.0]),
    (5, [-1.0, -0.5, 0.0, 0.5, 1.0]),
    (4, [-1.0, -0.3333333432674408, 0.3333333432674408, 1.0]),   # float32 nearest to 1/3
])
def test_encoder_coordinates(ws, expect):
    """Identity features expose the coordinates: both ends of [-1,1] included, float32 values."""
    L, hidden, R = 0, 2, 2
    Wh = np.eye(2, hidden)                 # h0 = relu(cy + 2), h1 = relu(cx + 2)
    bh = np.array([2.0, 2.0])
    Wq = np.eye(hidden, R)
    Wk = np.zeros((hidden, R))
    qp, kp = oracle.encode(ws, L, hidden, R, pack(Wh, bh, Wq, Wk))
    got_y = qp[::ws, 0] - 2.0
    got_x = qp[:ws, 1] - 2.0
    assert np.array_equal(got_y, expect) and np.array_equal(got_x, expect)
    assert np.all(kp == 0.0)


def test_encoder_feature_order_and_frequencies():
    """One-hot W_h picks a single feature: [c_y, c_x, then per 2^i: sin y, sin x, cos y, cos x]."""
    ws, L, hidden, R = 3, 3, 1, 2
    F = 2 + 4 * L
    c = coords32(ws)
    textbook = {  # sin/cos at the float32 coordinates -1, 0, 1 (exact values are +-1, 0)
        ("sin", 1.0): 0.8414709848078965, ("cos", 1.0): 0.5403023058681398,
        ("sin", 2.0): 0.9092974268256817, ("cos", 2.0): -0.4161468365471424,
        ("sin", 4.0): -0.7568024953079282, ("cos", 4.0): -0.6536436208636119,
    }
    for f in range(F):
        Wh = np.zeros((F, hidden)); Wh[f, 0] = 1.0
        bh = np.array([2.0])
        Wq = np.array([[1.0, 0.0]]); Wk = np.array([[0.0, -1.0]])
        qp, kp = oracle.encode(ws, L, hidden, R, pack(Wh, bh, Wq, Wk))
        for n in range(ws * ws):
            cy, cx = c[n // ws], c[n % ws]
            if f < 2:
                want = (cy, cx)[f]
            else:
                i, k = divmod(f - 2, 4)
                fn = math.sin if k < 2 else math.cos
                arg = (2.0 ** i) * (cy if k % 2 == 0 else cx)
                key = ("sin" if k < 2 else "cos", abs(arg))
                want = fn(arg)
                if key in textbook:
                    want = textbook[key] * (np.sign(arg) if fn is math.sin else 1.0)
                    if arg == 0.0:
                        want = 0.0 if fn is math.sin else 1.0
            assert qp[n, 0] == pytest.approx(want + 2.0, abs=1e-15), (f, n)
            assert kp[n, 1] == pytest.approx(-(want + 2.0), abs=1e-15)
            assert qp[n, 1] == 0.0 and kp[n, 0] == 0.0


def test_encoder_zero_heads_and_relu():
    ws, L, hidden, R = 4, 10, 64, 16
    rng = np.random.default_rng(0)
    F = 2 + 4 * L
    Wh = rng.standard_normal((F, hidden)); bh = rng.standard_normal(hidden)
    Wq = rng.standard_normal((hidden, R)); Wk = rng.standard_normal((hidden, R))
    qp, kp = oracle.encode(ws, L, hidden, R, pack(Wh, bh, 0 * Wq, 0 * Wk))
    assert np.all(qp == 0.0) and np.all(kp == 0.0)
    # W_h = 0 and negative bias: ReLU kills everything
    qp, kp = oracle.encode(ws, L, hidden, R, pack(0 * Wh, -np.abs(bh) - 0.1, Wq, Wk))
    assert np.all(qp == 0.0) and np.all(kp == 0.0)
    # W_h = 0 and positive bias: h = b, Qp = b Wq for every position (y = x W orientation)
    b = np.abs(bh) + 0.1
    qp, kp = oracle.encode(ws, L, hidden, R, pack(0 * Wh, b, Wq, Wk))
    np.testing.assert_allclose(qp, np.tile(b @ Wq, (ws * ws, 1)), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(kp, np.tile(b @ Wk, (ws * ws, 1)), rtol=1e-13, atol=1e-13)


def test_encoder_symmetries():
    """cos features are even: with only cos rows, Qp is mirror symmetric in y and in x (exactly);
    equal y/x rows make Qp symmetric under transposition of the window."""
    ws, L, hidden, R = 6, 4, 8, 3
    F = 2 + 4 * L
    rng = np.random.default_rng(1)
    Wh = np.zeros((F, hidden))
    for i in range(L):
        Wh[4 + 4 * i] = rng.standard_normal(hidden)
        Wh[5 + 4 * i] = rng.standard_normal(hidden)
    bh = rng.standard_normal(hidden); Wq = rng.standard_normal((hidden, R)); Wk = rng.standard_normal((hidden, R))
    qp, _ = oracle.encode(ws, L, hidden, R, pack(Wh, bh, Wq, Wk))
    q = qp.reshape(ws, ws, R)
    assert np.array_equal(q, q[::-1]) and np.array_equal(q, q[:, ::-1])
    Wh = rng.standard_normal((F, hidden))
    Wh[1::2][: (F // 2)] = Wh[0::2][: (F // 2)]        # x rows equal y rows
    qp, _ = oracle.encode(ws, L, hidden, R, pack(Wh, bh, Wq, Wk))
    q = qp.reshape(ws, ws, R)
    # the y and x terms swap places in the hidden-layer sum, so equal up to rounding order
    np.testing.assert_allclose(q, q.transpose(1, 0, 2), rtol=1e-13, atol=1e-13)
    assert not np.allclose(q, q[::-1], rtol=1e-6)      # while not mirror symmetric


def test_encoder_matches_brute():
    ws, L, hidden, R = 5, 10, 16, 4
    w = synthetic.draw_weights(np.random.default_rng(5), L, hidden, R).astype(np.float64)
    qp, kp = oracle.encode(ws, L, hidden, R, w)
    bq, bk = brute.encode(ws, L, hidden, R, w)
    np.testing.assert_allclose(qp, bq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(kp, bk, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pin 2: concatenation identity
def test_concatenation_identity():
    """[Qc/sqrt(dh), Qp/sqrt(R)] [Kc, Kp]^T == Sc + Bm, the oracle's explicit content and bias."""
    p = small_problem(B=1, H=7, W=8, heads=2, dh=5, R=6, L=3, hidden=7)
    ws = 4
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    for (wy, wx) in [(0, 0), (1, 1), (0, 1)]:
        for h in range(p.heads):
            Sc, Bm, P, toks = oracle.window_debug(p.qc, p.kc, p.v, p.g, qp, kp, p.heads, ws, 0, wy, wx, h)
            ys, xs, ns = toks[:, 0], toks[:, 1], toks[:, 2]
            sl = slice(h * p.dh, (h + 1) * p.dh)
            qc64, kc64 = p.qc.astype(np.float64), p.kc.astype(np.float64)
            Qt = np.concatenate([qc64[0, ys, xs, sl] / math.sqrt(p.dh), qp[ns] / math.sqrt(p.R)], axis=1)
            Kt = np.concatenate([kc64[0, ys, xs, sl], kp[ns]], axis=1)
            S = Qt @ Kt.T
            np.testing.assert_allclose(Sc + Bm, S, rtol=1e-12, atol=1e-13)
            # and the bias alone really is Qp Kp^T / sqrt(R) over in-window positions
            np.testing.assert_allclose(Bm, qp[ns] @ kp[ns].T / math.sqrt(p.R), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- pin 3: brute force
@pytest.mark.parametrize("ws,H,W", [(2, 5, 7), (4, 9, 6), (4, 5, 7), (2, 9, 6)])
def test_attention_matches_brute_force(ws, H, W):
    p = small_problem(B=2, H=H, W=W, heads=2, dh=3, R=4, L=2, hidden=5, seed=ws * 100 + H)
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    got = oracle.window_attn(p.qc, p.kc, p.v, p.g, qp, kp, p.heads, ws)
    bq, bk = brute.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = brute.window_attn(p.qc, p.kc, p.v, p.g, bq, bk, p.heads, ws)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pin 4: softmax rows
def test_softmax_rows_sum_to_one():
    p = small_problem(B=1, H=11, W=10, heads=2, dh=4, R=4, L=3, hidden=6)
    ws = 4
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    for (wy, wx) in [(0, 0), (2, 2), (2, 0)]:
        _, _, P, toks = oracle.window_debug(p.qc, p.kc, p.v, p.g, qp, kp, p.heads, ws, 0, wy, wx, 1)
        assert P.shape[0] == toks.shape[0] > 0
        assert np.all(P >= 0.0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pin 5: window mean
@pytest.mark.parametrize("ws,H,W", [(4, 10, 7), (3, 8, 8), (16, 20, 37)])
def test_zero_scores_give_gated_window_mean(ws, H, W):
    """Qc = Kc = 0 and Wp = 0: every score is 0, softmax is uniform over the window's real tokens,
    so O = sigmoid(G) * mean(V over the real tokens of the window) -- edge windows included."""
    p = small_problem(B=2, H=H, W=W, heads=3, dh=4, R=4, L=2, hidden=6)
    w = p.weights.astype(np.float64).copy()
    F = 2 + 4 * p.L
    w[F * p.hidden + p.hidden:] = 0.0              # Wp_q = Wp_k = 0
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, w)
    z = np.zeros_like(p.qc)
    got = oracle.window_attn(z, z, p.v, p.g, qp, kp, p.heads, ws)
    wv = window_pad_view(p.v.astype(np.float64), ws)                 # [B,nWy,nWx,N,C]
    mean = np.nanmean(wv, axis=3)                                     # per window
    B = p.B
    want = np.zeros_like(got)
    for y in range(H):
        for x in range(W):
            want[:, y, x] = mean[:, y // ws, x // ws] * sigmoid(p.g[:, y, x].astype(np.float64))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- pin 6: library attention
def _sdpa_windows(q, k, v, ws, scale):
    """Window attention through torch's SDPA (CPU, float64) with a boolean key mask for padding."""
    import torch
    qv, kv, vv = (window_pad_view(a, ws) for a in (q, k, v))           # [B,nWy,nWx,N,c]
    mask = ~np.isnan(kv[..., 0])
    qt, kt, vt = (torch.from_numpy(np.nan_to_num(a)) for a in (qv, kv, vv))
    m = torch.from_numpy(mask)[..., None, :]                            # [B,nWy,nWx,1,N]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out.numpy()


def _unwindow(o, B, H, W, ws):
    Bn, nWy, nWx, N, c = o.shape
    o = o.reshape(B, nWy, nWx, ws, ws, c).transpose(0, 1, 3, 2, 4, 5).reshape(B, nWy * ws, nWx * ws, c)
    return o[:, :H, :W]


@pytest.mark.parametrize("ws,H,W", [(4, 10, 7), (8, 16, 16), (8, 13, 21)])
def test_zero_bias_is_plain_window_attention(ws, H, W):
    """Wp = 0: the bias vanishes and the oracle must equal softmax(QcKc^T/sqrt(dh)) V * sigmoid(G)
    computed by PyTorch's scaled_dot_product_attention (CPU, float64)."""
    p = small_problem(B=2, H=H, W=W, heads=2, dh=8, R=4, L=3, hidden=6)
    w = p.weights.astype(np.float64).copy()
    F = 2 + 4 * p.L
    w[F * p.hidden + p.hidden:] = 0.0
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, w)
    got = oracle.window_attn(p.qc, p.kc, p.v, p.g, qp, kp, p.heads, ws)
    for h in range(p.heads):
        sl = slice(h * p.dh, (h + 1) * p.dh)
        q, k, v = (a[..., sl].astype(np.float64) for a in (p.qc, p.kc, p.v))
        o = _unwindow(_sdpa_windows(q, k, v, ws, 1.0 / math.sqrt(p.dh)), p.B, H, W, ws)
        want = o * sigmoid(p.g[..., sl].astype(np.float64))
        np.testing.assert_allclose(got[..., sl], want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("ws,H,W", [(4, 10, 7), (8, 13, 21)])
def test_zero_content_is_bias_only_attention(ws, H, W):
    """Qc = Kc = 0: the scores are the bias alone, Qp Kp^T / sqrt(R), with the same (Qp, Kp) in
    every window -- checked against SDPA over the positional factors."""
    p = small_problem(B=1, H=H, W=W, heads=2, dh=5, R=6, L=4, hidden=9)
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    z = np.zeros_like(p.qc)
    got = oracle.window_attn(z, z, p.v, p.g, qp, kp, p.heads, ws)
    Hp, Wp = -(-H // ws) * ws, -(-W // ws) * ws
    pos = qp.reshape(ws, ws, p.R)
    kpos = kp.reshape(ws, ws, p.R)
    qmap = np.tile(pos, (Hp // ws, Wp // ws, 1))[None, :H, :W]
    kmap = np.tile(kpos, (Hp // ws, Wp // ws, 1))[None, :H, :W]
    for h in range(p.heads):
        sl = slice(h * p.dh, (h + 1) * p.dh)
        o = _unwindow(_sdpa_windows(qmap, kmap, p.v[..., sl].astype(np.float64), ws, 1.0 / math.sqrt(p.R)),
                      p.B, H, W, ws)
        want = o * sigmoid(p.g[..., sl].astype(np.float64))
        np.testing.assert_allclose(got[..., sl], want, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- pin 7: locality / equivariance
def test_locality_and_equivariance():
    ws, H, W = 4, 12, 12
    p = small_problem(B=2, H=H, W=W, heads=2, dh=4, R=4, L=2, hidden=6)
    qc, kc, v, g = (a.astype(np.float64) for a in (p.qc, p.kc, p.v, p.g))
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    base = oracle.window_attn(qc, kc, v, g, qp, kp, p.heads, ws)
    # perturb one key token: only its window (in its image) may change
    kc2, v2 = kc.copy(), v.copy()
    kc2[1, 5, 6] += 1.5
    v2[1, 5, 6] -= 2.0
    out = oracle.window_attn(qc, kc2, v2, g, qp, kp, p.heads, ws)
    changed = np.any(out != base, axis=-1)
    inside = np.zeros_like(changed)
    inside[1, 4:8, 4:8] = True
    assert np.all(changed[inside]) and not np.any(changed[~inside])
    # swapping two whole windows swaps the outputs exactly
    def swap(a):
        a = a.copy()
        t = a[:, 0:4, 4:8].copy()
        a[:, 0:4, 4:8] = a[:, 8:12, 0:4]
        a[:, 8:12, 0:4] = t
        return a
    out = oracle.window_attn(swap(qc), swap(kc), swap(v), swap(g), qp, kp, p.heads, ws)
    assert np.array_equal(out, swap(base))
    # identical images -> identical outputs
    same = [np.stack([a[0], a[0]]) for a in (qc, kc, v, g)]
    out = oracle.window_attn(*same, qp, kp, p.heads, ws)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], base[0])


# ---------------------------------------------------------------- pin 8: index mapping
def one_hot_problem(ws, H, W, B=2, heads=2, dh=16, alpha=32.0, seed=3):
    """Qc = Kc = alpha * e_{n mod dh} (n = in-window index), G = +100: P is one-hot on the
    diagonal, sigmoid is 1, so O == V exactly (requires dh >= ws*ws)."""
    rng = np.random.default_rng(seed)
    C = heads * dh
    qc = np.zeros((B, H, W, C), np.float32)
    for y in range(H):
        for x in range(W):
            n = (y % ws) * ws + (x % ws)
            for h in range(heads):
                qc[:, y, x, h * dh + n] = alpha
    v = synthetic.round_bf16(rng.standard_normal((B, H, W, C)).astype(np.float32) + 3.0)[1]
    g = np.full((B, H, W, C), 100.0, np.float32)
    return qc, qc.copy(), v, g


@pytest.mark.parametrize("ws,H,W", [(2, 5, 7), (4, 9, 6), (4, 8, 8)])
def test_one_hot_index_mapping_returns_v(ws, H, W):
    qc, kc, v, g = one_hot_problem(ws, H, W)
    R = 4
    qp = np.zeros((ws * ws, R)); kp = np.zeros((ws * ws, R))
    out = oracle.window_attn(qc, kc, v, g, qp, kp, 2, ws)
    assert np.array_equal(out, v.astype(np.float64))


def test_large_scores_stay_finite():
    """Scores near 1000 (alpha = 64): exp would overflow without the max subtraction; the
    softmax is still exactly one-hot and O == V."""
    ws, H, W = 4, 7, 9
    qc, kc, v, g = one_hot_problem(ws, H, W, alpha=64.0)
    qp = np.zeros((ws * ws, 4)); kp = np.zeros((ws * ws, 4))
    out = oracle.window_attn(qc, kc, v, g, qp, kp, 2, ws)
    assert np.all(np.isfinite(out)) and np.array_equal(out, v.astype(np.float64))


# ---------------------------------------------------------------- rows entry point
def test_rows_entry_matches_full():
    p = small_problem(B=2, H=13, W=9, heads=2, dh=4, R=4, L=2, hidden=5)
    ws = 4
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    full = oracle.window_attn(p.qc, p.kc, p.v, p.g, qp, kp, p.heads, ws)
    tb, ty, tx = [1, 0, 1, 0], [12, 0, 5, 3], [8, 0, 2, 7]
    rows = oracle.window_attn_rows(p.qc, p.kc, p.v, p.g, qp, kp, p.heads, ws, tb, ty, tx)
    assert np.array_equal(rows, full[tb, ty, tx])


# ---------------------------------------------------------------- mutations: the pins bite

# ---------------------------------------------------------------- per-head positional tables
def test_per_head_tables_match_brute_force():
    """Tables [heads, N, R] (one pair per head): the C oracle against the pure-Python brute force."""
    p = small_problem(B=2, H=5, W=7, heads=2, dh=3, R=4, seed=31)
    ws = 4
    rng = np.random.default_rng(32)
    qp = rng.standard_normal((2, ws * ws, 4))
    kp = rng.standard_normal((2, ws * ws, 4))
    got = oracle.window_attn(p.qc, p.kc, p.v, p.g, qp, kp, 2, ws)
    want = brute.window_attn(p.qc, p.kc, p.v, p.g, qp.tolist(), kp.tolist(), 2, ws)
    assert np.abs(got - want).max() <= 1e-12


def test_per_head_tables_reduce_to_shared_and_separate():
    """Equal per-head tables give the shared-table result; each head of a per-head run equals a
    shared-table run with that head's tables (head h reads table h, not another one)."""
    p = small_problem(B=1, H=9, W=6, heads=3, dh=2, R=4, seed=33)
    ws = 4
    rng = np.random.default_rng(34)
    q1, k1 = rng.standard_normal((ws * ws, 4)), rng.standard_normal((ws * ws, 4))
    shared = oracle.window_attn(p.qc, p.kc, p.v, p.g, q1, k1, 3, ws)
    same = oracle.window_attn(p.qc, p.kc, p.v, p.g, np.stack([q1] * 3), np.stack([k1] * 3), 3, ws)
    assert np.array_equal(shared, same)
    qh, kh = rng.standard_normal((3, ws * ws, 4)), rng.standard_normal((3, ws * ws, 4))
    per = oracle.window_attn(p.qc, p.kc, p.v, p.g, qh, kh, 3, ws)
    for h in range(3):
        one = oracle.window_attn(p.qc, p.kc, p.v, p.g, qh[h], kh[h], 3, ws)
        assert np.array_equal(per[..., 2 * h:2 * h + 2], one[..., 2 * h:2 * h + 2])


# ---------------------------------------------------------------- CLA gate producer
def gate_weights(C, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((C, 3, 3)) / 3.0, rng.standard_normal(C) * 0.1,
            rng.standard_normal((C, C)) / math.sqrt(C), rng.standard_normal(C) * 0.1)


def torch_gate(x, dw_w, dw_b, pw_w, pw_b):
    """The same definition through PyTorch's conv2d (CPU, float64): depth-wise 3x3 with zero
    padding (groups = C), then a 1x1 convolution whose weight is pw_w transposed."""
    import torch
    C = x.shape[-1]
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).permute(0, 3, 1, 2)
    d = torch.nn.functional.conv2d(xt, torch.from_numpy(dw_w)[:, None], torch.from_numpy(dw_b),
                                   padding=1, groups=C)
    g = torch.nn.functional.conv2d(d, torch.from_numpy(pw_w.T.copy())[:, :, None, None],
                                   torch.from_numpy(pw_b))
    return g.permute(0, 2, 3, 1).numpy()


@pytest.mark.parametrize("B,H,W,C", [(2, 5, 7, 6), (1, 1, 1, 3), (1, 3, 13, 48), (2, 9, 4, 30)])
def test_cla_gate_matches_torch_conv2d(B, H, W, C):
    rng = np.random.default_rng(B * 100 + H * 10 + W + C)
    x = rng.standard_normal((B, H, W, C))
    w = gate_weights(C, C)
    got = oracle.cla_gate(x, *w)
    want = torch_gate(x, *w)
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_cla_gate_identity_weights_return_x():
    """Centre tap 1, identity point-wise weights, no biases: G == X exactly."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 6, 5, 7))
    dw = np.zeros((7, 3, 3))
    dw[:, 1, 1] = 1.0
    g = oracle.cla_gate(x, dw, np.zeros(7), np.eye(7), np.zeros(7))
    assert np.array_equal(g, x)


def test_cla_gate_constant_input_counts_taps():
    """X = a everywhere, point-wise identity: D = a * (sum of the taps that fall inside the map)
    + b -- 9 taps inside, 6 on an edge, 4 in a corner (zero padding)."""
    C, a = 3, 1.5
    x = np.full((1, 4, 5, C), a)
    dw = np.arange(1.0, 1.0 + 9 * C).reshape(C, 3, 3)
    db = np.array([0.25, -0.5, 1.0])
    g = oracle.cla_gate(x, dw, db, np.eye(C), np.zeros(C))
    inner = a * dw.sum(axis=(1, 2)) + db
    corner = a * dw[:, 1:, 1:].sum(axis=(1, 2)) + db      # top-left: rows/cols -1 are outside
    edge = a * dw[:, 1:, :].sum(axis=(1, 2)) + db         # top edge: row -1 outside
    assert np.allclose(g[0, 2, 2], inner, rtol=0, atol=1e-12)
    assert np.allclose(g[0, 0, 0], corner, rtol=0, atol=1e-12)
    assert np.allclose(g[0, 0, 2], edge, rtol=0, atol=1e-12)


def test_cla_gate_point_wise_orientation():
    """Depth-wise identity, one-hot point-wise weight W[c_in=1][c_out=2] = 1: channel 2 of G is
    channel 1 of X (y = x W orientation), the others are their biases."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 3, 3, 4))
    dw = np.zeros((4, 3, 3))
    dw[:, 1, 1] = 1.0
    pw = np.zeros((4, 4))
    pw[1, 2] = 1.0
    pb = np.array([0.5, -1.0, 0.0, 2.0])
    g = oracle.cla_gate(x, dw, np.zeros(4), pw, pb)
    assert np.array_equal(g[..., 2], x[..., 1])
    assert np.all(g[..., 0] == 0.5) and np.all(g[..., 1] == -1.0) and np.all(g[..., 3] == 2.0)

MUTATIONS = {
    "bias dropped": ("Bm[j] = bb * inv_sqrt_r;", "Bm[j] = 0.0 * bb;"),
    "bias unscaled": ("Bm[j] = bb * inv_sqrt_r;", "Bm[j] = bb;"),
    "content scale 1/dh": ("1.0 / sqrt((double)p->dh)", "1.0 / (double)p->dh"),
    "gate sign": ("exp(-p->g[", "exp(p->g["),
    "gate missing": ("out[d] = a * gate;", "out[d] = a + 0.0 * gate;"),
    "key positional index": ("const double* kpos = p->kp + (size_t)h * p->tstride + (size_t)tn[j] * p->R;",
                             "const double* kpos = p->kp + (size_t)h * p->tstride + (size_t)tn[i] * p->R;"),
    "sin/cos swapped": ("out[f++] = sin(freq * cy);", "out[f++] = cos(freq * cy);"),
    "frequency off by one": ("double freq = ldexp(1.0, i);", "double freq = ldexp(1.0, i + 1);"),
    "coordinate endpoints": ("float num = (float)(2 * k - (ws - 1));", "float num = (float)(2 * k - ws);"),
    "window of x uses wy": ("if (x / p->ws != wx) continue;", "if (x / p->ws != wy) continue;"),
    "no max subtraction": ("P[j] = exp(P[j] - mx);", "P[j] = exp(P[j]);"),
    "hidden relu dropped": ("h[j] = acc > 0.0 ? acc : 0.0;", "h[j] = acc;"),
    "kp uses Wq": ("ak += h[j] * Wk[(size_t)j * R + r];", "ak += h[j] * Wq[(size_t)j * R + r];"),
    "gate point-wise transposed": ("acc += d[c] * pw_w[(size_t)c * C + o];", "acc += d[c] * pw_w[(size_t)o * C + c];"),
    "gate taps transposed": ("dw_w[(size_t)c * 9 + (dy + 1) * 3 + (dx + 1)]", "dw_w[(size_t)c * 9 + (dx + 1) * 3 + (dy + 1)]"),
    "gate depth-wise bias dropped": ("double acc = dw_b[c];", "double acc = 0.0 * dw_b[c];"),
    "gate point-wise bias dropped": ("double acc = pw_b[o];", "double acc = 0.0 * pw_b[o];"),
    "per-head table of head 0": ("p->qp + (size_t)h * p->tstride", "p->qp + (size_t)0 * p->tstride"),
    "gate padding on the wrong side": ("if (yy < 0 || yy >= H || xs < 0 || xs >= W) continue;",
                                       "if (yy < 0 || yy >= H || xs < 0 || xs >= W || (dy == 1 && dx == 1 && y == 0)) continue;"),
}

PINS = [
    test_encoder_feature_order_and_frequencies,
    lambda: test_encoder_coordinates(4, [-1.0, -0.3333333432674408, 0.3333333432674408, 1.0]),
    test_encoder_zero_heads_and_relu,
    test_concatenation_identity,
    lambda: test_attention_matches_brute_force(4, 9, 6),
    lambda: test_attention_matches_brute_force(2, 5, 7),
    test_softmax_rows_sum_to_one,
    lambda: test_zero_scores_give_gated_window_mean(4, 10, 7),
    lambda: test_zero_bias_is_plain_window_attention(8, 13, 21),
    lambda: test_zero_content_is_bias_only_attention(4, 10, 7),
    lambda: test_one_hot_index_mapping_returns_v(4, 9, 6),
    test_large_scores_stay_finite,
    test_encoder_matches_brute,
    test_per_head_tables_match_brute_force,
    lambda: test_cla_gate_matches_torch_conv2d(2, 5, 7, 6),
    test_cla_gate_identity_weights_return_x,
    test_cla_gate_constant_input_counts_taps,
    test_cla_gate_point_wise_orientation,
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
