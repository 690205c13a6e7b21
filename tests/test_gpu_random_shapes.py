"""GPU parity on seeded random shapes: forward attention (rib_window_attn and the training forward's
row log-sum-exp) against the fp64 oracle over whole outputs, at the forward's bars (max abs error
2e-2 for bf16 maps, 1e-5 for fp32; the log-sum-exp at a bound derived from the rounding of the score
operands, as in the score-range tests).

Each case draws B, H, W, heads, (dh, R) among the compiled shapes and a window size, so the cases
fall across the three bf16 kernels (whole-window up to 256 tokens, chunked above, tiled for the
(32, 16), (16, 32) and (30, 32) shapes above 2,048 tokens), both XCD dealings of the chunked
kernel (whole windows, or window units when a large window's count is not a multiple of 8), ragged
edge windows and windows larger than the map.  The draws come from fixed seeds and each case's
shape is in its test id.
"""
import sys

import numpy as np
import pytest

import oracle
import super_resolution_transformer_amd as rib
from super_resolution_transformer_amd import synthetic

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
SHAPES = [(30, 16), (16, 16), (8, 8), (32, 16), (16, 32), (30, 32)]


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    rib.lib()
    return t


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    dh, R = SHAPES[rng.integers(len(SHAPES))]
    ws = int(rng.choice([2, 5, 8, 13, 16, 17, 24, 32, 40, 47, 48, 64, 72, 96],
                        p=[.04, .04, .06, .04, .08, .06, .06, .1, .08, .08, .08, .1, .08, .1]))
    if ws >= 64:
        # up to four windows of one image and two heads: the fp64 oracle takes n^2 per window
        H = int(rng.integers(ws // 2, ws + 20))
        W = int(rng.integers(ws // 2, ws + 20))
        B, heads = 1, int(rng.integers(1, 3))
    else:
        # one to three windows per side, ragged edges
        H = int(rng.integers(max(1, ws // 2), 2 * ws + 15))
        W = int(rng.integers(max(1, ws // 2), 2 * ws + 15))
        B, heads = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    dtype = "f32" if seed % 8 == 7 and dh <= 64 else "bf16"
    return B, H, W, heads, dh, R, ws, dtype


CASES = [draw(s) for s in range(32)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}W{}h{}d{}R{}ws{}-{}".format(*c))
def test_random_shape_matches_oracle(torch, case):
    B, H, W, heads, dh, R, ws, dtype = case
    note(f"random shape {case}")
    p = synthetic.make_problem(B, H, W, heads, dh, R, dtype=dtype, seed=B + H + W + ws)
    if dtype == "bf16":
        maps = [torch.from_numpy(p.bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("qc", "kc", "v", "g")]
    else:
        maps = [torch.from_numpy(getattr(p, n)).cuda() for n in ("qc", "kc", "v", "g")]
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, torch.from_numpy(p.weights).cuda())
    o, lse = rib.window_attn_train(*maps, qp, kp, heads, ws)
    o_plain = rib.window_attn(*maps, qp, kp, heads, ws)
    torch.cuda.synchronize()
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, heads, ws)
    got = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - want).max())
    ref = oracle.window_lse(p.qc, p.kc, oq, ok, heads, ws)
    lerr = float(np.abs(lse.cpu().numpy() - ref).max())
    note(f"  O max|err| {err:.3g}  lse max|err| {lerr:.3g}")
    # lse: a score's rounding error is bounded by S, the largest sum of |products| of a score
    # (Cauchy-Schwarz per part), times 2^-7 for bf16 operands (each rounded to 2^-8) or
    # (dh + R) 2^-24 for fp32
    qn = np.linalg.norm(p.qc.reshape(-1, heads, dh), axis=-1).max()
    kn = np.linalg.norm(p.kc.reshape(-1, heads, dh), axis=-1).max()
    S = float(qn * kn) / np.sqrt(dh) + float(np.linalg.norm(oq, axis=1).max() * np.linalg.norm(ok, axis=1).max()) / np.sqrt(R)
    lbound = TOL[dtype] + (2.0 ** -7 if dtype == "bf16" else (dh + R) * 2.0 ** -24) * S
    note(f"  lse bound {lbound:.3g}")
    assert err <= TOL[dtype]
    assert lerr <= lbound
    same = torch.equal(o.view(torch.int16), o_plain.view(torch.int16)) if dtype == "bf16" else torch.equal(o, o_plain)
    assert same, "train forward and plain forward differ"
