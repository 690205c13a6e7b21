"""GPU parity for scores far above, or all far below, the reference of the softmax.

The tiled kernel (windows of more than 2,048 tokens for the (dh, R) shapes (32, 16), (16, 32) and
(30, 32)) takes the exact row maximum on the first key tile and then checks every later tile: the
packed bf16 P words are OR-reduced, and a value of 2 or more (the maximum grew by more than 8 base-2
units) sends the wave through an exact re-maximum and rescale before P is used.  The whole-window kernel (at
most 256 tokens) and the chunked kernel take no maximum in a first pass: every tile is
exponentiated against the fixed reference 0 with an offset of 64 base-2 units, unchecked; a block
whose row sum or output ends non-finite, or whose row sum is below 2^-86 (whole-window) or 2^-80
(chunked), is computed again with the checked loop.  The first set of inputs places two keys in
later tiles whose score, for half of the queries, exceeds everything else by about 84 base-2 units
(the checked rescale in the tiled kernel; the first pass holds it in the others, with p up to
~2^20) or by about 250 (p overflows: the tiled kernel rescales, the others' checked re-run takes
over).  A second set places every score far below zero (about -60 and -20 base-2 units): at -60
the whole-window and chunked kernels' row sums fall below their thresholds and the checked re-run
takes over, at -20 the first pass is kept; the tiled kernel takes the exact maximum of its first
tile either way.
Outputs are compared with the oracle over the whole map at the forward's bars (max abs error
2e-2 for bf16; 1e-5 for fp32 plus the rounding of two spike scores of ~175, derived in the
test); the row log-sum-exp at a bound derived from the rounding of the score operands.
"""
import sys

import numpy as np
import pytest

import oracle
import super_resolution_transformer_amd as rib
from super_resolution_transformer_amd import synthetic

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    rib.lib()
    return t


def dev(torch, p, nm):
    if p.dtype == "bf16":
        return torch.from_numpy(p.bits[nm].view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(getattr(p, nm)).cuda()


CASES = [
    # B, H, W, heads, dh, R, ws, b (key spike), dtype
    (1, 70, 64, 2, 30, 16, 64, 10.0, "bf16"),   # chunked kernel (4,096 tokens, few workgroups), +84: the first pass
    (1, 70, 64, 2, 30, 16, 64, 30.0, "bf16"),   # chunked kernel, +250: the checked re-run
    (1, 96, 100, 1, 30, 16, 96, 30.0, "bf16"),  # chunked kernel, 96x96 windows, ragged right column
    (1, 96, 100, 1, 30, 16, 96, 10.0, "bf16"),  # chunked kernel, 96x96 windows, +84
    (1, 96, 100, 1, 30, 32, 96, 30.0, "bf16"),  # tiled kernel ((30, 32) at 96x96), +250
    (1, 96, 100, 1, 30, 32, 96, 10.0, "bf16"),  # tiled kernel, +84
    (1, 40, 33, 2, 16, 16, 32, 30.0, "bf16"),   # chunked kernel, dh = 16 variant, ragged windows
    (2, 37, 40, 2, 30, 16, 16, 10.0, "bf16"),   # whole-window kernel, +84: the unchecked pass
    (2, 37, 40, 2, 30, 16, 16, 30.0, "bf16"),   # whole-window kernel, +250: the checked re-run
    (1, 70, 64, 1, 30, 16, 64, 30.0, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H{1}W{2}h{3}d{4}ws{6}b{7:g}-{8}".format(*c))
def test_score_jump_matches_oracle(torch, case):
    B, H, W, heads, dh, R, ws, b, dtype = case
    note(f"score jump {case}")
    p = synthetic.make_spike_problem(B, H, W, heads, dh, R, ws, 32.0, b, dtype=dtype, seed=H + W + ws)
    maps = [dev(torch, p, nm) for nm in ("qc", "kc", "v", "g")]
    w = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, w)
    o_plain = rib.window_attn(*maps, qp, kp, heads, ws)
    o, lse = rib.window_attn_train(*maps, qp, kp, heads, ws)
    torch.cuda.synchronize()
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, heads, ws)
    got = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    # S: largest sum of |products| in a score (Cauchy-Schwarz for the positional part)
    S = 32.0 * b / np.sqrt(dh) + float(np.linalg.norm(oq, axis=1).max() * np.linalg.norm(ok, axis=1).max()) / np.sqrt(R)
    # fp32: the two spike scores are rounded at magnitude S (each within 2^-24 S, twice:
    # the score and its difference with the maximum), and the output moves by at most a
    # quarter of that difference times |V1 - V2| <= 2 max|V|: 2^-23 S max|V| on top of the
    # 1e-5 bar.  bf16 keeps the 2e-2 bar.
    bound = TOL[dtype] + (2.0 ** -23 * S * float(np.abs(p.v).max()) if dtype == "f32" else 0.0)
    err = float(np.abs(got - want).max())
    note(f"  O max|err| {err:.3g}  max|O| {float(np.abs(want).max()):.3g}  bound {bound:.3g}")
    assert err <= bound
    same = torch.equal(o.view(torch.int16), o_plain.view(torch.int16)) if dtype == "bf16" else torch.equal(o, o_plain)
    assert same, "train forward and plain forward differ"
    # lse: the spike score itself carries the rounding of the scaled query operand
    # (bf16: u = 2^-8 per operand, a product of two rounded operands within 2^-7 of
    # S = the largest sum of |products| of a score; fp32: (dh + R) * 2^-24 * S)
    ref = oracle.window_lse(p.qc, p.kc, oq, ok, heads, ws)
    bound = TOL[dtype] + (2.0 ** -7 if dtype == "bf16" else (dh + R) * 2.0 ** -24) * S
    lerr = float(np.abs(lse.cpu().numpy() - ref).max())
    note(f"  lse max|err| {lerr:.3g}  max|lse| {float(np.abs(ref).max()):.3g}  bound {bound:.3g}")
    assert lerr <= bound


LOW = [
    # B, H, W, heads, dh, R, ws, target base-2 score, rows of low queries, dtype
    (2, 37, 40, 2, 30, 16, 16, -60.0, "all", "bf16"),   # whole-window kernel: the checked re-run
    (2, 37, 40, 2, 30, 16, 16, -20.0, "all", "bf16"),   # whole-window kernel: the first pass is kept
    (1, 40, 41, 3, 16, 16, 16, -60.0, "all", "bf16"),   # whole-window kernel, dh = 16
    (1, 40, 33, 2, 16, 16, 32, -60.0, "all", "bf16"),   # chunked kernel: every block re-runs
    (1, 40, 33, 2, 16, 16, 32, -20.0, "all", "bf16"),   # chunked kernel: the first pass is kept
    # 32x32 windows: a wave's block 0 holds an even window row, block 1 an odd one, so one block
    # of each wave re-runs while the other keeps its first pass
    (1, 64, 70, 2, 30, 16, 32, -60.0, "even", "bf16"),
    (1, 64, 70, 2, 30, 16, 32, -60.0, "odd", "bf16"),
    (1, 96, 100, 1, 30, 16, 96, -60.0, "all", "bf16"),  # chunked kernel, 96x96 windows
    (1, 96, 100, 1, 30, 32, 96, -60.0, "all", "bf16"),  # tiled kernel
    (1, 37, 40, 2, 30, 16, 16, -60.0, "all", "f32"),
]


@pytest.mark.parametrize("case", LOW, ids=lambda c: "H{1}W{2}h{3}d{4}ws{6}s{7:g}{8}-{9}".format(*c))
def test_scores_far_below_zero_match_oracle(torch, case):
    B, H, W, heads, dh, R, ws, target, rows, dtype = case
    note(f"low scores {case}")
    a = -target * np.sqrt(dh) / np.log2(np.e)
    p = synthetic.make_low_score_problem(B, H, W, heads, dh, R, a, dtype=dtype, seed=H + W + ws, rows=rows)
    maps = [dev(torch, p, nm) for nm in ("qc", "kc", "v", "g")]
    w = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, w)
    o_plain = rib.window_attn(*maps, qp, kp, heads, ws)
    o, lse = rib.window_attn_train(*maps, qp, kp, heads, ws)
    torch.cuda.synchronize()
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, heads, ws)
    got = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    ref = oracle.window_lse(p.qc, p.kc, oq, ok, heads, ws)
    note(f"  lse range [{float(ref.min()):.3g}, {float(ref.max()):.3g}] (natural units)")
    err = float(np.abs(got - want).max())
    note(f"  O max|err| {err:.3g}  max|O| {float(np.abs(want).max()):.3g}")
    assert err <= TOL[dtype]
    same = torch.equal(o.view(torch.int16), o_plain.view(torch.int16)) if dtype == "bf16" else torch.equal(o, o_plain)
    assert same, "train forward and plain forward differ"
    # lse: S bounds the sum of |products| of a score (Cauchy-Schwarz per part)
    qn = np.linalg.norm(p.qc.reshape(-1, heads, dh), axis=-1).max()
    kn = np.linalg.norm(p.kc.reshape(-1, heads, dh), axis=-1).max()
    S = float(qn * kn) / np.sqrt(dh) + float(np.linalg.norm(oq, axis=1).max() * np.linalg.norm(ok, axis=1).max()) / np.sqrt(R)
    bound = TOL[dtype] + (2.0 ** -7 if dtype == "bf16" else (dh + R) * 2.0 ** -24) * S
    lerr = float(np.abs(lse.cpu().numpy() - ref).max())
    note(f"  lse max|err| {lerr:.3g}  bound {bound:.3g}")
    assert lerr <= bound
