"""GPU parity of the chunked kernel's two-pair form.

The host runs a chunked call with four 32-query blocks per wave (512 queries per workgroup, two
workgroups per CU) when its grid still fills at least four rounds of them; a grouped launch always
runs the one-pair form (two blocks per wave, 256 queries per workgroup).  Every query's arithmetic
is the same in both forms (the same 64-key tiles in the same order, the same 32-query blocks for
the re-run decision), so their outputs must agree bit for bit.  Here 20 images of one 96x96 window,
6 heads x dh 30, R = 16, select the two-pair form, with inputs that send blocks through the
checked re-run: score jumps of about +250 base-2 units past the first key tile (make_spike_problem)
and every score far below zero (make_low_score_problem).  The single call is compared with the
same call through rib_window_attn_multi bit for bit, with the training forward's O bit for bit,
and on sampled rows (spiked and plain queries, every head) with the oracle at the forward's bf16 bar.
The (16, 16) and (8, 8) shapes, which take the same form on large grids, are checked the same way
on plain inputs (ragged window rows and columns included).
"""
import sys

import numpy as np
import pytest

import oracle
import super_resolution_transformer_amd as rib
from super_resolution_transformer_amd import synthetic

pytestmark = pytest.mark.gpu

B, H, W, HEADS, DH, R, WS = 20, 96, 96, 6, 30, 16, 96
TOL = 2e-2


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
    return torch.from_numpy(p.bits[nm].view(np.int16)).view(torch.bfloat16).cuda()


def selects_two_pairs(torch, b=B, h=H, w=W, heads=HEADS, ws=WS):
    """The host's rule: (window units) x (512-query blocks per window) >= 8 x (compute units)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = b * ((h + ws - 1) // ws) * ((w + ws - 1) // ws) * heads
    return units * ((ws * ws + 511) // 512) >= 8 * cus


def problem(kind):
    if kind == "spike":
        return synthetic.make_spike_problem(B, H, W, HEADS, DH, R, WS, 32.0, 30.0, seed=11)
    a = 60.0 * np.sqrt(DH) / np.log2(np.e)  # scores about -60 base-2 units
    return synthetic.make_low_score_problem(B, H, W, HEADS, DH, R, a, seed=12, rows="all")


@pytest.mark.parametrize("kind", ["spike", "low"])
def test_two_pair_form_matches_grouped_and_oracle(torch, kind):
    note(f"two-pair chunked form, {kind} scores, {B} x {H}x{W}, {HEADS} heads x dh {DH}, ws {WS}")
    assert selects_two_pairs(torch), "this map no longer selects the two-pair form"
    p = problem(kind)
    maps = [dev(torch, p, nm) for nm in ("qc", "kc", "v", "g")]
    w = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(WS, p.L, p.hidden, p.R, w)
    o = rib.window_attn(*maps, qp, kp, HEADS, WS)
    (o_group,) = rib.window_attn_multi([(*maps, qp, kp, HEADS, WS)])
    o_train, _ = rib.window_attn_train(*maps, qp, kp, HEADS, WS)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_group.view(torch.int16)), "two-pair and one-pair forms differ"
    assert torch.equal(o.view(torch.int16), o_train.view(torch.int16)), "train forward and plain forward differ"
    got = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    # sampled rows: every image, plain and spiked positions, the last row and column of the window
    rng = np.random.default_rng(5)
    tb = np.concatenate([np.arange(B), rng.integers(0, B, 44)])
    ty = np.concatenate([rng.integers(0, H, B), rng.integers(0, H, 40), [0, H - 1, 31, 64]])
    tx = np.concatenate([rng.integers(0, W, B), rng.integers(0, W, 40), [0, W - 1, 33, 95]])
    oq, ok = oracle.encode(WS, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn_rows(p.qc, p.kc, p.v, p.g, oq, ok, HEADS, WS, tb, ty, tx)
    err = float(np.abs(got[tb, ty, tx] - want).max())
    note(f"  {tb.size} rows x {HEADS * DH} channels: max|err| {err:.3g}")
    assert err <= TOL


SHAPES = [
    # B, H, W, heads, dh, R, ws: the other (dh, R) shapes that take the four-block form
    (40, 96, 96, 3, 16, 16, 96),   # SST-lite heads, 96x96 windows
    (2, 380, 640, 3, 16, 16, 64),  # 64x64 windows, a ragged bottom row of windows (60 rows)
    (40, 96, 100, 3, 8, 8, 96),    # dh = R = 8, ragged right column of windows
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "B{0}H{1}W{2}h{3}d{4}R{5}ws{6}".format(*c))
def test_two_pair_form_other_shapes(torch, shape):
    b, h, w, heads, dh, r, ws = shape
    note(f"two-pair chunked form, plain scores, {shape}")
    assert selects_two_pairs(torch, b, h, w, heads, ws), "this map no longer selects the two-pair form"
    p = synthetic.make_problem(b, h, w, heads, dh, r, dtype="bf16", seed=b + h + w + dh)
    maps = [dev(torch, p, nm) for nm in ("qc", "kc", "v", "g")]
    wt = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, wt)
    o = rib.window_attn(*maps, qp, kp, heads, ws)
    (o_group,) = rib.window_attn_multi([(*maps, qp, kp, heads, ws)])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_group.view(torch.int16)), "two-pair and one-pair forms differ"
    got = o.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(6)
    tb = rng.integers(0, b, 48)
    ty = np.concatenate([rng.integers(0, h, 44), [0, h - 1, 0, h - 1]])
    tx = np.concatenate([rng.integers(0, w, 44), [0, w - 1, w - 1, 0]])
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn_rows(p.qc, p.kc, p.v, p.g, oq, ok, heads, ws, tb, ty, tx)
    err = float(np.abs(got[tb, ty, tx] - want).max())
    note(f"  {tb.size} rows x {heads * dh} channels: max|err| {err:.3g}")
    assert err <= TOL
