"""GPU parity of the chunked kernel's three- and four-block forms.

A chunked call's own launch runs two, three or four 32-query blocks per wave (256, 384 or 512
queries per workgroup; three workgroups per CU with two blocks, two with more), picked from the
size of its grid; a grouped launch always runs two.  Every query's arithmetic is the same in all
forms (the same 64-key tiles in the same order, the same 32-query blocks for the re-run decision),
so their outputs must agree bit for bit.  Maps that select three or four blocks are checked here
with inputs that send blocks through the checked re-run (score jumps of about +250 base-2 units
past the first key tile, make_spike_problem; every score far below zero, make_low_score_problem)
and with plain inputs for every (dh, R) shape that takes those forms, ragged window rows and
columns included: the single call against the same call through rib_window_attn_multi bit for bit,
the training forward's O against the plain forward's bit for bit, and sampled rows against the
oracle at the forward's bf16 bar.
"""
import sys

import numpy as np
import pytest

import oracle
import super_resolution_transformer_amd as rib
from super_resolution_transformer_amd import synthetic

pytestmark = pytest.mark.gpu

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


def blocks_per_wave(torch, b, h, w, heads, ws):
    """The host's choice for a chunked call of the (30, 16), (16, 16) or (8, 8) shapes."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = b * ((h + ws - 1) // ws) * ((w + ws - 1) // ws) * heads
    nw = ws * ws
    if units * ((nw + 511) // 512) >= 8 * cus:
        return 4
    if nw >= 4096 and 2 * units * ((nw + 383) // 384) >= 7 * cus:
        return 3
    return 2


def check(torch, p, b, h, w, heads, dh, ws, train=False):
    maps = [dev(torch, p, nm) for nm in ("qc", "kc", "v", "g")]
    wt = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, wt)
    o = rib.window_attn(*maps, qp, kp, heads, ws)
    (o_group,) = rib.window_attn_multi([(*maps, qp, kp, heads, ws)])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_group.view(torch.int16)), "the form and the grouped launch differ"
    if train:
        o_train, _ = rib.window_attn_train(*maps, qp, kp, heads, ws)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_train.view(torch.int16)), "train forward and plain forward differ"
    got = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    # sampled rows: every image, random positions, the map's corners
    rng = np.random.default_rng(5)
    n = 44
    tb = np.concatenate([np.arange(b), rng.integers(0, b, n), [0, b - 1, 0, b - 1]])
    ty = np.concatenate([rng.integers(0, h, b + n), [0, h - 1, 0, h - 1]])
    tx = np.concatenate([rng.integers(0, w, b + n), [0, w - 1, w - 1, 0]])
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn_rows(p.qc, p.kc, p.v, p.g, oq, ok, heads, ws, tb, ty, tx)
    err = float(np.abs(got[tb, ty, tx] - want).max())
    note(f"  {tb.size} rows x {heads * dh} channels: max|err| {err:.3g}")
    assert err <= TOL


RERUN = [
    # B, H, W, heads, dh, R, ws, blocks per wave, input
    (20, 96, 96, 6, 30, 16, 96, 4, "spike"),
    (20, 96, 96, 6, 30, 16, 96, 4, "low"),
    (1, 180, 320, 6, 30, 16, 64, 3, "spike"),   # the SST inference map, 64x64 windows, ragged bottom row
    (1, 180, 320, 6, 30, 16, 64, 3, "low"),
]


@pytest.mark.parametrize("case", RERUN, ids=lambda c: "B{0}H{1}W{2}ws{6}nb{7}-{8}".format(*c))
def test_rerun_matches_grouped_and_oracle(torch, case):
    b, h, w, heads, dh, r, ws, nb, kind = case
    note(f"{nb} blocks per wave, {kind} scores, {case[:7]}")
    assert blocks_per_wave(torch, b, h, w, heads, ws) == nb, "this map no longer selects that form"
    if kind == "spike":
        p = synthetic.make_spike_problem(b, h, w, heads, dh, r, ws, 32.0, 30.0, seed=11)
    else:
        a = 60.0 * np.sqrt(dh) / np.log2(np.e)  # scores about -60 base-2 units
        p = synthetic.make_low_score_problem(b, h, w, heads, dh, r, a, seed=12, rows="all")
    check(torch, p, b, h, w, heads, dh, ws, train=True)


SHAPES = [
    # B, H, W, heads, dh, R, ws, blocks per wave: the other (dh, R) shapes that take those forms
    (40, 96, 96, 3, 16, 16, 96, 4),   # SST-lite heads, 96x96 windows
    (2, 380, 640, 3, 16, 16, 64, 4),  # 64x64 windows, a ragged bottom row of windows (60 rows)
    (40, 96, 100, 3, 8, 8, 96, 4),    # dh = R = 8, ragged right column of windows
    (1, 380, 640, 3, 16, 16, 64, 3),  # three blocks, ragged bottom row
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "B{0}H{1}W{2}h{3}d{4}R{5}ws{6}nb{7}".format(*c))
def test_other_shapes_match_grouped_and_oracle(torch, shape):
    b, h, w, heads, dh, r, ws, nb = shape
    note(f"{nb} blocks per wave, plain scores, {shape[:7]}")
    assert blocks_per_wave(torch, b, h, w, heads, ws) == nb, "this map no longer selects that form"
    p = synthetic.make_problem(b, h, w, heads, dh, r, dtype="bf16", seed=b + h + w + dh)
    check(torch, p, b, h, w, heads, dh, ws)
