"""GPU parity for scores far above the first key tile's maximum.

The bf16 tiled kernel takes the exact row maximum on the first key tile only;
later tiles are exponentiated against that reference without a check, and a
workgroup whose O or row sum ends non-finite repeats its pass with a check and
rescale on every tile.  These inputs place two keys in later tiles whose score
for half of the queries exceeds everything else by about 84 base-2 units (the
unchecked pass holds it: p up to ~2^80) or by about 250 (p overflows: the
exact pass must take over).  Outputs are compared with the oracle over the
whole map at the forward's bars (max abs error 2e-2 for bf16; 1e-5 for fp32
plus the rounding of two spike scores of ~175, derived in the test); the row
log-sum-exp at a bound derived from the rounding of the score operands.
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
    (1, 70, 64, 2, 30, 16, 64, 10.0, "bf16"),   # +84 base-2 units: the unchecked pass
    (1, 70, 64, 2, 30, 16, 64, 30.0, "bf16"),   # +250: overflow, exact pass
    (1, 96, 100, 1, 30, 16, 96, 30.0, "bf16"),  # 96x96 windows, ragged right column
    (1, 40, 33, 2, 16, 16, 32, 30.0, "bf16"),   # dh = 16 variant, ragged windows
    (2, 37, 40, 2, 30, 16, 16, 30.0, "bf16"),   # whole-window kernel (its own check)
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
