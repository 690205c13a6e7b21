"""GPU parity of rib_window_attn_lnq: LayerNorm and the Q projection computed inside the tiled
attention kernel (the Q side of the block's input projection fused into the attention), K and V
from rib_ln_qkv with q = NULL.

Against the oracle chain: rib_oracle_ln_qkv (fp64 q, k, v), each map rounded to bf16 (the precision
in which both GPU paths hold q, k and v), then rib_oracle_attn on those maps, at the attention's
bf16 bar (max abs error 2e-2).  The GPU accumulates the projection in fp32 before its rounding, so
an element of q, k or v can sit one bf16 unit from the oracle's rounded value; at these magnitudes
(|q|, |k| ~ 1) that moves a score by ~2^-8 and the output far less than the bar.

Against the unfused GPU path (rib_ln_qkv with q, then rib_window_attn): the fused kernel folds
LayerNorm's affine part into the weights and multiplies the raw bf16 x, where rib_ln_qkv rounds
LN(x) to bf16 first, so q can differ by about one bf16 unit; the outputs are compared at the same
2e-2.  K and V come from the same rib_ln_qkv kernel in both paths and must match bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
import super_resolution_transformer_amd as rib
from super_resolution_transformer_amd import synthetic

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    rib.lib()
    return t


CASES = [
    # B, H, W, heads, dh, ws
    (1, 37, 53, 6, 30, 16),    # 256-token windows on the tiled kernel, ragged edges
    (2, 40, 33, 6, 30, 32),    # two images, 1,024-token windows
    (1, 70, 61, 2, 30, 64),    # ragged 64x64 windows
    (1, 96, 100, 1, 30, 96),   # a 96x96 window and a 4-column window (18 query blocks)
    (1, 40, 41, 3, 16, 24),    # dh = 16 variant
    (1, 9, 11, 6, 30, 8),      # small windows, C = 180 (the last 16-channel step is partial)
]


def run_case(torch, B, H, W, heads, dh, ws, seed):
    C = heads * dh
    lp = synthetic.make_ln_qkv_problem(B, H, W, C, "bf16", seed=seed)
    ap = synthetic.make_problem(B, H, W, heads, dh, 16, dtype="bf16", seed=seed + 1)
    x = torch.from_numpy(lp.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    prm = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (lp.gamma, lp.beta, lp.w, lp.bias)]
    g = torch.from_numpy(ap.bits["g"].view(np.int16)).view(torch.bfloat16).cuda()
    qp, kp = rib.encode(ws, ap.L, ap.hidden, ap.R, torch.from_numpy(ap.weights).cuda())
    k, v = torch.empty_like(x), torch.empty_like(x)
    rib.ln_qkv_into(x, *prm, None, k, v)
    o = rib.window_attn_lnq(x, *prm, k, v, g, qp, kp, heads, ws)
    q2, k2, v2 = (torch.empty_like(x) for _ in range(3))
    rib.ln_qkv_into(x, *prm, q2, k2, v2)
    o2 = rib.window_attn(q2, k2, v2, g, qp, kp, heads, ws)
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16), k2.view(torch.int16)) and torch.equal(v.view(torch.int16), v2.view(torch.int16))
    return lp, ap, o.float().cpu().numpy().astype(np.float64), o2.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,H,W,heads,dh,ws", CASES)
def test_fused_q_matches_oracle_chain(torch, B, H, W, heads, dh, ws):
    note(f"lnq B={B} H={H} W={W} heads={heads} dh={dh} ws={ws}")
    lp, ap, got, unfused = run_case(torch, B, H, W, heads, dh, ws, seed=H + W + ws)
    assert np.all(np.isfinite(got))
    q, k, v = (synthetic.round_bf16(a.astype(np.float32))[1] for a in oracle.ln_qkv(lp.x, lp.gamma, lp.beta, lp.w, lp.bias))
    oq, ok = oracle.encode(ws, ap.L, ap.hidden, ap.R, ap.weights)
    want = oracle.window_attn(q, k, v, ap.g, oq, ok, heads, ws)
    err = float(np.abs(got - want).max())
    err2 = float(np.abs(got - unfused).max())
    note(f"  max|err| vs oracle {err:.3g}, vs unfused GPU path {err2:.3g}, max|O| {float(np.abs(want).max()):.3g}")
    assert err <= 2e-2
    assert err2 <= 2e-2


def test_fused_q_locality(torch):
    """Changing one token of x changes the output only inside that token's window (bit-exact elsewhere);
    k and v are held fixed, so the change reaches the output only through the fused Q."""
    B, H, W, heads, dh, ws = 1, 48, 48, 6, 30, 16
    lp = synthetic.make_ln_qkv_problem(B, H, W, heads * dh, "bf16", seed=5)
    ap = synthetic.make_problem(B, H, W, heads, dh, 16, dtype="bf16", seed=6)
    x = torch.from_numpy(lp.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    prm = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (lp.gamma, lp.beta, lp.w, lp.bias)]
    g = torch.from_numpy(ap.bits["g"].view(np.int16)).view(torch.bfloat16).cuda()
    qp, kp = rib.encode(ws, ap.L, ap.hidden, ap.R, torch.from_numpy(ap.weights).cuda())
    k, v = torch.empty_like(x), torch.empty_like(x)
    rib.ln_qkv_into(x, *prm, None, k, v)
    base = rib.window_attn_lnq(x, *prm, k, v, g, qp, kp, heads, ws)
    x2 = x.clone()
    x2[0, 20, 37] += 1.5
    out = rib.window_attn_lnq(x2, *prm, k, v, g, qp, kp, heads, ws)
    changed = (out.view(torch.int16) != base.view(torch.int16)).any(dim=-1).cpu().numpy()
    assert changed[0, 20, 37] and changed.sum() == 1   # only that query's own row: Q is per token


@pytest.mark.parametrize("B,H,W", [(32, 96, 96), (1, 360, 640)], ids=["32x96x96", "1x360x640"])
def test_fused_q_full_size(torch, B, H, W):
    """The 96x96-window workloads at full size, in the launch bench.py times (C = 180, 6 heads):
    - the whole output against the unfused GPU path (rib_ln_qkv + rib_window_attn, itself compared
      with the oracle over whole outputs at these sizes) at 2e-2;
    - sampled rows of two windows (the first window of the first image, the bottom-right window
      of the last image: full, or ragged at 72x64) against the oracle chain, run on the window's
      own region of x (LayerNorm and the projection act per token, so the region is exact)."""
    heads, dh, ws = 6, 30, 96
    C = heads * dh
    note(f"lnq full size B={B} H={H} W={W}")
    lp = synthetic.make_ln_qkv_problem(B, H, W, C, "bf16", seed=11)
    gp = synthetic.make_gate_problem(B, H, W, C, "bf16", seed=12)     # its X serves as the gate map G
    ap = synthetic.make_problem(1, 8, 8, heads, dh, 16, dtype="bf16", seed=13)
    x = torch.from_numpy(lp.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    g = torch.from_numpy(gp.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    prm = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (lp.gamma, lp.beta, lp.w, lp.bias)]
    qp, kp = rib.encode(ws, ap.L, ap.hidden, ap.R, torch.from_numpy(ap.weights).cuda())
    k, v = torch.empty_like(x), torch.empty_like(x)
    rib.ln_qkv_into(x, *prm, None, k, v)
    got = rib.window_attn_lnq(x, *prm, k, v, g, qp, kp, heads, ws)
    q2 = torch.empty_like(x)
    rib.ln_qkv_into(x, *prm, q2, k, v)
    ref = rib.window_attn(q2, k, v, g, qp, kp, heads, ws)
    torch.cuda.synchronize()
    err_gpu = float((got.float() - ref.float()).abs().max())
    note(f"  whole output vs unfused GPU path: max|err| {err_gpu:.3g}")
    assert err_gpu <= 2e-2
    got = got.float().cpu().numpy().astype(np.float64)
    del x, g, k, v, q2, ref
    torch.cuda.empty_cache()
    oq, ok = oracle.encode(ws, ap.L, ap.hidden, ap.R, ap.weights)
    rng = np.random.default_rng(B + H)
    for b, wy, wx in ((0, 0, 0), (B - 1, (H - 1) // ws, (W - 1) // ws)):
        y0, x0 = wy * ws, wx * ws
        y1, x1 = min(H, y0 + ws), min(W, x0 + ws)
        reg = lambda a: np.ascontiguousarray(a[b:b + 1, y0:y1, x0:x1])
        q, kk, vv = (synthetic.round_bf16(a.astype(np.float32))[1]
                     for a in oracle.ln_qkv(reg(lp.x), lp.gamma, lp.beta, lp.w, lp.bias))
        hh, ww = y1 - y0, x1 - x0
        ty = np.concatenate([[0, 0, hh - 1, hh - 1], rng.integers(0, hh, 60)])
        tx = np.concatenate([[0, ww - 1, 0, ww - 1], rng.integers(0, ww, 60)])
        want = oracle.window_attn_rows(q, kk, vv, reg(gp.x), oq, ok, heads, ws, np.zeros_like(ty), ty, tx)
        err = float(np.abs(got[b, y0 + ty, x0 + tx] - want).max())
        note(f"  image {b} window ({wy},{wx}) {hh}x{ww}: 64 rows, max|err| vs oracle {err:.3g}")
        assert err <= 2e-2
