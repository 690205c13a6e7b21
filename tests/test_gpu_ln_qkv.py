"""GPU parity of the block input projection (rib_ln_qkv: LayerNorm, then x W + b into Q | K | V),
through the C ABI, against the fp64 oracle.

Bounds derived from the arithmetic (as for the gate producer).  bf16 keeps an 8-bit significand:
round-to-nearest has relative error <= u = 2^-8.
- bf16 maps: LayerNorm runs in fp32 on the exact bf16 inputs (relative error ~1e-6); xn and W are
  each rounded to bf16 before an fp32-accumulated product, so a term carries at most
  (2u + u^2) |xn_c W_co| < 2^-7 |xn_c W_co|, and the output is rounded (<= u).  Per element
  |err| <= 2^-7 S + 2^-8 |y| + 1e-5 with S = |xn| |W| + |b| (the product on absolute values, from
  the oracle's xn).  xn itself is the fp32 LayerNorm rounded once: |err| <= 2^-8 |xn| + 1e-5 (1 + |xn|).
- fp32 maps: a length-C fp32 dot product, |err| <= (C + 8) * 2^-24 * (S + |y|) + 1e-6.
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


def run(torch, p, eps, with_xn):
    if p.dtype == "bf16":
        x = torch.from_numpy(p.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(p.x).cuda()
    w = [torch.from_numpy(a).cuda() for a in (p.gamma, p.beta, p.w, p.bias)]
    outs = rib.ln_qkv(x, *w, eps=eps, with_xn=with_xn)
    torch.cuda.synchronize()
    return [o.float().cpu().numpy().astype(np.float64) for o in outs]


def check(torch, p, eps=1e-5, with_xn=True, what=""):
    got = run(torch, p, eps, with_xn)
    q, k, v, xn = oracle.ln_qkv(p.x, p.gamma, p.beta, p.w, p.bias, eps, with_xn=True)
    C = p.x.shape[-1]
    S = np.abs(xn) @ np.abs(p.w.astype(np.float64)) + np.abs(p.bias.astype(np.float64))
    worst = 0.0
    for part, (g, want) in enumerate(zip(got[:3], (q, k, v))):
        Sp = S[..., part * C:(part + 1) * C]
        if p.dtype == "bf16":
            bound = 2.0 ** -7 * Sp + 2.0 ** -8 * np.abs(want) + 1e-5
        else:
            bound = (C + 8) * 2.0 ** -24 * (Sp + np.abs(want)) + 1e-6
        assert np.all(np.isfinite(g))
        worst = max(worst, float((np.abs(g - want) / bound).max()))
    if with_xn:
        if p.dtype == "bf16":
            bound = 2.0 ** -8 * np.abs(xn) + 1e-5 * (1.0 + np.abs(xn))
        else:
            bound = (C + 8) * 2.0 ** -24 * np.abs(xn) + 1e-5
        worst = max(worst, float((np.abs(got[3] - xn) / bound).max()))
    note(f"  {what} max err/bound {worst:.3f}")
    assert worst <= 1.0, what


CASES = [
    # (B, H, W, C, dtype)
    (1, 5, 7, 180, "bf16"),     # 35 tokens: one full tile and a 3-token tail
    (2, 16, 16, 48, "bf16"),    # SST-lite width
    (1, 3, 11, 4, "bf16"),      # one 32-channel step, 12 outputs
    (1, 33, 1, 192, "bf16"),    # widest matrix-core shape
    (1, 9, 9, 96, "bf16"),      # 3 steps
    (1, 4, 8, 160, "bf16"),     # 5 steps, exact tiles
    (1, 4, 5, 194, "bf16"),     # plain kernel, bf16 storage (C > 192)
    (1, 4, 5, 6, "bf16"),       # plain kernel, bf16 storage (C % 4 != 0)
    (1, 6, 7, 180, "f32"),
    (2, 3, 5, 7, "f32"),
    (1, 2, 3, 256, "f32"),
    (1, 1, 1, 1, "f32"),        # one token, one channel: xn = beta
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}W{}C{}-{}".format(*c))
def test_ln_qkv_whole_output(torch, case):
    B, H, W, C, dtype = case
    note(f"ln_qkv {case}")
    p = synthetic.make_ln_qkv_problem(B, H, W, C, dtype, seed=B + H + W + C)
    check(torch, p, what=str(case))


def test_ln_qkv_without_xn_and_other_eps(torch):
    p = synthetic.make_ln_qkv_problem(1, 7, 9, 180, "bf16", seed=9)
    check(torch, p, eps=1e-6, with_xn=False, what="no xn, eps 1e-6")
    check(torch, p, eps=0.0, with_xn=True, what="eps 0")


@pytest.mark.parametrize("shape", [(32, 96, 96, 180), (1, 180, 320, 48), (1, 360, 640, 180)],
                         ids=["32x96x96x180", "1x180x320x48", "1x360x640x180"])
def test_ln_qkv_full_size(torch, shape):
    """The workloads' full maps, whole output, in the launch configuration the benchmark times."""
    note(f"ln_qkv full size {shape}")
    p = synthetic.make_ln_qkv_problem(*shape, "bf16", seed=11)
    check(torch, p, what=str(shape))


def test_ln_qkv_feeds_the_attention(torch):
    """rib_ln_qkv's q, k, v go straight into rib_window_attn (bf16), against the oracle chain."""
    B, H, W, heads, dh, ws = 1, 40, 33, 6, 30, 32
    C = heads * dh
    p = synthetic.make_ln_qkv_problem(B, H, W, C, "bf16", seed=21)
    x = torch.from_numpy(p.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    w = [torch.from_numpy(a).cuda() for a in (p.gamma, p.beta, p.w, p.bias)]
    q, k, v, xn = rib.ln_qkv(x, *w, with_xn=True)
    g = xn  # any map works as the gate input here
    ap = synthetic.make_problem(1, 2, 2, heads, dh, 16, dtype="f32", seed=22)  # encoder weights only
    wt = torch.from_numpy(ap.weights).cuda()
    qp, kp = rib.encode(ws, ap.L, ap.hidden, ap.R, wt)
    o = rib.window_attn(q, k, v, g, qp, kp, heads, ws).float().cpu().numpy()
    torch.cuda.synchronize()
    maps = [t.float().cpu().numpy().astype(np.float64) for t in (q, k, v, g)]  # the GPU's own bf16 operands
    oq, ok = oracle.encode(ws, ap.L, ap.hidden, ap.R, ap.weights)
    want = oracle.window_attn(*maps, oq, ok, heads, ws)
    err = float(np.abs(o - want).max())
    note(f"  chain max|err| {err:.3g}")
    assert err <= 2e-2
