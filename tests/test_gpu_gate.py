"""GPU parity of the CLA gate producer G = PWConv1x1(DWConv3x3(X)) (rib_cla_gate, through the
C ABI) against the fp64 CPU oracle.

Tolerances: fp32 maps, max abs error <= 1e-5.  bf16 maps, derived from the arithmetic.  The bf16
kernel rounds the depth-wise taps and the point-wise weights to bf16 (nearest even) before using
them; the reference is the oracle run on those same rounded values (the biases stay fp32, as in
the kernel), so the bar covers only what the kernel rounds on top: the stencil D (fp32 sums of
exact bf16 products, then rounded to bf16: relative error <= u = 2^-8 plus 10 * 2^-24 for the
sums), the fp32 point-wise sum (<= C 2^-24 of its absolute terms) and G itself (<= u).  Per
element
    |err| <= 2^-8 (1 + 2^-7) S + 2^-8 |G| + 1e-5,   S = sum_c |D_c|_abs |W_co| + |b_o|,
where S is the oracle run on the absolute values of the inputs and of the rounded weights (the
factor 1 + 2^-7 covers 2^-20 + C 2^-24 <= 2^-16 for C <= 256 and the rounding of G's own
error).  Identity weights and locality are checked bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
import super_resolution_transformer_amd as rib
from super_resolution_transformer_amd import synthetic

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    rib.lib()
    return t


def to_dev(torch, p):
    if p.dtype == "bf16":
        x = torch.from_numpy(p.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(p.x).cuda()
    w = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (p.dw_w, p.dw_b, p.pw_w, p.pw_b)]
    return x, w


def rb(a):
    """The bf16-rounded (nearest even) values of an fp32 array, as float32."""
    return synthetic.round_bf16(np.asarray(a, dtype=np.float32))[1]


def reference(p, x=None):
    """The oracle on the weights the kernel uses: fp32 maps as given; bf16 maps with the
    depth-wise taps and point-wise weights rounded to bf16 (biases fp32)."""
    x = p.x if x is None else x
    if p.dtype == "bf16":
        return oracle.cla_gate(x, rb(p.dw_w), p.dw_b, rb(p.pw_w), p.pw_b)
    return oracle.cla_gate(x, p.dw_w, p.dw_b, p.pw_w, p.pw_b)


def abs_bound(p, x=None):
    """Upper bound of sum_c |D_c| |W_co| + |b_o| per element: the oracle on absolute values
    (of the rounded weights, for bf16 maps)."""
    x = p.x if x is None else x
    dw, pw = (rb(p.dw_w), rb(p.pw_w)) if p.dtype == "bf16" else (p.dw_w, p.pw_w)
    return oracle.cla_gate(np.abs(x), np.abs(dw), np.abs(p.dw_b), np.abs(pw), np.abs(p.pw_b))


def compare(got, want, dtype, what, S=None):
    err = np.abs(got - want)
    if dtype == "f32":
        tol = np.full_like(want, TOL["f32"])
    else:
        tol = 2.0 ** -8 * (1.0 + 2.0 ** -7) * S + 2.0 ** -8 * np.abs(want) + 1e-5
    worst = float((err / tol).max()) if err.size else 0.0
    note(f"  {what}: max|err| {float(err.max()) if err.size else 0.0:.3g}  max|G| {float(np.abs(want).max()):.3g}"
         f"  max err/tol {worst:.3f}")
    assert worst <= 1.0, what


GATE = [
    # B, H, W, C, dtype
    (2, 5, 7, 6, "f32"),
    (1, 1, 1, 4, "f32"),
    (2, 9, 40, 30, "f32"),
    (1, 6, 33, 180, "f32"),
    (2, 5, 7, 6, "bf16"),
    (1, 1, 1, 4, "bf16"),
    (1, 3, 13, 48, "bf16"),
    (2, 9, 40, 30, "bf16"),
    (1, 6, 33, 180, "bf16"),
    (1, 3, 70, 62, "bf16"),
    (1, 4, 5, 256, "bf16"),
    (2, 17, 65, 96, "bf16"),
    (2, 5, 9, 2, "bf16"),   # one channel pair: the smallest map the kernels take
    (1, 4, 33, 2, "f32"),
]


@pytest.mark.parametrize("B,H,W,C,dtype", GATE)
def test_gate_whole_output(torch, B, H, W, C, dtype):
    note(f"gate whole B={B} H={H} W={W} C={C} {dtype}")
    p = synthetic.make_gate_problem(B, H, W, C, dtype, seed=B * 1000 + H * 100 + W + C)
    x, w = to_dev(torch, p)
    g = rib.cla_gate(x, *w)
    torch.cuda.synchronize()
    want = reference(p)
    compare(g.float().cpu().numpy().astype(np.float64), want, dtype, "G", abs_bound(p) if dtype == "bf16" else None)


@pytest.mark.parametrize("B,H,W,C", [(2, 203, 90, 180), (3, 150, 70, 48)])
def test_gate_whole_output_long_ranges(torch, B, H, W, C):
    """Maps with several times more 32-token tiles than workgroups (1218 tiles at C = 180, 1350 at
    C = 48), ragged in W and H: every workgroup walks a range of tiles down the map's columns, the
    ranges start and end mid-column and cross column and image boundaries.  Whole output."""
    note(f"gate long ranges B={B} H={H} W={W} C={C}")
    p = synthetic.make_gate_problem(B, H, W, C, "bf16", seed=B + H + W + C)
    x, w = to_dev(torch, p)
    g = rib.cla_gate(x, *w)
    torch.cuda.synchronize()
    want = reference(p)
    compare(g.float().cpu().numpy().astype(np.float64), want, "bf16", "G", abs_bound(p))


@pytest.mark.parametrize("shape", [(32, 96, 96, 180), (1, 180, 320, 48), (1, 360, 640, 180)])
def test_gate_full_size_bands(torch, shape):
    """Full-size maps of the workloads; row bands (top, middle, bottom) of the first and last
    images are checked against the oracle run on the band plus its one-row halo."""
    B, H, W, C = shape
    note(f"gate full size {shape}")
    p = synthetic.make_gate_problem(B, H, W, C, "bf16", seed=H + W + C)
    x, w = to_dev(torch, p)
    g = rib.cla_gate(x, *w).float().cpu().numpy()
    for b in sorted({0, B - 1}):
        for y0 in (0, H // 2 - 3, H - 6):
            y1 = y0 + 6
            lo, hi = max(0, y0 - 1), min(H, y1 + 1)
            band = reference(p, p.x[b:b + 1, lo:hi])[0]
            S = abs_bound(p, p.x[b:b + 1, lo:hi])[0]
            compare(g[b, y0:y1].astype(np.float64), band[y0 - lo:y1 - lo], "bf16", f"image {b} rows {y0}-{y1}",
                    S[y0 - lo:y1 - lo])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_identity_weights_bit_exact(torch, dtype):
    """Centre tap 1, identity point-wise weights, zero biases: G == X bit for bit."""
    B, H, W, C = 2, 7, 37, 180
    p = synthetic.make_gate_problem(B, H, W, C, dtype, seed=3)
    x, _ = to_dev(torch, p)
    dw = torch.zeros((C, 3, 3), dtype=torch.float32, device="cuda")
    dw[:, 1, 1] = 1.0
    z = torch.zeros(C, dtype=torch.float32, device="cuda")
    eye = torch.eye(C, dtype=torch.float32, device="cuda")
    g = rib.cla_gate(x, dw, z, eye, z)
    assert torch.equal(g, x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_locality_bit_exact(torch, dtype):
    """Changing one token of X changes G only in its 3x3 neighbourhood (exactly)."""
    B, H, W, C = 2, 12, 40, 48
    p = synthetic.make_gate_problem(B, H, W, C, dtype, seed=4)
    x, w = to_dev(torch, p)
    base = rib.cla_gate(x, *w)
    x2 = x.clone()
    x2[1, 5, 31] += 2.0
    out = rib.cla_gate(x2, *w)
    changed = (out != base).any(dim=-1).cpu().numpy()
    inside = np.zeros_like(changed)
    inside[1, 4:7, 30:33] = True
    assert changed[inside].all() and not changed[~inside].any()


def test_gate_then_attention_matches_oracle_chain(torch):
    """The CLA block output: G from rib_cla_gate feeds rib_window_attn (bf16, window 16)."""
    B, H, W, heads, dh, ws = 1, 37, 53, 3, 16, 16
    p = synthetic.make_problem(B, H, W, heads, dh, dtype="bf16", seed=21)
    gp = synthetic.make_gate_problem(B, H, W, heads * dh, "bf16", seed=22)
    x, w = to_dev(torch, gp)
    g = rib.cla_gate(x, *w)
    bf = lambda nm: torch.from_numpy(p.bits[nm].view(np.int16)).view(torch.bfloat16).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, torch.from_numpy(p.weights).cuda())
    o = rib.window_attn(bf("qc"), bf("kc"), bf("v"), g, qp, kp, heads, ws).float().cpu().numpy()
    g_host = g.float().cpu().numpy()                  # the gate as the attention saw it (bf16)
    want_g = reference(gp)
    compare(g_host.astype(np.float64), want_g, "bf16", "G", abs_bound(gp))
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn(p.qc, p.kc, p.v, want_g, oq, ok, heads, ws)
    err = float(np.abs(o.astype(np.float64) - want).max())
    note(f"  O: max|err| {err:.3g} (attention bound 2e-2)")
    assert err <= 2e-2
