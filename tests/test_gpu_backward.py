"""GPU parity of the backward pass, called through the C ABI, against the fp64 oracle.

The GPU side runs its own training forward (rib_window_attn_train) for O and
the row log-sum-exp, then rib_window_attn_backward; the oracle differentiates its exact forward.  Every
gradient is compared over its whole extent with

    max |got - ref| <= tol * max |ref|      (tol 1e-5 fp32, 2e-2 bf16)

normalised by the tensor's largest entry: gradient entries are sums in which
rows of dS cancel exactly (each row of dS sums to zero), so a fixed absolute
bound would be meaningless across shapes, and the forward's bound (1e-5, 2e-2
on outputs of order one) is applied on the tensor's own scale.  bf16 storage
adds the rounding of dA = dO * sigmoid(G), of O (which enters D = dO . O) and
of every stored gradient, each 2^-9 relative.
"""
import sys

import numpy as np
import pytest

import oracle
import super_resolution_transformer_amd as rib
from super_resolution_transformer_amd import synthetic

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
NAMES = ("dqc", "dkc", "dv", "dg", "dqp", "dkp")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    rib.lib()
    return t


def dev(torch, vals, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(vals, np.float32)).cuda()


def gpu_backward(torch, p, ws, dout_vals, dout_bits):
    maps = [dev(torch, getattr(p, nm), p.bits.get(nm), p.dtype) for nm in ("qc", "kc", "v", "g")]
    w = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, w)
    o, lse = rib.window_attn_train(*maps, qp, kp, p.heads, ws)
    dout = dev(torch, dout_vals, dout_bits, p.dtype)
    grads = rib.window_attn_backward(*maps, qp, kp, o, lse, dout, p.heads, ws)
    dw = rib.encode_backward(ws, p.L, p.hidden, p.R, w, grads[4], grads[5])
    torch.cuda.synchronize()
    out = [t.float().cpu().numpy().astype(np.float64) for t in grads]
    return out, dw.cpu().numpy().astype(np.float64)


def oracle_backward(p, ws, dout_vals):
    qp, kp = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    ref = oracle.window_attn_backward(p.qc, p.kc, p.v, p.g, qp, kp, dout_vals, p.heads, ws)
    dw = oracle.encode_backward(ws, p.L, p.hidden, p.R, p.weights, ref[4], ref[5])
    return ref, dw


def compare(got, ref, tol, what):
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    note(f"  {what}: max|err| {err:.3g}  max|ref| {scale:.3g}  ratio {err / max(scale, 1e-30):.3g}  tol {tol}")
    assert np.all(np.isfinite(got)), what
    assert err <= tol * scale, what


CASES = [
    # (B, H, W, heads, dh, R, L, hidden, ws, dtype)
    (1, 16, 16, 2, 16, 16, 10, 64, 16, "f32"),     # one exact window, one row block
    (2, 21, 13, 2, 16, 16, 10, 64, 8, "f32"),      # ragged edge windows on both axes
    (1, 24, 24, 1, 30, 16, 10, 64, 24, "f32"),     # 576 rows: three row blocks, ragged last one
    (1, 17, 40, 3, 7, 5, 4, 16, 17, "f32"),        # odd head shape, 289-token windows
    (2, 40, 24, 6, 30, 16, 10, 64, 16, "bf16"),    # the SST head shape, bf16 storage
    (1, 40, 33, 6, 30, 16, 10, 64, 32, "bf16"),    # ws 32 with a ragged right column
    (1, 20, 20, 2, 16, 16, 10, 64, 16, "bf16"),    # dh 16, partial windows
    (1, 20, 20, 2, 8, 8, 4, 16, 16, "bf16"),       # a head shape without matrix-core kernels (fp32 rows)
    (1, 96, 100, 1, 30, 16, 10, 64, 96, "bf16"),   # 96x96 window and a 4-column window: 18 row blocks
    (1, 70, 64, 2, 16, 16, 10, 64, 64, "bf16"),    # 64x64 windows, ragged bottom row of windows
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}W{}h{}d{}R{}ws{}-{}".format(*c[:6], c[8], c[9]))
def test_backward_whole_output(torch, case):
    B, H, W, heads, dh, R, L, hidden, ws, dtype = case
    note(f"backward {case}")
    p = synthetic.make_problem(B, H, W, heads, dh, R, L, hidden, dtype=dtype, seed=B * 7 + ws)
    dv, db = synthetic.make_upstream_grad(p.qc.shape, dtype, seed=ws + 99)
    got, gdw = gpu_backward(torch, p, ws, dv, db)
    ref, rdw = oracle_backward(p, ws, dv)
    for nm, a, b in zip(NAMES, got, ref):
        compare(a, b, TOL[dtype], nm)
    compare(gdw, rdw, TOL[dtype], "dweights")


def test_encode_backward_alone(torch):
    """The encoder's backward on its own, fp32, from the oracle's (dqp, dkp) cast to float32."""
    for (ws, L, hidden, R) in [(16, 10, 64, 16), (96, 10, 64, 16), (5, 0, 8, 4), (9, 16, 256, 64), (2, 3, 1, 1)]:
        note(f"encode backward ws={ws} L={L} hidden={hidden} R={R}")
        rng = np.random.default_rng(ws + L)
        w = synthetic.draw_weights(rng, L, hidden, R)
        gq = rng.standard_normal((ws * ws, R)).astype(np.float32)
        gk = rng.standard_normal((ws * ws, R)).astype(np.float32)
        got = rib.encode_backward(ws, L, hidden, R, torch.from_numpy(w).cuda(), torch.from_numpy(gq).cuda(),
                                  torch.from_numpy(gk).cuda())
        torch.cuda.synchronize()
        ref = oracle.encode_backward(ws, L, hidden, R, w, gq, gk)
        compare(got.cpu().numpy().astype(np.float64), ref, 1e-5, "dweights")


def test_backward_is_linear_in_images(torch):
    """dQp and dKp of a batch equal the sum of those of its images; per-image gradients are unchanged
    by the rest of the batch (bit-exact: each image's rows go through the same kernels and the table
    reduce adds images in a fixed order only when B > 1, so compare within tolerance for the tables)."""
    p = synthetic.make_problem(3, 20, 20, 2, 16, 16, 10, 64, dtype="bf16", seed=5)
    dv, db = synthetic.make_upstream_grad(p.qc.shape, "bf16", seed=6)
    full, _ = gpu_backward(torch, p, 16, dv, db)
    tabs = [np.zeros_like(full[4]), np.zeros_like(full[5])]
    for b in range(3):
        q = synthetic.Problem(1, 20, 20, 2, 16, 16, 10, 64, "bf16", *(getattr(p, nm)[b:b + 1] for nm in
                              ("qc", "kc", "v", "g")), weights=p.weights,
                              bits={nm: p.bits[nm][b:b + 1] for nm in p.bits})
        one, _ = gpu_backward(torch, q, 16, dv[b:b + 1], db[b:b + 1])
        for k in range(4):
            assert np.array_equal(one[k][0], full[k][b]), (b, NAMES[k])
        tabs[0] += one[4]
        tabs[1] += one[5]
    for k in range(2):
        compare(full[4 + k], tabs[k], 1e-5, NAMES[4 + k] + " sum over images")


LSE_CASES = [
    (1, 64, 64, 3, 16, 16, 16, "f32"),
    (1, 21, 13, 2, 30, 16, 8, "f32"),
    (1, 40, 24, 6, 30, 16, 16, "bf16"),     # small-window kernel
    (1, 70, 33, 6, 30, 16, 32, "bf16"),     # chunked forward, ragged windows
    (1, 64, 64, 3, 16, 16, 64, "bf16"),
    (1, 100, 96, 2, 30, 16, 96, "bf16"),    # 96x96 windows, one 4-row window below
]


@pytest.mark.parametrize("case", LSE_CASES, ids=lambda c: "B{}H{}W{}h{}d{}R{}ws{}-{}".format(*c))
def test_train_forward_lse(torch, case):
    """rib_window_attn_train: O bit-identical to rib_window_attn, lse against the oracle's
    (max abs error 1e-5 fp32, 2e-2 bf16: the forward's bars, on values of order log n)."""
    B, H, W, heads, dh, R, ws, dtype = case
    note(f"train forward {case}")
    p = synthetic.make_problem(B, H, W, heads, dh, R, 10, 64, dtype=dtype, seed=ws + H)
    maps = [dev(torch, getattr(p, nm), p.bits.get(nm), p.dtype) for nm in ("qc", "kc", "v", "g")]
    w = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, w)
    o_plain = rib.window_attn(*maps, qp, kp, heads, ws)
    o, lse = rib.window_attn_train(*maps, qp, kp, heads, ws)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if dtype == "bf16" else o, o_plain.view(torch.int16) if dtype == "bf16"
                       else o_plain)
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    ref = oracle.window_lse(p.qc, p.kc, oq, ok, heads, ws)
    err = float(np.abs(lse.cpu().numpy() - ref).max())
    note(f"  lse max|err| {err:.3g}  max|lse| {float(np.abs(ref).max()):.3g}")
    assert err <= TOL[dtype]


# ---------------------------------------------------------------- one positional pair per head
HEAD_CASES = [
    # (B, H, W, heads, dh, R, ws, dtype)
    (2, 40, 24, 6, 30, 16, 16, "bf16"),     # matrix-core path, the SST head shape
    (1, 40, 33, 3, 16, 16, 32, "bf16"),     # matrix-core path, dh 16, ragged windows
    (1, 20, 20, 2, 8, 8, 16, "bf16"),       # no matrix-core variant: fp32-register rows on bf16 maps
    (2, 21, 13, 3, 16, 16, 8, "f32"),       # fp32, ragged edge windows
]


@pytest.mark.parametrize("case", HEAD_CASES, ids=lambda c: "B{}H{}W{}h{}d{}R{}ws{}-{}".format(*c))
def test_per_head_backward_whole_output(torch, case):
    """rib_window_attn_heads_train + rib_window_attn_heads_backward against the oracle with one
    (Qp, Kp) pair per head (each from its own encoder weights): every gradient, dQp and dKp per
    head, at the bars of the shared-pair tests; the lse against the oracle's per-head lse."""
    B, H, W, heads, dh, R, ws, dtype = case
    L, hidden = 10, 64
    note(f"per-head backward {case}")
    p = synthetic.make_problem(B, H, W, heads, dh, R, L, hidden, dtype=dtype, seed=B * 11 + ws)
    rng = np.random.default_rng(ws + heads)
    ws_list = [synthetic.draw_weights(rng, L, hidden, R) for _ in range(heads)]
    tabs = [oracle.encode(ws, L, hidden, R, w) for w in ws_list]
    oqp, okp = np.stack([t[0] for t in tabs]), np.stack([t[1] for t in tabs])
    dvals, dbits = synthetic.make_upstream_grad(p.qc.shape, dtype, seed=ws + 7)
    maps = [dev(torch, getattr(p, nm), p.bits.get(nm), dtype) for nm in ("qc", "kc", "v", "g")]
    gt = [rib.encode(ws, L, hidden, R, torch.from_numpy(w).cuda()) for w in ws_list]
    qp = torch.stack([t[0] for t in gt]).contiguous()
    kp = torch.stack([t[1] for t in gt]).contiguous()
    o, lse = rib.window_attn_train(*maps, qp, kp, heads, ws)
    o_plain = rib.window_attn(*maps, qp, kp, heads, ws)
    grads = rib.window_attn_backward(*maps, qp, kp, o, lse, dev(torch, dvals, dbits, dtype), heads, ws)
    torch.cuda.synchronize()
    same = torch.equal(o.view(torch.int16), o_plain.view(torch.int16)) if dtype == "bf16" else torch.equal(o, o_plain)
    assert same, "per-head train forward differs from the per-head forward"
    lref = oracle.window_lse(p.qc, p.kc, oqp, okp, heads, ws)
    lerr = float(np.abs(lse.cpu().numpy() - lref).max())
    note(f"  lse max|err| {lerr:.3g}")
    assert lerr <= TOL[dtype]
    ref = oracle.window_attn_backward(p.qc, p.kc, p.v, p.g, oqp, okp, dvals, heads, ws)
    got = [t.float().cpu().numpy().astype(np.float64) for t in grads]
    assert got[4].shape == (heads, ws * ws, R) and got[5].shape == (heads, ws * ws, R)
    for nm, a, b in zip(NAMES, got, ref):
        compare(a, b, TOL[dtype], nm)


def test_per_head_backward_with_equal_tables_matches_the_shared_pair(torch):
    """All heads holding one pair: map gradients bit-identical to rib_window_attn_backward's, and the
    per-head table gradients sum over heads to the shared ones (within fp32 summation order)."""
    ws = 16
    p = synthetic.make_problem(2, 40, 24, 6, 30, 16, 10, 64, dtype="bf16", seed=3)
    dvals, dbits = synthetic.make_upstream_grad(p.qc.shape, "bf16", seed=4)
    maps = [dev(torch, getattr(p, nm), p.bits.get(nm), "bf16") for nm in ("qc", "kc", "v", "g")]
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, torch.from_numpy(p.weights).cuda())
    qh, kh = qp.expand(6, -1, -1).contiguous(), kp.expand(6, -1, -1).contiguous()
    dout = dev(torch, dvals, dbits, "bf16")
    o, lse = rib.window_attn_train(*maps, qp, kp, 6, ws)
    oh, lseh = rib.window_attn_train(*maps, qh, kh, 6, ws)
    shared = rib.window_attn_backward(*maps, qp, kp, o, lse, dout, 6, ws)
    per = rib.window_attn_backward(*maps, qh, kh, oh, lseh, dout, 6, ws)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), oh.view(torch.int16)) and torch.equal(lse, lseh)
    for k in range(4):
        assert torch.equal(shared[k].view(torch.int16), per[k].view(torch.int16)), NAMES[k]
    for k in (4, 5):
        compare(per[k].sum(0).cpu().numpy().astype(np.float64), shared[k].cpu().numpy().astype(np.float64), 1e-5,
                NAMES[k] + " summed over heads")
