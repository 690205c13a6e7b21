"""GPU parity: the HIP path, called through the C ABI, against the fp64 CPU oracle.

Tolerances: max abs error <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs
with fp32 accumulation; window/index mapping (locality, equivariance, one-hot
index pins) bit-exact.  Every comparison is element by element over the whole
output: small problems, and the full-size workloads in the launch configuration
the benchmark times.
"""
import math
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


def to_dev(torch, p):
    if p.dtype == "bf16":
        cv = lambda nm: torch.from_numpy(p.bits[nm].view(np.int16)).view(torch.bfloat16).cuda()
    else:
        cv = lambda nm: torch.from_numpy(getattr(p, nm)).cuda()
    return [cv(nm) for nm in ("qc", "kc", "v", "g")], torch.from_numpy(p.weights).cuda()


def gpu_run(torch, p, ws):
    (qc, kc, v, g), w = to_dev(torch, p)
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, w)
    o = rib.window_attn(qc, kc, v, g, qp, kp, p.heads, ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), qp.cpu().numpy(), kp.cpu().numpy()


def compare(got, want, dtype, what):
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    note(f"  {what}: max|err| {mx:.3g}  max|O| {float(np.abs(want).max()):.3g}  tol {TOL[dtype]}")
    assert np.all(np.isfinite(got)), what
    assert mx <= TOL[dtype], what


# ---------------------------------------------------------------- encoder
@pytest.mark.parametrize("ws", [2, 3, 4, 7, 16, 32, 64, 96, 128])
def test_encode_matches_oracle(torch, ws):
    p = synthetic.config_problem(3)
    note(f"encode ws={ws}")
    w = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, w)
    torch.cuda.synchronize()
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    for got, want in ((qp, oq), (kp, ok)):
        e = np.abs(got.cpu().numpy() - want).max()
        note(f"  max|err| {e:.3g}")
        assert e <= 1e-5


def test_encode_other_sizes(torch):
    for (L, hidden, R, ws) in [(0, 8, 4, 5), (15, 32, 8, 16), (16, 256, 64, 9), (3, 1, 1, 2)]:
        note(f"encode L={L} hidden={hidden} R={R} ws={ws}")
        w = synthetic.draw_weights(np.random.default_rng(L), L, hidden, R)
        qp, kp = rib.encode(ws, L, hidden, R, torch.from_numpy(w).cuda())
        oq, ok = oracle.encode(ws, L, hidden, R, w)
        assert np.abs(qp.cpu().numpy() - oq).max() <= 1e-5
        assert np.abs(kp.cpu().numpy() - ok).max() <= 1e-5


# ---------------------------------------------------------------- whole outputs, small shapes
SMALL = [
    # B, H, W, heads, dh, R, ws, dtype
    (1, 64, 64, 3, 16, 16, 16, "f32"),        # tiny fp32 workload, whole
    (1, 5, 7, 1, 16, 16, 2, "f32"),
    (2, 37, 53, 3, 30, 16, 16, "f32"),
    (1, 20, 30, 2, 7, 5, 8, "f32"),
    (1, 9, 70, 1, 64, 64, 32, "f32"),
    (1, 5, 7, 1, 16, 16, 4, "bf16"),
    (1, 5, 7, 2, 16, 16, 96, "bf16"),          # window larger than the map
    (3, 37, 53, 3, 30, 16, 16, "bf16"),
    (1, 37, 53, 3, 30, 16, 32, "bf16"),
    (2, 37, 53, 2, 32, 16, 32, "bf16"),
    (1, 100, 61, 2, 16, 16, 64, "bf16"),
    (1, 70, 61, 1, 30, 16, 96, "bf16"),
    (1, 30, 31, 2, 8, 8, 8, "bf16"),
    (1, 30, 31, 2, 16, 32, 16, "bf16"),
    (1, 30, 31, 2, 30, 32, 16, "bf16"),
    (1, 1, 1, 2, 30, 16, 2, "bf16"),           # a window with one token
    (1, 1, 100, 1, 30, 16, 16, "bf16"),
    (1, 3, 130, 1, 16, 16, 128, "bf16"),       # largest window
    (2, 21, 19, 2, 32, 16, 16, "bf16"),        # whole-window kernel, (32, 16) variant
    (1, 16, 16, 1, 30, 16, 16, "bf16"),        # exactly one full 16x16 window
    (2, 17, 33, 3, 16, 16, 16, "bf16"),        # one-row bottom windows
    (1, 40, 41, 1, 16, 16, 17, "bf16"),        # 289 tokens: chunked kernel, two key chunks, one real query in a wave
    (1, 50, 47, 2, 30, 16, 45, "bf16"),        # 2,025 tokens: eight chunks, the last one ragged
    (1, 45, 50, 2, 8, 8, 24, "bf16"),          # chunked kernel, (8, 8) variant
    (1, 30, 31, 2, 16, 32, 32, "bf16"),        # chunked kernel, (16, 32) variant
    (1, 50, 47, 1, 30, 16, 46, "bf16"),        # 2,116 tokens: chunked, 4 windows dealt to the XCDs by unit
    (1, 50, 47, 1, 30, 32, 46, "bf16"),        # 2,116 tokens, (30, 32): the tiled kernel
    (1, 70, 61, 1, 32, 16, 96, "bf16"),        # (32, 16) at 96x96: the tiled kernel
    (1, 100, 61, 2, 16, 32, 64, "bf16"),       # (16, 32) at 64x64, grid resident at once: chunked
]


@pytest.mark.parametrize("B,H,W,heads,dh,R,ws,dtype", SMALL)
def test_attention_whole_output(torch, B, H, W, heads, dh, R, ws, dtype):
    note(f"attn whole B={B} H={H} W={W} heads={heads} dh={dh} R={R} ws={ws} {dtype}")
    p = synthetic.make_problem(B, H, W, heads, dh, R, dtype=dtype, seed=H * 1000 + W + ws)
    got, qp, kp = gpu_run(torch, p, ws)
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, heads, ws)
    compare(got, want, dtype, "O")


def test_sst_lite_cyclic_windows_whole_16(torch):
    """The SST-lite workload (180x320, C=48, 3 heads) at window 16, whole output."""
    p = synthetic.config_problem(2)
    got, _, _ = gpu_run(torch, p, 16)
    oq, ok = oracle.encode(16, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, p.heads, 16)
    compare(got, want, "bf16", "sst-lite ws16")


# ---------------------------------------------------------------- full-size workloads, whole outputs
@pytest.mark.parametrize("cfg,ws", [(2, 32), (2, 64), (3, 64), (5, 96), (4, 96)])
def test_full_size_workload_whole(torch, cfg, ws):
    """Every output of the full-size workloads, in the launch configuration the benchmark times
    (the 180x320 maps at 32x32 and 64x64 windows, C = 48 and 180; the 640x360 input and the
    32 x 96x96 training batch at 96x96 windows), against the threaded fp64 oracle: every image,
    window, head and query block, edge windows included.  The oracle takes about a minute for
    the 32 x 96x96 batch on 16 cores."""
    p = synthetic.config_problem(cfg)
    note(f"workload {synthetic.CONFIGS[cfg].name} ws={ws}: B={p.B} H={p.H} W={p.W} C={p.C} (whole output)")
    got, _, _ = gpu_run(torch, p, ws)
    assert np.all(np.isfinite(got))
    oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
    want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, p.heads, ws)
    compare(got, want, p.dtype, f"{got.size} outputs")


# ---------------------------------------------------------------- bit-exact index pins
def one_hot_inputs(ws, H, W, B, heads, dh, alpha=32.0, seed=3):
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
    return qc, v, g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ws,H,W", [(2, 5, 7), (4, 9, 6), (4, 8, 8), (4, 13, 11)])
def test_one_hot_index_mapping_is_bit_exact(torch, dtype, ws, H, W):
    note(f"one-hot ws={ws} H={H} W={W} {dtype}")
    B, heads, dh, R = 2, 2, 16, 16
    qc, v, g = one_hot_inputs(ws, H, W, B, heads, dh)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    qct, vt, gt = (torch.from_numpy(a).cuda().to(tdt) for a in (qc, v, g))
    z = torch.zeros((ws * ws, R), dtype=torch.float32, device="cuda")
    o = rib.window_attn(qct, qct, vt, gt, z, z, heads, ws)
    assert torch.equal(o, vt)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ws,H,W,R,dh", [(4, 4, 4, 16, 16), (4, 9, 6, 16, 30), (2, 5, 7, 16, 16),
                                         (5, 11, 8, 32, 16), (4, 7, 9, 32, 30)])
def test_positional_one_hot_is_bit_exact(torch, dtype, ws, H, W, R, dh):
    """Qc = Kc = 0 and Qp = Kp = alpha * I (R >= window^2): the bias alone makes P one-hot on
    the diagonal, so O == V bit for bit -- pins the positional columns and their indexing."""
    note(f"positional one-hot ws={ws} H={H} W={W} R={R} dh={dh} {dtype}")
    B, heads = 2, 2
    if dtype == "bf16" and not rib.supported(dh, R, ws, torch.bfloat16):
        pytest.skip("no bf16 variant")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(1)
    v = synthetic.round_bf16(rng.standard_normal((B, H, W, heads * dh)).astype(np.float32) + 3.0)[1]
    vt = torch.from_numpy(v).cuda().to(tdt)
    z = torch.zeros_like(vt)
    g = torch.full_like(vt, 100.0)
    eye = torch.zeros((ws * ws, R), dtype=torch.float32, device="cuda")
    eye[torch.arange(ws * ws), torch.arange(ws * ws)] = 32.0
    o = rib.window_attn(z, z, vt, g, eye, eye, heads, ws)
    assert torch.equal(o, vt)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ws", [16, 32, 48])
def test_locality_and_equivariance_bit_exact(torch, dtype, ws):
    """Window 16 runs the whole-window bf16 kernel, window 32 the chunked one with whole windows dealt
    to the XCDs, window 48 (2,304 tokens, 18 windows) the chunked one dealt by window unit."""
    note(f"locality ws={ws} {dtype}")
    H, W, B, heads, dh, R = 3 * ws, 3 * ws, 2, 3, 30 if dtype == "bf16" else 16, 16
    p = synthetic.make_problem(B, H, W, heads, dh, R, dtype=dtype, seed=7)
    (qc, kc, v, g), w = to_dev(torch, p)
    qp, kp = rib.encode(ws, p.L, p.hidden, R, w)
    base = rib.window_attn(qc, kc, v, g, qp, kp, heads, ws)
    kc2, v2 = kc.clone(), v.clone()
    ty, tx = ws + ws // 4, 2 * ws + ws // 3  # a token of window (1, 2)
    kc2[1, ty, tx] += 1.5
    v2[1, ty, tx] -= 2.0
    out = rib.window_attn(qc, kc2, v2, g, qp, kp, heads, ws)
    changed = (out != base).any(dim=-1).cpu().numpy()
    inside = np.zeros_like(changed)
    inside[1, ws:2 * ws, 2 * ws:3 * ws] = True
    assert changed[inside].mean() > 0.9 and not changed[~inside].any()

    def swap(a):
        a = a.clone()
        t = a[:, 0:ws, ws:2 * ws].clone()
        a[:, 0:ws, ws:2 * ws] = a[:, 2 * ws:3 * ws, 0:ws]
        a[:, 2 * ws:3 * ws, 0:ws] = t
        return a
    out = rib.window_attn(swap(qc), swap(kc), swap(v), swap(g), qp, kp, heads, ws)
    assert torch.equal(out, swap(base))
    same = [torch.stack([a[0], a[0]]).contiguous() for a in (qc, kc, v, g)]
    out = rib.window_attn(*same, qp, kp, heads, ws)
    assert torch.equal(out[0], out[1]) and torch.equal(out[0], base[0])


def test_repeat_calls_are_deterministic(torch):
    p = synthetic.make_problem(1, 96, 96, 6, 30, 16, dtype="bf16", seed=9)
    (qc, kc, v, g), w = to_dev(torch, p)
    qp, kp = rib.encode(96, p.L, p.hidden, p.R, w)
    a = rib.window_attn(qc, kc, v, g, qp, kp, 6, 96)
    b = rib.window_attn(qc, kc, v, g, qp, kp, 6, 96)
    assert torch.equal(a, b)


def test_unsupported_shape_raises(torch):
    x = torch.zeros((1, 8, 8, 2 * 31), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(rib.RibError) as e:
        rib.window_attn(x, x, x, x, z, z, 2, 8)
    assert e.value.status == rib.RIB_ERR_UNSUPPORTED


# ---------------------------------------------------------------- per-head positional tables
@pytest.mark.parametrize("B,H,W,heads,dh,R,ws,dtype", [
    (1, 20, 30, 3, 16, 16, 8, "f32"),
    (2, 37, 53, 3, 30, 16, 16, "bf16"),     # whole-window kernel
    (1, 37, 53, 2, 30, 16, 32, "bf16"),     # chunked kernel
    (1, 30, 31, 2, 16, 32, 16, "bf16"),
    (1, 70, 61, 2, 30, 32, 64, "bf16"),
])
def test_per_head_tables_whole_output(torch, B, H, W, heads, dh, R, ws, dtype):
    """rib_window_attn_heads: one (Qp, Kp) pair per head, each from rib_encode with its own weights."""
    note(f"per-head tables B={B} H={H} W={W} heads={heads} dh={dh} R={R} ws={ws} {dtype}")
    p = synthetic.make_problem(B, H, W, heads, dh, R, dtype=dtype, seed=H * 7 + W + ws)
    (qc, kc, v, g), _ = to_dev(torch, p)
    ws_h = [synthetic.draw_weights(np.random.default_rng(100 + h), p.L, p.hidden, R) for h in range(heads)]
    tabs = [rib.encode(ws, p.L, p.hidden, R, torch.from_numpy(w).cuda()) for w in ws_h]
    qp = torch.stack([t[0] for t in tabs]).contiguous()
    kp = torch.stack([t[1] for t in tabs]).contiguous()
    o = rib.window_attn(qc, kc, v, g, qp, kp, heads, ws)
    torch.cuda.synchronize()
    oq = np.stack([oracle.encode(ws, p.L, p.hidden, R, w)[0] for w in ws_h])
    ok = np.stack([oracle.encode(ws, p.L, p.hidden, R, w)[1] for w in ws_h])
    want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, heads, ws)
    compare(o.float().cpu().numpy().astype(np.float64), want, dtype, "O")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ws,dh", [(4, 16), (4, 30)])
def test_per_head_positional_permutation_is_bit_exact(torch, dtype, ws, dh):
    """Qc = Kc = 0; head h's tables are Qp[n] = a e_n, Kp[m] = a e_{(m + h + 1) mod N}, so query n
    of head h attends only to key m = (n - h - 1) mod N of its window: O == V moved by a per-head
    in-window shift, bit for bit (also pins that head h reads table h)."""
    B, H, W, heads, R = 2, 2 * ws, 3 * ws, 3, 16
    N = ws * ws
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(2)
    v = synthetic.round_bf16(rng.standard_normal((B, H, W, heads * dh)).astype(np.float32) + 3.0)[1]
    vt = torch.from_numpy(v).cuda().to(tdt)
    z = torch.zeros_like(vt)
    g = torch.full_like(vt, 100.0)
    qp = torch.zeros((heads, N, R), dtype=torch.float32, device="cuda")
    kp = torch.zeros_like(qp)
    for h in range(heads):
        qp[h, torch.arange(N), torch.arange(N)] = 32.0
        kp[h, torch.arange(N), (torch.arange(N) + h + 1) % N] = 32.0
    o = rib.window_attn(z, z, vt, g, qp, kp, heads, ws).cpu()
    want = torch.empty_like(o)
    vc = vt.cpu()
    for h in range(heads):
        sl = slice(h * dh, (h + 1) * dh)
        for y in range(H):
            for x in range(W):
                n = (y % ws) * ws + (x % ws)
                m = (n - h - 1) % N
                ky, kx = (y // ws) * ws + m // ws, (x // ws) * ws + m % ws
                want[:, y, x, sl] = vc[:, ky, kx, sl]
    assert torch.equal(o, want)
