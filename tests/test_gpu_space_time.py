"""GPU parity of the space-time (video) variant: rib_encode3d and rib_window_attn3d through the C ABI,
against the fp64 oracle (max abs error <= 1e-5 fp32, <= 2e-2 bf16, the bars of the image path), plus
bit-exact equivalences with the image path."""
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


def video_problem(B, T, H, W, heads, dh, dtype, seed):
    """Video maps [B, T, H, W, C]: the image problem of B*T frames, regrouped."""
    p = synthetic.make_problem(B * T, H, W, heads, dh, 16, dtype=dtype, seed=seed)
    shape = (B, T, H, W, heads * dh)
    maps = {nm: getattr(p, nm).reshape(shape) for nm in ("qc", "kc", "v", "g")}
    bits = {nm: p.bits[nm].reshape(shape) for nm in p.bits}
    return maps, bits


def to_dev(torch, maps, bits, dtype):
    if dtype == "bf16":
        return [torch.from_numpy(np.ascontiguousarray(bits[n]).view(np.int16)).view(torch.bfloat16).cuda()
                for n in ("qc", "kc", "v", "g")]
    return [torch.from_numpy(np.ascontiguousarray(maps[n])).cuda() for n in ("qc", "kc", "v", "g")]


def weights3d(L, hidden, R, seed):
    rng = np.random.default_rng(seed)
    F = 3 + 6 * L
    return np.concatenate([rng.standard_normal(F * hidden) / np.sqrt(F), rng.standard_normal(hidden) / np.sqrt(F),
                           rng.standard_normal(2 * hidden * R) / np.sqrt(hidden)]).astype(np.float32)


@pytest.mark.parametrize("wt,ws,L", [(1, 16, 10), (2, 16, 10), (4, 8, 10), (3, 17, 15), (8, 32, 10)])
def test_encode3d_matches_oracle(torch, wt, ws, L):
    note(f"encode3d wt={wt} ws={ws} L={L}")
    w = weights3d(L, 64, 16, wt * ws)
    qp, kp = rib.encode3d(wt, ws, L, 64, 16, torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    oq, ok = oracle.encode3d(wt, ws, L, 64, 16, w)
    for got, want in ((qp, oq), (kp, ok)):
        err = float(np.abs(got.cpu().numpy() - want).max())
        note(f"  max|err| {err:.3g}")
        assert err <= 1e-5



@pytest.mark.parametrize("wt,ws,L,hidden,R", [(2, 5, 16, 256, 64), (3, 4, 0, 1, 1)])
def test_encode3d_other_widths(torch, wt, ws, L, hidden, R):
    """The widest layers (weights too large to stage in LDS) and the narrowest."""
    note(f"encode3d wt={wt} ws={ws} L={L} hidden={hidden} R={R}")
    w = weights3d(L, hidden, R, 7)
    qp, kp = rib.encode3d(wt, ws, L, hidden, R, torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    oq, ok = oracle.encode3d(wt, ws, L, hidden, R, w)
    for got, want in ((qp, oq), (kp, ok)):
        err = float(np.abs(got.cpu().numpy() - want).max())
        note(f"  max|err| {err:.3g}")
        assert err <= 1e-5

CASES = [
    # (B, T, H, W, heads, dh, wt, ws, dtype)
    (1, 5, 9, 7, 2, 30, 2, 4, "bf16"),      # small kernel (32 tokens), ragged on every axis
    (1, 3, 20, 18, 2, 30, 2, 16, "bf16"),   # chunked kernel, 512-token windows, ragged
    (1, 4, 16, 16, 3, 16, 4, 8, "bf16"),    # 256 tokens: small kernel, dh 16
    (2, 3, 17, 20, 1, 30, 3, 17, "bf16"),   # 867 tokens: two query blocks, 14 key tiles with frame crossings
    (1, 7, 12, 12, 2, 16, 4, 16, "bf16"),   # 1024-token windows, a one-frame window at the end
    (1, 5, 9, 7, 2, 16, 2, 4, "f32"),
    (1, 3, 11, 10, 2, 7, 3, 8, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}H{}W{}h{}d{}wt{}ws{}-{}".format(*c))
def test_attn3d_whole_output(torch, case):
    B, T, H, W, heads, dh, wt, ws, dtype = case
    note(f"attn3d {case}")
    maps, bits = video_problem(B, T, H, W, heads, dh, dtype, seed=T * 10 + ws)
    w = weights3d(10, 64, 16, ws + wt)
    qp, kp = rib.encode3d(wt, ws, 10, 64, 16, torch.from_numpy(w).cuda())
    o = rib.window_attn3d(*to_dev(torch, maps, bits, dtype), qp, kp, heads, wt, ws)
    torch.cuda.synchronize()
    oq, ok = oracle.encode3d(wt, ws, 10, 64, 16, w)
    want = oracle.window_attn3d(maps["qc"], maps["kc"], maps["v"], maps["g"], oq, ok, heads, wt, ws)
    err = float(np.abs(o.float().cpu().numpy() - want).max())
    note(f"  max|err| {err:.3g}  tol {TOL[dtype]}")
    assert np.isfinite(err) and err <= TOL[dtype]


@pytest.mark.parametrize("dtype,ws", [("bf16", 16), ("bf16", 32), ("f32", 8)])
def test_one_frame_video_is_the_image_path(torch, dtype, ws):
    """T = 1, one-frame windows: rib_window_attn3d equals rib_window_attn bit for bit; and with one-frame
    windows over T frames, every frame equals its own image call."""
    heads, dh = 2, 30 if dtype == "bf16" else 16
    maps, bits = video_problem(1, 3, 40, 35, heads, dh, dtype, seed=ws)
    dev = to_dev(torch, maps, bits, dtype)
    w = weights3d(10, 64, 16, 1)
    qp, kp = rib.encode3d(1, ws, 10, 64, 16, torch.from_numpy(w).cuda())
    o3 = rib.window_attn3d(*dev, qp, kp, heads, 1, ws)
    for t in range(3):
        o2 = rib.window_attn(*[x[:, t].contiguous() for x in dev], qp, kp, heads, ws)
        a = o3[:, t].contiguous()
        assert torch.equal(a.view(torch.int16) if dtype == "bf16" else a,
                           o2.view(torch.int16) if dtype == "bf16" else o2), t
    one = [x[:, :1].contiguous() for x in dev]
    o31 = rib.window_attn3d(*one, qp, kp, heads, 1, ws)
    assert torch.equal(o31.view(torch.int16) if dtype == "bf16" else o31,
                       o3[:, :1].contiguous().view(torch.int16) if dtype == "bf16" else o3[:, :1].contiguous())


def test_attn3d_locality(torch):
    """Changing one token's key and value changes outputs in its space-time window only (bf16, chunked kernel)."""
    B, T, H, W, heads, dh, wt, ws = 1, 4, 20, 20, 1, 30, 2, 16
    maps, bits = video_problem(B, T, H, W, heads, dh, "bf16", seed=3)
    dev = to_dev(torch, maps, bits, "bf16")
    w = weights3d(10, 64, 16, 4)
    qp, kp = rib.encode3d(wt, ws, 10, 64, 16, torch.from_numpy(w).cuda())
    base = rib.window_attn3d(*dev, qp, kp, heads, wt, ws).view(torch.int16).cpu().numpy()
    dev[1][0, 2, 17, 3] += 1.0
    dev[2][0, 2, 17, 3] += 1.0
    moved = rib.window_attn3d(*dev, qp, kp, heads, wt, ws).view(torch.int16).cpu().numpy()
    changed = (base != moved).any(axis=-1)[0]
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    inside = (t // wt == 1) & (y // ws == 1) & (x // ws == 0)
    assert changed[inside].any() and not changed[~inside].any()
