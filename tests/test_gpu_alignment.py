"""GPU: the attention and gate entry points take maps that are only 4-byte aligned (and fp32
tables that are only 8-byte aligned), e.g. a batch slice of a bf16 map with an odd H*W*C.

Each case copies the inputs into buffers that start 4 bytes past a 16-byte boundary (qp, kp:
8 bytes), runs the entry point there and on the ordinary (aligned) tensors, and requires the
outputs to be bit-identical: the kernels do the same arithmetic whatever the alignment, and only
the width of some copies changes.
"""
import sys

import numpy as np
import pytest

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


def shifted(torch, t, nbytes):
    """A contiguous copy of t whose data starts nbytes past a 16-byte boundary."""
    k = nbytes // t.element_size()
    flat = torch.empty(t.numel() + 16, dtype=t.dtype, device=t.device)
    base = (16 - flat.data_ptr() % 16) % 16 // t.element_size()
    out = flat[base + k: base + k + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 == nbytes
    return out


def bits(torch, t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def maps_of(torch, p):
    return [torch.from_numpy(p.bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("qc", "kc", "v", "g")]


@pytest.mark.parametrize("ws,R", [(16, 16), (32, 16), (96, 16), (96, 32)])
def test_forward_on_dword_aligned_maps(torch, ws, R):
    """An image of 37x53 tokens at C = 90 (odd H*W*C): whole-window (16), chunked (32; 96 at R = 16)
    and tiled (96 at R = 32) kernels."""
    note(f"alignment forward ws={ws} R={R}")
    p = synthetic.make_problem(1, 37, 53, 3, 30, R, dtype="bf16", seed=ws)
    maps = maps_of(torch, p)
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, torch.from_numpy(p.weights).cuda())
    want = rib.window_attn(*maps, qp, kp, 3, ws)
    smaps = [shifted(torch, m, 4) for m in maps]
    sqp, skp = shifted(torch, qp, 8), shifted(torch, kp, 8)
    got = shifted(torch, torch.zeros_like(want), 4)
    rib.window_attn_into(*smaps, sqp, skp, 3, ws, got)
    torch.cuda.synchronize()
    assert torch.equal(bits(torch, got), bits(torch, want))


def test_backward_on_dword_aligned_maps(torch):
    """The training forward and the backward (prep kernel's dword copies) on 4-byte-aligned maps."""
    ws, heads = 16, 3
    note("alignment backward")
    p = synthetic.make_problem(1, 37, 53, heads, 30, 16, dtype="bf16", seed=5)
    maps = maps_of(torch, p)
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, torch.from_numpy(p.weights).cuda())
    o, lse = rib.window_attn_train(*maps, qp, kp, heads, ws)
    torch.manual_seed(5)
    dout = torch.randn(o.shape, device="cuda").to(torch.bfloat16)
    want = rib.window_attn_backward(*maps, qp, kp, o, lse, dout, heads, ws)
    s = [shifted(torch, t, 4) for t in (*maps, o, lse, dout)]
    sqp, skp = shifted(torch, qp, 8), shifted(torch, kp, 8)
    outs = [shifted(torch, torch.zeros_like(maps[0]), 4) for _ in range(4)]
    dqp, dkp = shifted(torch, torch.zeros_like(qp), 8), shifted(torch, torch.zeros_like(kp), 8)
    nbytes = rib.backward_workspace_bytes(maps[0], qp, heads, ws)
    work = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
    off = (16 - work.data_ptr() % 16) % 16
    work = work[off: off + nbytes]
    rib.window_attn_backward_into(s[0], s[1], s[2], s[3], sqp, skp, s[4], s[5], s[6], heads, ws, *outs, dqp, dkp,
                                  work)
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip((*outs, dqp, dkp), want)):
        assert torch.equal(bits(torch, a), bits(torch, b)), f"gradient {k}"


def test_gate_on_dword_aligned_maps(torch):
    note("alignment gate")
    B, H, W, C = 1, 37, 53, 90
    p = synthetic.make_gate_problem(B, H, W, C, "bf16", seed=11)
    x = torch.from_numpy(p.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    w = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (p.dw_w, p.dw_b, p.pw_w, p.pw_b)]
    want = rib.cla_gate(x, *w)
    got = shifted(torch, torch.zeros_like(want), 4)
    rib.cla_gate_into(shifted(torch, x, 4), *w, got)
    torch.cuda.synchronize()
    assert torch.equal(bits(torch, got), bits(torch, want))
