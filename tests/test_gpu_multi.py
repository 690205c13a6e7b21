"""GPU: rib_window_attn_multi runs several independent calls in few launches.

Calls whose windows take the 256-thread kernels (whole-window up to 256 tokens,
chunked above) share one launch per 8 calls; calls of the tiled kernel (the
(dh, R) shapes (32, 16), (16, 32) and (30, 32) above 2,048 tokens) share
another.  Each call's output must be bit-identical to rib_window_attn on the
same arguments (the batched kernels run the same per-workgroup code), which
makes the index mapping of the grouped grid (call ranges, XCD dealing, padding
workgroups, the per-call kernel branch) checkable exactly; one batch is also
compared with the oracle.
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


def make_call(torch, B, H, W, heads, dh, R, ws, dtype, seed):
    p = synthetic.make_problem(B, H, W, heads, dh, R, dtype=dtype, seed=seed)
    if dtype == "bf16":
        maps = [torch.from_numpy(p.bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("qc", "kc", "v", "g")]
    else:
        maps = [torch.from_numpy(getattr(p, n)).cuda() for n in ("qc", "kc", "v", "g")]
    qp, kp = rib.encode(ws, p.L, p.hidden, p.R, torch.from_numpy(p.weights).cuda())
    return p, (*maps, qp, kp, heads, ws)


def same(torch, a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def check_batch(torch, specs, dtype):
    calls = [make_call(torch, *sp, dtype, seed=100 + k)[1] for k, sp in enumerate(specs)]
    outs = rib.window_attn_multi(calls)
    for k, c in enumerate(calls):
        want = rib.window_attn(*c)
        torch.cuda.synchronize()
        assert same(torch, outs[k], want), f"call {k} {specs[k]} differs from rib_window_attn"


def test_cyclic_schedule_sst_lite(torch):
    """The three window sizes of the cyclic schedule on the SST-lite shape (180x320, C=48): whole-window
    (16), chunked (32, and 64 whose 720 workgroups are resident at once), one launch."""
    note("multi: cyclic 16/32/64 on 1x180x320, 3 heads x 16")
    check_batch(torch, [(1, 180, 320, 3, 16, 16, ws) for ws in (16, 32, 64)], "bf16")


def test_cyclic_schedule_inference_shape(torch):
    """The cyclic schedule at C = 180 (6 heads x 30): 16, 32 and 64 in one launch (64 dealt to the XCDs
    by window unit: 15 windows)."""
    note("multi: cyclic 16/32/64 on 1x180x320, 6 heads x 30")
    check_batch(torch, [(1, 180, 320, 6, 30, 16, ws) for ws in (16, 32, 64)], "bf16")


@pytest.mark.parametrize("ws,n,R", [(32, 10, 16), (16, 12, 16), (96, 9, 16), (96, 9, 32)])
def test_more_calls_than_one_group(torch, ws, n, R):
    """More than 8 calls of one kernel kind and one (dh, R) variant: the batch is split over two launches
    of the same grouped kernel (chunked, whole-window, chunked dealt by unit, tiled at R = 32); ragged
    maps of different sizes."""
    specs = [(1 + k % 2, 37 + 3 * k, 41 + 5 * k, 1 + k % 3, 30, R, ws) for k in range(n)]
    note(f"multi: {n} calls at window {ws}, R = {R}")
    check_batch(torch, specs, "bf16")


def test_sixteen_mixed_window_calls(torch):
    """Sixteen whole-window and chunked calls (windows 8 to 45), the most one multi call takes."""
    specs = [(1, 29 + 2 * k, 33 + k, 2, 16, 16, (8, 16, 17, 24, 32, 45)[k % 6]) for k in range(16)]
    note("multi: 16 mixed whole-window and chunked calls")
    check_batch(torch, specs, "bf16")


def test_many_mixed_calls(torch):
    """Ten calls of the 256-thread kernels in two launches (8 + 2): windows 2, 4, 16, 16 and 17 (whole
    window), 32 and 64 (whole windows per XCD), 96, 96 and 128 (chunked, some dealt by unit); ragged
    maps."""
    specs = [(1, 70, 61, 2, 30, 16, 96), (2, 37, 53, 3, 30, 16, 32), (1, 100, 61, 1, 30, 16, 64),
             (1, 40, 41, 1, 30, 16, 17), (3, 37, 53, 3, 30, 16, 16), (1, 5, 7, 2, 30, 16, 4),
             (1, 96, 96, 6, 30, 16, 96), (2, 21, 19, 2, 30, 16, 16), (1, 33, 130, 1, 30, 16, 128),
             (1, 1, 1, 2, 30, 16, 2)]
    note(f"multi: {len(specs)} mixed calls")
    check_batch(torch, specs, "bf16")


def test_tiled_and_chunked_calls_of_one_variant(torch):
    """(dh, R) = (30, 32): windows 96 and 128 take the tiled kernel (one launch), 16, 32 and a
    resident 64 the 256-thread kernels (another); ragged maps."""
    specs = [(1, 70, 61, 2, 30, 32, 96), (1, 33, 130, 1, 30, 32, 128), (2, 37, 53, 2, 30, 32, 16),
             (1, 37, 53, 3, 30, 32, 32), (1, 100, 61, 1, 30, 32, 64)]
    note("multi: tiled and chunked calls at (30, 32)")
    check_batch(torch, specs, "bf16")


def test_two_variants_in_one_batch(torch):
    note("multi: (dh, R) = (16, 16) and (30, 16) in one batch")
    check_batch(torch, [(1, 64, 64, 3, 16, 16, 32), (1, 70, 61, 2, 30, 16, 64), (2, 40, 33, 2, 16, 16, 16),
                        (1, 30, 31, 2, 30, 32, 16)], "bf16")


def test_f32_batch(torch):
    note("multi: fp32 calls")
    check_batch(torch, [(1, 64, 64, 3, 16, 16, 16), (1, 37, 53, 2, 30, 16, 32)], "f32")


def test_batch_against_oracle(torch):
    note("multi: against the oracle")
    specs = [(1, 40, 33, 2, 16, 16, 32), (1, 37, 40, 2, 16, 16, 16)]
    made = [make_call(torch, *sp, "bf16", seed=7 + k) for k, sp in enumerate(specs)]
    outs = rib.window_attn_multi([c for _, c in made])
    torch.cuda.synchronize()
    for (p, c), o, sp in zip(made, outs, specs):
        ws = sp[-1]
        oq, ok = oracle.encode(ws, p.L, p.hidden, p.R, p.weights)
        want = oracle.window_attn(p.qc, p.kc, p.v, p.g, oq, ok, p.heads, ws)
        err = float(np.abs(o.float().cpu().numpy() - want).max())
        note(f"  {sp}: max|err| {err:.3g}")
        assert err <= 2e-2
