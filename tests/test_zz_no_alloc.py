"""GPU check of rib_encode_backward_noalloc, the encoder backward whose partial gradients go to
the library's fixed per-device array instead of a caller's workspace.

Two calls in a row on one stream, the second smaller, each compared with rib_encode_backward
(the workspace-taking entry point) on the same inputs:
  - window 96 (576 position chunks, more than the 218 rows the 4 MiB array holds for 4,800
    weights, so a workgroup sums two or three chunks): max |difference| <= 1e-5 max |dW|, the
    fp32 bar of the encoder's parity tests (only the summation order differs);
  - window 32 (64 chunks, one per row, as in rib_encode_backward): bit-identical, which also
    shows that the rows left by the first call do not leak into the second.
The first result is also checked against the oracle at the same bar.
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


def test_noalloc_matches_workspace_entry_point_twice(torch):
    L, hidden, R = 10, 64, 16
    rng = np.random.default_rng(7)
    w_host = synthetic.draw_weights(rng, L, hidden, R)
    w = torch.from_numpy(w_host).cuda()
    for ws, exact in [(96, False), (32, True)]:
        note(f"encode backward noalloc ws={ws} L={L} hidden={hidden} R={R}")
        gq_host = rng.standard_normal((ws * ws, R)).astype(np.float32)
        gk_host = rng.standard_normal((ws * ws, R)).astype(np.float32)
        gq, gk = torch.from_numpy(gq_host).cuda(), torch.from_numpy(gk_host).cuda()
        want = rib.encode_backward(ws, L, hidden, R, w, gq, gk)
        got = torch.full_like(w, float("nan"))
        rib.encode_backward_noalloc_into(ws, L, hidden, R, w, gq, gk, got)
        torch.cuda.synchronize()
        a, b = got.cpu().numpy().astype(np.float64), want.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a))
        scale = float(np.abs(b).max())
        err = float(np.abs(a - b).max())
        note(f"  max|noalloc - workspace| {err:.3g}  max|dW| {scale:.3g}")
        if exact:
            assert torch.equal(got, want)
        else:
            assert err <= 1e-5 * scale
            ref = oracle.encode_backward(ws, L, hidden, R, w_host, gq_host, gk_host)
            oerr = float(np.abs(a - ref).max())
            note(f"  max|noalloc - oracle| {oerr:.3g}")
            assert oerr <= 1e-5 * float(np.abs(ref).max())
