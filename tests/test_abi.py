"""The C ABI library on the host: it loads, exports what include/rib.h declares,
and rejects bad arguments before any HIP call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import super_resolution_transformer_amd as rib


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rib.LIB_PATH):
        from super_resolution_transformer_amd import build
        build.build()
    return rib.lib()


def test_header_declares_the_boundary():
    assert set(rib.header_functions()) == {
        "rib_encode", "rib_window_attn", "rib_attn_supported", "rib_last_error", "rib_abi_version",
        "rib_cla_gate", "rib_window_attn_heads", "rib_window_attn_train", "rib_window_attn_backward", "rib_window_attn_backward_workspace",
        "rib_encode_backward", "rib_encode_backward_workspace", "rib_encode_backward_noalloc", "rib_ln_qkv", "rib_encode3d",
        "rib_window_attn3d", "rib_window_attn_multi", "rib_window_attn_heads_train", "rib_window_attn_lnq",
        "rib_window_attn_heads_backward"}


def test_library_exports_every_declared_symbol(L):
    for name in rib.header_functions():
        assert hasattr(L, name), name


def test_abi_version_matches_header(L):
    m = re.search(r"#define\s+RIB_ABI_VERSION\s+(\d+)", open(rib.HEADER).read())
    assert L.rib_abi_version() == int(m.group(1))


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        rib.lib(str(tmp_path / "librib.so"))


def test_support_query(L):
    assert L.rib_attn_supported(30, 16, 96, rib.RIB_BF16) == rib.RIB_OK
    assert L.rib_attn_supported(16, 16, 16, rib.RIB_BF16) == rib.RIB_OK
    assert L.rib_attn_supported(16, 16, 16, rib.RIB_F32) == rib.RIB_OK
    assert L.rib_attn_supported(7, 5, 16, rib.RIB_F32) == rib.RIB_OK
    assert L.rib_attn_supported(31, 16, 16, rib.RIB_BF16) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_attn_supported(30, 16, 129, rib.RIB_BF16) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_attn_supported(65, 16, 16, rib.RIB_F32) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_attn_supported(30, 16, 1, rib.RIB_BF16) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_attn_supported(30, 16, 16, 7) == rib.RIB_ERR_INVALID_ARG
    assert "dtype" in L.rib_last_error().decode()


# Fake, never-dereferenced device addresses: every call below must fail validation.
# (Skipped where a GPU is visible, so a validation bug can never launch on them.)
def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


fake = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation checks run only without a GPU")
MB = 1 << 20
P = [ctypes.c_void_p(0x10000000 + i * 64 * MB) for i in range(8)]


def attn(L, ptrs=None, B=1, H=8, W=8, heads=2, dh=30, R=16, window=8, dtype=rib.RIB_BF16, stream=None):
    p = list(ptrs or P[:7])
    return L.rib_window_attn(*p, B, H, W, heads, dh, R, window, dtype, stream)


@fake
def test_attn_validation(L):
    assert attn(L, [None] + P[1:7]) == rib.RIB_ERR_INVALID_ARG
    assert "null" in L.rib_last_error().decode()
    assert attn(L, P[:6] + [None]) == rib.RIB_ERR_INVALID_ARG
    assert attn(L, B=0) == rib.RIB_ERR_INVALID_ARG
    assert attn(L, heads=0) == rib.RIB_ERR_INVALID_ARG
    assert attn(L, window=1) == rib.RIB_ERR_INVALID_ARG
    assert attn(L, dtype=5) == rib.RIB_ERR_INVALID_ARG
    assert attn(L, dh=31) == rib.RIB_ERR_UNSUPPORTED
    assert attn(L, window=200) == rib.RIB_ERR_UNSUPPORTED
    assert attn(L, B=1 << 12, H=1 << 10, W=1 << 10) == rib.RIB_ERR_UNSUPPORTED   # >= 2^31 elements
    assert "2^31" in L.rib_last_error().decode()
    mis = [ctypes.c_void_p(P[0].value + 2)] + P[1:7]                     # maps: dword alignment
    assert attn(L, mis) == rib.RIB_ERR_INVALID_ARG
    assert "aligned" in L.rib_last_error().decode()
    mis_tab = P[:4] + [ctypes.c_void_p(P[4].value + 4)] + P[5:7]           # tables: float pairs
    assert attn(L, mis_tab) == rib.RIB_ERR_INVALID_ARG
    assert "8-byte" in L.rib_last_error().decode()
    alias = P[:6] + [ctypes.c_void_p(P[2].value + 256)]                     # o inside v
    assert attn(L, alias) == rib.RIB_ERR_INVALID_ARG
    assert "overlap" in L.rib_last_error().decode()
    alias_qp = P[:6] + [P[4]]                                               # o == qp
    assert attn(L, alias_qp) == rib.RIB_ERR_INVALID_ARG


@fake
def test_attn_train_validation(L):
    def train(ptrs, **kw):
        a = dict(B=1, H=8, W=8, heads=2, dh=30, R=16, window=8, dtype=rib.RIB_BF16)
        a.update(kw)
        return L.rib_window_attn_train(*ptrs, a["B"], a["H"], a["W"], a["heads"], a["dh"], a["R"], a["window"],
                                       a["dtype"], None)
    assert train(P[:7] + [None]) == rib.RIB_ERR_INVALID_ARG
    assert "rib_window_attn_train" in L.rib_last_error().decode()
    assert train(P[:7] + [ctypes.c_void_p(P[6].value + 64)]) == rib.RIB_ERR_INVALID_ARG     # lse inside o
    assert "overlap" in L.rib_last_error().decode()
    assert train(P[:7] + [P[4]]) == rib.RIB_ERR_INVALID_ARG                                # lse == qp
    assert train(P[:8], dh=31) == rib.RIB_ERR_UNSUPPORTED


@fake
def test_attn_heads_validation(L):
    def heads_call(ptrs, **kw):
        a = dict(B=1, H=8, W=8, heads=2, dh=30, R=16, window=8, dtype=rib.RIB_BF16)
        a.update(kw)
        return L.rib_window_attn_heads(*ptrs, a["B"], a["H"], a["W"], a["heads"], a["dh"], a["R"], a["window"],
                                       a["dtype"], None)
    assert heads_call([None] + P[1:7]) == rib.RIB_ERR_INVALID_ARG
    assert "rib_window_attn_heads" in L.rib_last_error().decode()
    assert heads_call(P[:7], dh=31) == rib.RIB_ERR_UNSUPPORTED
    # the per-head tables are heads times larger: o just past one table still overlaps the second
    tail = P[:6] + [ctypes.c_void_p(P[4].value + 64 * 16 * 4 + 256)]
    assert heads_call(tail) == rib.RIB_ERR_INVALID_ARG
    assert "overlap" in L.rib_last_error().decode()


@fake
def test_encode_validation(L):
    w, q, k = P[0], P[1], P[2]
    assert L.rib_encode(16, 10, 64, 16, None, q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode(1, 10, 64, 16, w, q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode(16, -1, 64, 16, w, q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode(16, 10, 0, 16, w, q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode(129, 10, 64, 16, w, q, k, None) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_encode(16, 17, 64, 16, w, q, k, None) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_encode(16, 10, 64, 16, w, q, q, None) == rib.RIB_ERR_INVALID_ARG     # qp == kp
    assert L.rib_encode(16, 10, 64, 16, w, w, k, None) == rib.RIB_ERR_INVALID_ARG     # qp == weights
    assert L.rib_encode(16, 10, 64, 16, ctypes.c_void_p(w.value + 2), q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_last_error().decode() != ""


def gate(L, ptrs=None, B=1, H=8, W=8, C=180, dtype=rib.RIB_BF16, stream=None):
    p = list(ptrs or P[:6])
    return L.rib_cla_gate(*p, B, H, W, C, dtype, stream)


@fake
def test_gate_validation(L):
    assert gate(L, [None] + P[1:6]) == rib.RIB_ERR_INVALID_ARG
    assert gate(L, P[:5] + [None]) == rib.RIB_ERR_INVALID_ARG
    assert gate(L, B=0) == rib.RIB_ERR_INVALID_ARG
    assert gate(L, dtype=3) == rib.RIB_ERR_INVALID_ARG
    assert gate(L, C=181) == rib.RIB_ERR_UNSUPPORTED
    assert gate(L, C=258) == rib.RIB_ERR_UNSUPPORTED
    assert gate(L, B=1 << 12, H=1 << 10, W=1 << 10, C=2) == rib.RIB_ERR_UNSUPPORTED
    assert gate(L, [ctypes.c_void_p(P[0].value + 2)] + P[1:6]) == rib.RIB_ERR_INVALID_ARG
    assert "aligned" in L.rib_last_error().decode()
    assert gate(L, P[:5] + [ctypes.c_void_p(P[0].value + 64)]) == rib.RIB_ERR_INVALID_ARG  # g inside x
    assert "overlap" in L.rib_last_error().decode()
    assert gate(L, P[:5] + [P[3]]) == rib.RIB_ERR_INVALID_ARG                             # g == pw_w


PB = [ctypes.c_void_p(0x10000000 + i * 64 * MB) for i in range(16)]


def bwd(L, ptrs=None, nbytes=None, B=1, H=8, W=8, heads=2, dh=30, R=16, window=8, dtype=rib.RIB_BF16):
    p = list(ptrs or PB)
    if nbytes is None:
        nbytes = L.rib_window_attn_backward_workspace(B, H, W, heads, dh, R, window, dtype)
    return L.rib_window_attn_backward(*p, nbytes, B, H, W, heads, dh, R, window, dtype, None)


@fake
def test_backward_validation(L):
    need = L.rib_window_attn_backward_workspace(1, 8, 8, 2, 30, 16, 8, rib.RIB_BF16)
    # dA (bf16) + D + two per-row tables + two packed operand images (matrix-core path:
    # 2 units x one 64-row tile x 10 chunks x 1 KB), each region 256-byte aligned
    rows = 64 * 2
    up = lambda x: (x + 255) // 256 * 256
    assert need == up(rows * 30 * 2) + up(rows * 4) + 2 * up(rows * 16 * 4) + 2 * 2 * 10 * 1024
    f32 = L.rib_window_attn_backward_workspace(1, 8, 8, 2, 30, 16, 8, rib.RIB_F32)
    assert f32 == up(rows * 30 * 4) + up(rows * 4) + 2 * up(rows * 16 * 4)      # no images on the fp32 path
    assert L.rib_window_attn_backward_workspace(0, 8, 8, 2, 30, 16, 8, rib.RIB_BF16) == 0
    assert L.rib_window_attn_backward_workspace(1, 8, 8, 2, 30, 16, 1, rib.RIB_BF16) == 0
    assert bwd(L, [None] + PB[1:]) == rib.RIB_ERR_INVALID_ARG
    assert "null" in L.rib_last_error().decode()
    assert bwd(L, PB[:15] + [None]) == rib.RIB_ERR_INVALID_ARG
    assert bwd(L, PB[:7] + [None] + PB[8:]) == rib.RIB_ERR_INVALID_ARG          # lse
    assert bwd(L, B=0) == rib.RIB_ERR_INVALID_ARG
    assert bwd(L, window=1) == rib.RIB_ERR_INVALID_ARG
    assert bwd(L, dtype=4) == rib.RIB_ERR_INVALID_ARG
    assert bwd(L, dh=65) == rib.RIB_ERR_UNSUPPORTED
    assert bwd(L, R=65) == rib.RIB_ERR_UNSUPPORTED
    assert bwd(L, window=129) == rib.RIB_ERR_UNSUPPORTED
    assert bwd(L, nbytes=need - 1) == rib.RIB_ERR_INVALID_ARG
    assert "workspace" in L.rib_last_error().decode()
    assert bwd(L, [ctypes.c_void_p(PB[0].value + 2)] + PB[1:]) == rib.RIB_ERR_INVALID_ARG   # maps: dwords
    assert "4-byte" in L.rib_last_error().decode()
    assert bwd(L, PB[:4] + [ctypes.c_void_p(PB[4].value + 4)] + PB[5:]) == rib.RIB_ERR_INVALID_ARG  # qp: pairs
    assert "8-byte" in L.rib_last_error().decode()
    assert bwd(L, PB[:15] + [ctypes.c_void_p(PB[15].value + 8)]) == rib.RIB_ERR_INVALID_ARG  # workspace
    assert "16-byte" in L.rib_last_error().decode()
    alias = PB[:10] + [PB[2]] + PB[11:]                                   # dkc == v
    assert bwd(L, alias) == rib.RIB_ERR_INVALID_ARG
    assert "overlap" in L.rib_last_error().decode()
    alias = PB[:15] + [ctypes.c_void_p(PB[9].value + 256)]                # workspace inside dqc
    assert bwd(L, alias) == rib.RIB_ERR_INVALID_ARG
    alias = PB[:13] + [PB[14], PB[14], PB[15]]                            # dqp == dkp
    assert bwd(L, alias) == rib.RIB_ERR_INVALID_ARG
    assert bwd(L, PB[:13] + [PB[4]] + PB[14:]) == rib.RIB_ERR_INVALID_ARG  # dqp == qp (an input)
    assert bwd(L, PB[:12] + [PB[7]] + PB[13:]) == rib.RIB_ERR_INVALID_ARG  # dg == lse (an input)


@fake
def test_heads_training_validation(L):
    def hb(ptrs=None, nbytes=None, **kw):
        a = dict(B=1, H=8, W=8, heads=2, dh=30, R=16, window=8, dtype=rib.RIB_BF16)
        a.update(kw)
        p = list(ptrs or PB)
        if nbytes is None:
            nbytes = L.rib_window_attn_backward_workspace(a["B"], a["H"], a["W"], a["heads"], a["dh"], a["R"],
                                                          a["window"], a["dtype"])
        return L.rib_window_attn_heads_backward(*p, nbytes, a["B"], a["H"], a["W"], a["heads"], a["dh"], a["R"],
                                                a["window"], a["dtype"], None)
    assert hb([None] + PB[1:]) == rib.RIB_ERR_INVALID_ARG
    assert "rib_window_attn_heads_backward" in L.rib_last_error().decode()
    assert hb(dh=65) == rib.RIB_ERR_UNSUPPORTED
    assert hb(nbytes=16) == rib.RIB_ERR_INVALID_ARG
    # the per-head tables are heads times larger: dqp just past one table still overlaps qp's second
    tab = 8 * 8 * 16 * 4
    assert hb(PB[:13] + [ctypes.c_void_p(PB[4].value + tab + 256)] + PB[14:]) == rib.RIB_ERR_INVALID_ARG
    assert "overlap" in L.rib_last_error().decode()

    def ht(ptrs, **kw):
        a = dict(B=1, H=8, W=8, heads=2, dh=30, R=16, window=8, dtype=rib.RIB_BF16)
        a.update(kw)
        return L.rib_window_attn_heads_train(*ptrs, a["B"], a["H"], a["W"], a["heads"], a["dh"], a["R"],
                                             a["window"], a["dtype"], None)
    assert ht(P[:7] + [None]) == rib.RIB_ERR_INVALID_ARG
    assert "rib_window_attn_heads_train" in L.rib_last_error().decode()
    assert ht(P[:8], dh=31) == rib.RIB_ERR_UNSUPPORTED
    assert ht(P[:6] + [ctypes.c_void_p(P[4].value + tab + 256), P[7]]) == rib.RIB_ERR_INVALID_ARG   # o in qp's 2nd table


@fake
def test_encode_backward_validation(L):
    need = L.rib_encode_backward_workspace(16, 10, 64, 16)
    nw = 42 * 64 + 64 + 2 * 64 * 16
    assert need == 4 * nw * 16                                             # 256 positions / 16 per block
    assert L.rib_encode_backward_workspace(1, 10, 64, 16) == 0
    w, q, k, d, ws = PB[:5]
    assert L.rib_encode_backward(16, 10, 64, 16, None, q, k, d, ws, need, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode_backward(1, 10, 64, 16, w, q, k, d, ws, need, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode_backward(16, 17, 64, 16, w, q, k, d, ws, need, None) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_encode_backward(16, 10, 64, 16, w, q, k, d, ws, need - 4, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode_backward(16, 10, 64, 16, w, q, k, w, ws, need, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode_backward(16, 10, 64, 16, w, q, k, d, d, need, None) == rib.RIB_ERR_INVALID_ARG
    assert "overlap" in L.rib_last_error().decode()


@fake
def test_encode_backward_noalloc_validation(L):
    """The fixed-workspace variant refuses what rib_encode_backward refuses, before any HIP call."""
    w, q, k, d = PB[:4]
    f = L.rib_encode_backward_noalloc
    assert f(16, 10, 64, 16, None, q, k, d, None) == rib.RIB_ERR_INVALID_ARG
    assert "rib_encode_backward_noalloc" in L.rib_last_error().decode()
    assert f(1, 10, 64, 16, w, q, k, d, None) == rib.RIB_ERR_INVALID_ARG
    assert f(129, 10, 64, 16, w, q, k, d, None) == rib.RIB_ERR_UNSUPPORTED
    assert f(16, 17, 64, 16, w, q, k, d, None) == rib.RIB_ERR_UNSUPPORTED
    assert f(16, 10, 257, 16, w, q, k, d, None) == rib.RIB_ERR_UNSUPPORTED
    assert f(16, 10, 64, 65, w, q, k, d, None) == rib.RIB_ERR_UNSUPPORTED
    assert f(16, 10, 64, 16, w, q, k, ctypes.c_void_p(d.value + 2), None) == rib.RIB_ERR_INVALID_ARG
    assert "aligned" in L.rib_last_error().decode()
    assert f(16, 10, 64, 16, w, q, k, w, None) == rib.RIB_ERR_INVALID_ARG
    assert "overlap" in L.rib_last_error().decode()


def lnq(L, ptrs=None, B=1, H=8, W=8, C=180, eps=1e-5, dtype=rib.RIB_BF16):
    p = list(ptrs or P[:5] + [P[5], P[6], P[7], None])
    return L.rib_ln_qkv(*p, B, H, W, C, ctypes.c_float(eps), dtype, None)


@fake
def test_ln_qkv_validation(L):
    assert lnq(L, [None] + P[1:8] + [None]) == rib.RIB_ERR_INVALID_ARG
    assert "rib_ln_qkv" in L.rib_last_error().decode()
    assert lnq(L, P[:7] + [None, None]) == rib.RIB_ERR_INVALID_ARG          # v missing
    assert lnq(L, B=0) == rib.RIB_ERR_INVALID_ARG
    assert lnq(L, dtype=2) == rib.RIB_ERR_INVALID_ARG
    assert lnq(L, eps=-1.0) == rib.RIB_ERR_INVALID_ARG
    assert lnq(L, C=257) == rib.RIB_ERR_UNSUPPORTED
    assert lnq(L, C=181) == rib.RIB_ERR_UNSUPPORTED                          # odd C, bf16
    assert lnq(L, [ctypes.c_void_p(P[0].value + 4)] + P[1:8] + [None]) == rib.RIB_ERR_INVALID_ARG
    assert "aligned" in L.rib_last_error().decode()
    assert lnq(L, P[:5] + [P[0], P[6], P[7], None]) == rib.RIB_ERR_INVALID_ARG  # q == x
    assert "overlap" in L.rib_last_error().decode()
    assert lnq(L, P[:5] + [P[5], P[5], P[7], None]) == rib.RIB_ERR_INVALID_ARG  # q == k
    assert lnq(L, P[:8] + [P[3]]) == rib.RIB_ERR_INVALID_ARG                     # xn == w


@fake
def test_window_attn_lnq_validation(L):
    X = [ctypes.c_void_p(0x10000000 + i * 64 * MB) for i in range(11)]   # x gamma beta w bias kc v g qp kp o

    def call(ptrs=None, B=1, H=8, W=8, heads=6, dh=30, R=16, window=8, eps=1e-5, dtype=rib.RIB_BF16):
        return L.rib_window_attn_lnq(*(ptrs or X), B, H, W, heads, dh, R, window, ctypes.c_float(eps), dtype, None)
    assert call(X[:1] + [None] + X[2:]) == rib.RIB_ERR_INVALID_ARG                  # gamma missing
    assert "rib_window_attn_lnq" in L.rib_last_error().decode()
    assert call([None] + X[1:]) == rib.RIB_ERR_INVALID_ARG                          # x missing
    assert call(X[:10] + [None]) == rib.RIB_ERR_INVALID_ARG                         # o missing
    assert call(dtype=rib.RIB_F32) == rib.RIB_ERR_UNSUPPORTED
    assert call(dh=8, R=8) == rib.RIB_ERR_UNSUPPORTED
    assert call(heads=7) == rib.RIB_ERR_UNSUPPORTED                                 # C = 210 > 192
    assert call(eps=-1.0) == rib.RIB_ERR_INVALID_ARG
    assert call(eps=float("nan")) == rib.RIB_ERR_INVALID_ARG
    assert call(window=1) == rib.RIB_ERR_INVALID_ARG
    assert call(X[:1] + [ctypes.c_void_p(X[1].value + 2)] + X[2:]) == rib.RIB_ERR_INVALID_ARG
    assert "aligned" in L.rib_last_error().decode()
    assert call(X[:10] + [X[3]]) == rib.RIB_ERR_INVALID_ARG                         # o == w
    assert "overlap" in L.rib_last_error().decode()
    assert call(X[:10] + [ctypes.c_void_p(X[3].value + 12 * 180 * 180 - 64)]) == rib.RIB_ERR_INVALID_ARG  # o in w's tail
    assert call(X[:10] + [X[0]]) == rib.RIB_ERR_INVALID_ARG                         # o == x
    # rib_ln_qkv without q still needs k and v
    assert lnq(L, P[:5] + [None, None, P[7], None]) == rib.RIB_ERR_INVALID_ARG


@fake
def test_space_time_validation(L):
    def a3(ptrs=None, **kw):
        a = dict(B=1, T=4, H=8, W=8, heads=2, dh=30, R=16, frames=2, window=8, dtype=rib.RIB_BF16)
        a.update(kw)
        return L.rib_window_attn3d(*(ptrs or P[:7]), a["B"], a["T"], a["H"], a["W"], a["heads"], a["dh"], a["R"],
                                   a["frames"], a["window"], a["dtype"], None)
    assert a3([None] + P[1:7]) == rib.RIB_ERR_INVALID_ARG
    assert "rib_window_attn3d" in L.rib_last_error().decode()
    assert a3(T=0) == rib.RIB_ERR_INVALID_ARG
    assert a3(frames=0) == rib.RIB_ERR_INVALID_ARG
    assert a3(frames=2, window=96) == rib.RIB_ERR_UNSUPPORTED                    # 18432 tokens per window
    assert "16384" in L.rib_last_error().decode()
    assert a3(dh=31) == rib.RIB_ERR_UNSUPPORTED
    assert a3(B=1 << 10, T=1 << 10, H=64, W=64, dh=30) == rib.RIB_ERR_UNSUPPORTED  # >= 2^31 elements
    # the tables are frames times longer: o just past one 2-D table still overlaps
    assert a3(P[:6] + [ctypes.c_void_p(P[4].value + 64 * 16 * 4 + 256)]) == rib.RIB_ERR_INVALID_ARG
    w, q, k = P[0], P[1], P[2]
    assert L.rib_encode3d(2, 8, 10, 64, 16, None, q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode3d(0, 8, 10, 64, 16, w, q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode3d(2, 1, 10, 64, 16, w, q, k, None) == rib.RIB_ERR_INVALID_ARG
    assert L.rib_encode3d(2, 96, 10, 64, 16, w, q, k, None) == rib.RIB_ERR_UNSUPPORTED
    assert L.rib_encode3d(2, 8, 10, 64, 16, w, q, q, None) == rib.RIB_ERR_INVALID_ARG


@fake
def test_multi_validation(L):
    def call(base=0, **kw):
        a = dict(B=1, H=8, W=8, heads=2, dh=30, R=16, window=8)
        a.update(kw)
        ptrs = [ctypes.c_void_p(p.value + base) for p in P[:7]]
        return rib.AttnCall(*[p.value for p in ptrs], a["B"], a["H"], a["W"], a["heads"], a["dh"], a["R"],
                            a["window"])

    def multi(calls, n=None, dtype=rib.RIB_BF16):
        arr = (rib.AttnCall * max(len(calls), 1))(*calls)
        return L.rib_window_attn_multi(len(calls) if n is None else n, arr, dtype, None)

    assert L.rib_window_attn_multi(1, None, rib.RIB_BF16, None) == rib.RIB_ERR_INVALID_ARG
    assert "rib_window_attn_multi" in L.rib_last_error().decode()
    assert multi([call()], n=0) == rib.RIB_ERR_INVALID_ARG
    assert multi([call()] * 17) == rib.RIB_ERR_INVALID_ARG                     # more than RIB_MAX_CALLS
    assert multi([call(), call(MB, window=1)]) == rib.RIB_ERR_INVALID_ARG      # one bad call fails the batch
    assert multi([call(), call(MB, dh=31)]) == rib.RIB_ERR_UNSUPPORTED
    bad = call(MB)
    bad.o = P[2].value + 256                                                  # output of call 1 inside v of call 0
    assert multi([call(), bad]) == rib.RIB_ERR_INVALID_ARG
    assert "overlap" in L.rib_last_error().decode()
    same_out = call(MB)
    same_out.o = P[6].value                                                   # both calls write one buffer
    assert multi([call(), same_out]) == rib.RIB_ERR_INVALID_ARG
    assert multi([call()], dtype=9) == rib.RIB_ERR_INVALID_ARG


def test_python_binding_argument_checks():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 4, 8)
    with pytest.raises(ValueError):
        rib.encode(4, 10, 64, 16, torch.zeros(3))          # not a GPU tensor
    with pytest.raises(ValueError):
        rib.window_attn_into(x, x, x, x[:, :2], torch.zeros(16, 4), torch.zeros(16, 4), 2, 4, x)
    with pytest.raises(ValueError):
        rib.window_attn_into(x, x, x, x, torch.zeros(16, 4), torch.zeros(16, 4), 2, 4, x)  # CPU tensors
    with pytest.raises(ValueError):
        rib.cla_gate_into(x, torch.zeros(8, 3, 3), torch.zeros(8), torch.zeros(8, 8), torch.zeros(8), x)
    with pytest.raises(ValueError):
        rib.window_attn_backward(x, x, x, x, torch.zeros(16, 4), torch.zeros(16, 4), x, torch.zeros(1, 4, 4, 2),
                                 x[:, :2], 2, 4)
    with pytest.raises(ValueError):
        rib.window_attn_backward(x, x, x, x, torch.zeros(16, 4), torch.zeros(16, 4), x, torch.zeros(1, 4, 4, 2),
                                 x, 2, 4)  # CPU tensors
    with pytest.raises(ValueError):
        rib.window_attn_train(x, x, x, x, torch.zeros(16, 4), torch.zeros(16, 4), 2, 4)       # CPU tensors
    with pytest.raises(ValueError):
        rib.encode_backward(4, 10, 64, 16, torch.zeros(3), torch.zeros(16, 16), torch.zeros(16, 16))
    with pytest.raises(ValueError):
        rib.cla_gate_into(x, torch.zeros(8, 9), torch.zeros(8), torch.zeros(8, 8), torch.zeros(8), x)
    with pytest.raises(ValueError):
        rib.window_attn_multi([(x, x, x, x, torch.zeros(16, 4), torch.zeros(16, 4), 2, 4)])          # CPU tensors
    with pytest.raises(ValueError):
        rib.window_attn_multi_into([], [])
