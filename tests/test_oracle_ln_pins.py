"""Pins of the oracle's block input projection: LayerNorm over the channels of each token, then
x W + b into the Q | K | V maps (explainer section 3.1: an SST block starts with LayerNorm before the
RIB attention; the projection to Q, K, V is what the attention's inputs are).

Held against PyTorch's layer_norm and matmul on the CPU in float64, closed forms and invariances;
planted mistakes in the oracle source must each fail a pin."""
import os

import numpy as np
import pytest

import oracle
from super_resolution_transformer_amd import synthetic


def torch_ref(p, eps):
    import torch
    x = torch.from_numpy(p.x.astype(np.float64))
    C = x.shape[-1]
    xn = torch.nn.functional.layer_norm(x, (C,), torch.from_numpy(p.gamma.astype(np.float64)),
                                        torch.from_numpy(p.beta.astype(np.float64)), eps)
    y = xn @ torch.from_numpy(p.w.astype(np.float64)) + torch.from_numpy(p.bias.astype(np.float64))
    return y[..., :C].numpy(), y[..., C:2 * C].numpy(), y[..., 2 * C:].numpy(), xn.numpy()


@pytest.mark.parametrize("shape,eps", [((2, 5, 7, 6), 1e-5), ((1, 3, 4, 48), 1e-6), ((1, 1, 1, 2), 1e-3)])
def test_matches_torch_layer_norm_and_matmul(shape, eps):
    p = synthetic.make_ln_qkv_problem(*shape, dtype="f32", seed=sum(shape))
    got = oracle.ln_qkv(p.x, p.gamma, p.beta, p.w, p.bias, eps, with_xn=True)
    for a, b, nm in zip(got, torch_ref(p, eps), ("q", "k", "v", "xn")):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12, err_msg=nm)


def test_unit_affine_identity_projection_gives_standardised_tokens():
    """gamma = 1, beta = 0, W = [I | 2I | -I], bias 0: q = xn has zero mean and mean square
    var / (var + eps) per token; k = 2 q; v = -q."""
    p = synthetic.make_ln_qkv_problem(1, 4, 5, 8, dtype="f32", seed=3)
    C, eps = 8, 1e-5
    I = np.eye(C)
    q, k, v = oracle.ln_qkv(p.x, np.ones(C), np.zeros(C), np.concatenate([I, 2 * I, -I], axis=1), np.zeros(3 * C), eps)
    x = p.x.astype(np.float64)
    var = x.var(axis=-1)
    np.testing.assert_allclose(q.mean(axis=-1), 0.0, atol=1e-14)
    np.testing.assert_allclose((q ** 2).mean(axis=-1), var / (var + eps), rtol=1e-13)
    np.testing.assert_array_equal(k, 2 * q)
    np.testing.assert_array_equal(v, -q)


def test_invariant_to_per_token_shift_and_scale():
    """With eps = 0, LayerNorm(a x + b) = LayerNorm(x) for a > 0."""
    p = synthetic.make_ln_qkv_problem(1, 3, 3, 12, dtype="f32", seed=4)
    base = oracle.ln_qkv(p.x, p.gamma, p.beta, p.w, p.bias, 0.0)
    moved = oracle.ln_qkv(3.5 * p.x.astype(np.float64) - 2.0, p.gamma, p.beta, p.w, p.bias, 0.0)
    for a, b in zip(base, moved):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_constant_token_gives_beta():
    """A token whose channels are all equal has zero variance: xn = beta exactly, q = beta W_q + b_q."""
    p = synthetic.make_ln_qkv_problem(1, 1, 2, 6, dtype="f32", seed=5)
    x = p.x.astype(np.float64).copy()
    x[0, 0, 1, :] = 1.25
    q, k, v, xn = oracle.ln_qkv(x, p.gamma, p.beta, p.w, p.bias, 1e-5, with_xn=True)
    np.testing.assert_array_equal(xn[0, 0, 1], p.beta.astype(np.float64))
    want = p.beta.astype(np.float64) @ p.w.astype(np.float64) + p.bias
    np.testing.assert_allclose(np.concatenate([q[0, 0, 1], k[0, 0, 1], v[0, 0, 1]]), want, rtol=1e-13, atol=1e-14)


MUTATIONS = {
    "unbiased variance": ("var /= C;", "var /= (C - 1);"),
    "eps outside the root": ("1.0 / sqrt(var + eps);", "1.0 / (sqrt(var) + eps);"),
    "gamma dropped": ("* inv * gamma[c] + beta[c];", "* inv + beta[c];"),
    "beta dropped": ("* inv * gamma[c] + beta[c];", "* inv * gamma[c];"),
    "projection transposed": ("w[(size_t)c * 3 * C + o]", "w[(size_t)(o % C) * 3 * C + (o / C) * C + c]"),
    "projection bias dropped": ("double acc = bias[o];", "double acc = 0.0 * bias[o];"),
    "k and v swapped": ("double* dst = o < C ? q : (o < 2 * C ? k : v);", "double* dst = o < C ? q : (o < 2 * C ? v : k);"),
}

PINS = [
    lambda: test_matches_torch_layer_norm_and_matmul((2, 5, 7, 6), 1e-5),
    test_unit_affine_identity_projection_gives_standardised_tokens,
    test_invariant_to_per_token_shift_and_scale,
    test_constant_token_gives_beta,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "rib_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor missing: {old}"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = oracle.compile_oracle(str(mut), str(tmp_path / "libmut.so"))
    caught = 0
    with oracle.using(so):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught += 1
    assert caught > 0, f"no pin caught the planted mistake '{name}'"
