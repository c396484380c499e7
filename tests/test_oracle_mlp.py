"""Pins of the oracle's two-layer compression (compress_mlp) against facts
that do not come from its own arithmetic: the linear compression (itself
pinned in test_oracle_pins) it reduces to, the ReLU identity
relu(a) - relu(-a) = a, a closed form for one-hot maps, and bf16
representability.  CPU only."""
import math

import numpy as np
import torch

from oracle import oracle as orc


def _case(T=100, B=2, H=2, dim=8, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, T, dim))
    W1 = rng.standard_normal((dim, 32 * dim)) / math.sqrt(32 * dim)
    PE = rng.standard_normal((32, dim)) / math.sqrt(dim)
    W2 = rng.standard_normal((dim, dim)) / math.sqrt(dim)
    return x, W1, PE, W2


def test_identity_second_layer_on_nonnegative_inputs_is_the_linear_map():
    # every pre-activation >= 0 (nonnegative x, PE, W1): relu is the identity
    x, W1, PE, _ = _case(seed=1)
    x, W1, PE = np.abs(x), np.abs(W1), np.abs(PE)
    I = np.eye(x.shape[-1])
    np.testing.assert_array_equal(orc.compress_mlp(x, W1, PE, I), orc.compress(x, W1, PE))


def test_negative_preactivations_give_zero():
    x, W1, PE, W2 = _case(seed=2)
    x, W1, PE = -np.abs(x) - 0.1, np.abs(W1) + 1e-3, -np.abs(PE)
    out = orc.compress_mlp(x, W1, PE, W2)
    assert out.shape[2] == orc.n_cmp(x.shape[2]) and np.all(out == 0.0)


def test_relu_identity_gives_the_composed_linear_map():
    # relu(a) - relu(-a) = a, so mlp(W1) - mlp(-W1) = W2 W1 vec(x + PE),
    # the linear compression with the product map W2 @ W1 (the only order
    # whose shape fits: [dim, dim] @ [dim, 32 dim])
    x, W1, PE, W2 = _case(seed=3)
    got = orc.compress_mlp(x, W1, PE, W2) - orc.compress_mlp(x, -W1, PE, W2)
    ref = orc.compress(x, W2 @ W1, PE)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_one_hot_maps_closed_form():
    # W1 row j picks token tau_j, channel e_j of the block; W2 a permutation:
    # out[i][c] = relu(x[16 i + tau_p(c)][e_p(c)] + PE[tau_p(c)][e_p(c)]),
    # p = the permutation (out[c] = h[p(c)]); a transposed W2 applies p^-1
    rng = np.random.default_rng(4)
    dim, T = 6, 80
    x = rng.standard_normal((1, 1, T, dim))
    PE = rng.standard_normal((32, dim)) * 0.3
    taus = rng.integers(0, 32, dim)
    es = rng.integers(0, dim, dim)
    W1 = np.zeros((dim, 32 * dim))
    W1[np.arange(dim), taus * dim + es] = 1.0
    perm = np.array([3, 0, 5, 1, 4, 2])
    W2 = np.zeros((dim, dim))
    W2[np.arange(dim), perm] = 1.0
    out = orc.compress_mlp(x, W1, PE, W2)
    for i in range(orc.n_cmp(T)):
        for c in range(dim):
            j = perm[c]
            a = x[0, 0, 16 * i + taus[j], es[j]] + PE[taus[j], es[j]]
            assert out[0, 0, i, c] == max(a, 0.0)


def test_bf16_rounding_points():
    # with rounding the output is bf16-representable and past N_cmp zero
    x, W1, PE, W2 = _case(seed=5)
    out = orc.compress_mlp(x, W1, PE, W2, n_out=64, round_bf16=True)
    t = torch.from_numpy(out)
    assert torch.equal(t.to(torch.bfloat16).double(), t)
    assert np.all(out[:, :, orc.n_cmp(x.shape[2]):] == 0.0)
    # and within one bf16 rounding (plus the rounded hidden layer) of the
    # unrounded network
    ref = orc.compress_mlp(x, W1, PE, W2, n_out=64)
    bound = np.abs(ref) * 2.0 ** -8 + (np.abs(W2) @ np.abs(orc.compress(x, W1, PE, n_out=64))[..., None])[..., 0] * 2.0 ** -8
    assert np.all(np.abs(out - ref) <= bound + 1e-12)
