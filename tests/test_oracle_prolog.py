"""Pins of the indexer-prolog oracle: torch's RMSNorm in float64, closed forms, exact integer
projections against Python integer arithmetic, and the column layout of the fused weight
matrix through an identity weight."""
import math

import numpy as np
import pytest

import oracle


def bf16_bits(a):
    return oracle.encode_bf16_rne(np.asarray(a, dtype=np.float32))


def test_rms_norm_matches_torch_float64():
    import torch
    rng = np.random.default_rng(1)
    v = rng.standard_normal((7, 128)) * rng.uniform(0.01, 100, (7, 1))
    g = rng.uniform(0.5, 2.0, 128)
    for eps in (0.0, 1e-6, 1e-2):
        want = torch.nn.functional.rms_norm(torch.from_numpy(v), (128,), torch.from_numpy(g), eps).numpy()
        assert np.allclose(oracle.rms_norm(v, g, eps), want, rtol=1e-14, atol=0)


def test_rms_norm_closed_forms():
    # [3, 4]: mean square 12.5
    k = oracle.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    assert np.allclose(k, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)
    # a constant row c: c / sqrt(c^2 + eps) * gain
    c, eps = -2.5, 0.75
    g = np.array([1.0, 2.0, -3.0, 0.5])
    k = oracle.rms_norm(np.full((1, 4), c), g, eps)
    assert np.allclose(k, c / math.sqrt(c * c + eps) * g, rtol=1e-15)
    # without eps the result does not depend on a positive scale of the row
    v = np.random.default_rng(2).standard_normal((3, 64))
    assert np.allclose(oracle.rms_norm(v * 37.0, np.ones(64), 0.0), oracle.rms_norm(v, np.ones(64), 0.0),
                       rtol=1e-13)


def test_projection_is_exact_on_small_integers():
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, (5, 40))
    W = rng.integers(-8, 9, (40, 23))
    Y = oracle.project(bf16_bits(x), bf16_bits(W))
    want = [[sum(int(x[i, k]) * int(W[k, j]) for k in range(40)) for j in range(23)] for i in range(5)]
    assert np.array_equal(Y, np.array(want, dtype=np.float64))


def test_projection_matches_fsum_on_random_bf16():
    rng = np.random.default_rng(4)
    xb = bf16_bits(rng.standard_normal((3, 50)))
    Wb = bf16_bits(rng.standard_normal((50, 7)))
    x, W = oracle.decode_bf16(xb), oracle.decode_bf16(Wb)
    Y = oracle.project(xb, Wb)
    for i in range(3):
        for j in range(7):
            assert abs(Y[i, j] - math.fsum(x[i, k] * W[k, j] for k in range(50))) <= 1e-12


@pytest.mark.parametrize("H,D", [(2, 4), (4, 8)])
def test_column_layout_through_an_identity_weight(H, D):
    """With W the identity the outputs are slices of x: q[t, h, d] = x[t, h D + d], the key
    columns follow the query's, then the head weights."""
    N = H * D + D + H
    rng = np.random.default_rng(H)
    xb = bf16_bits(rng.standard_normal((3, N)))
    x = oracle.decode_bf16(xb)
    g = rng.uniform(0.5, 1.5, D)
    q, k, w = oracle.indexer_prolog(xb, bf16_bits(np.eye(N)), g, 1e-6, H, D)
    for t in range(3):
        for h in range(H):
            for d in range(D):
                assert q[t, h, d] == x[t, h * D + d]
    assert np.array_equal(w, x[:, H * D + D:])
    kr = x[:, H * D:H * D + D]
    assert np.allclose(k, kr / np.sqrt(np.mean(kr ** 2, axis=1, keepdims=True) + 1e-6) * g, rtol=1e-15)
