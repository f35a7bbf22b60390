"""Pins of the oracle's RoPE ("standard RoPE" with base theta: zhao9797 page,
模型架构; RoFormer) against hand values, a complex-number formulation and the
rotation's invariants."""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def complex_rope(x, pos, theta):
    """Rotation written as complex multiplication: z_i = x[2i] + 1j x[2i+1]
    times exp(1j * pos * theta^(-2i/D))."""
    D = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    w = theta ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = pos[..., None].astype(np.float64) * w
    z = z * np.exp(1j * ang)
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def test_hand_values(oracle):
    g = json.load(open(os.path.join(GOLDEN, "rope_hand.json")))
    for case in g["cases"]:
        D = case["D"]
        if "x" in case:
            x = np.array(case["x"], dtype=np.float64).reshape(1, 1, 1, D)
            pos = np.array([[case["pos"]]], dtype=np.int32)
            y = oracle.rope(x, pos, case["theta"])
            np.testing.assert_allclose(y.ravel(), case["y"], rtol=0, atol=1e-15)
        else:
            i = case["pair"]
            x = np.zeros((1, 1, 1, D))
            x[..., 2 * i] = 1.0
            pos = np.array([[case["pos"]]], dtype=np.int32)
            y = oracle.rope(x, pos, case["theta"]).ravel()
            assert abs(np.arctan2(y[2 * i + 1], y[2 * i]) - case["angle"]) < 1e-14
            # the other pairs stay zero
            mask = np.ones(D, bool)
            mask[2 * i:2 * i + 2] = False
            assert np.all(y[mask] == 0.0)


@pytest.mark.parametrize("theta", [1e4, 1e6, 1e7, 5e7])
def test_matches_complex_form(oracle, theta):
    rng = np.random.default_rng(0)
    B, H, S, D = 2, 3, 17, 128
    x = rng.standard_normal((B, H, S, D))
    pos = rng.integers(0, 1 << 20, size=(B, S)).astype(np.int32)
    y = oracle.rope(x, pos, theta)
    ref = complex_rope(x, pos[:, None, :], theta)
    # angles up to 1e6 rad: fp64 argument error ~1e-10
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-9)


def test_default_positions_are_indices(oracle):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 2, 33, 64))
    pos = np.arange(33, dtype=np.int32)[None, :]
    np.testing.assert_array_equal(oracle.rope(x, None, 1e6), oracle.rope(x, pos, 1e6))


def test_position_zero_is_identity(oracle):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 2, 5, 64))
    pos = np.zeros((1, 5), dtype=np.int32)
    np.testing.assert_array_equal(oracle.rope(x, pos, 1e7), x)


def test_pair_norms_preserved_and_inverse(oracle):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 4, 50, 128))
    pos = rng.integers(0, 1 << 20, size=(1, 50)).astype(np.int32)
    y = oracle.rope(x, pos, 5e7)
    n_x = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_y = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n_y, n_x, rtol=1e-12)
    back = oracle.rope(y, pos, 5e7, inverse=True)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-12)


def test_scores_depend_on_relative_position_only(oracle):
    """<R_m q, R_n k> = <R_{m+d} q, R_{n+d} k> (RoFormer's defining property)."""
    rng = np.random.default_rng(4)
    D = 128
    q = rng.standard_normal((1, 1, 1, D))
    k = rng.standard_normal((1, 1, 1, D))
    for m, n, d in [(5, 3, 12345), (1000, 0, 1 << 19), (70000, 69999, 7)]:
        for theta in (1e4, 1e7, 5e7):
            a = np.dot(oracle.rope(q, np.array([[m]], np.int32), theta).ravel(),
                       oracle.rope(k, np.array([[n]], np.int32), theta).ravel())
            b = np.dot(oracle.rope(q, np.array([[m + d]], np.int32), theta).ravel(),
                       oracle.rope(k, np.array([[n + d]], np.int32), theta).ravel())
            assert abs(a - b) < 1e-9 * (1 + abs(a))
