"""Pins of the oracle's backward: hand values, torch autograd through a float64
attention written with library ops, central finite differences, and closed
forms."""
import json
import os

import numpy as np
import pytest
import torch

from test_oracle_fwd import mask_matrix

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_grads(q, k, v, dout, seg, pos, theta, causal):
    """Gradients by torch autograd of float64 masked softmax attention with
    RoPE written as complex multiplication."""
    B, H, S, D = q.shape
    if pos is None:
        pos = np.tile(np.arange(S, dtype=np.int32), (B, 1))
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))

    def rot(x):
        if theta <= 0:
            return x
        w = theta ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
        ang = torch.from_numpy(pos.astype(np.float64))[:, None, :, None] * w
        z = torch.complex(x[..., 0::2], x[..., 1::2]) * torch.polar(torch.ones_like(ang), ang)
        return torch.stack([z.real, z.imag], dim=-1).reshape(x.shape)

    qr, kr = rot(qt), rot(kt)
    m = torch.from_numpy(np.stack([mask_matrix(S, None if seg is None else seg[b], causal) for b in range(B)]))
    s = torch.matmul(qr, kr.transpose(-1, -2)) / np.sqrt(D)
    s = s.masked_fill(~m[:, None], float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vt)
    (o * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_hand_values(oracle):
    g = json.load(open(os.path.join(GOLDEN, "attn_hand.json")))
    q, k, v = (np.array(g[n])[None, None] for n in ("q", "k", "v"))
    dout = np.array(g["bwd"]["dout"])[None, None]
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, theta=0.0, causal=True)
    np.testing.assert_allclose(dq[0, 0], g["bwd"]["dq"], atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], g["bwd"]["dk"], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], g["bwd"]["dv"], atol=1e-14)


@pytest.mark.parametrize("S,D,n_docs,causal,theta", [
    (1, 8, 0, True, 1e4), (9, 8, 0, True, 0.0), (40, 16, 0, True, 1e6), (64, 64, 3, True, 1e7),
    (33, 32, 4, False, 1e4), (70, 128, 2, True, 5e7)])
def test_matches_torch_autograd(oracle, S, D, n_docs, causal, theta):
    rng = np.random.default_rng(S + 7 * D)
    B, H = 2, 2
    q, k, v, dout = (rng.standard_normal((B, H, S, D)) for _ in range(4))
    pos = rng.integers(0, 1 << 20, size=(B, S)).astype(np.int32)
    seg = np.sort(rng.integers(0, n_docs, size=(B, S)), axis=1).astype(np.int32) if n_docs else None
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, seg, pos, theta=theta, causal=causal)
    rq, rk, rv = torch_grads(q, k, v, dout, seg, pos, theta, causal)
    np.testing.assert_allclose(dq, rq, atol=1e-11)
    np.testing.assert_allclose(dk, rk, atol=1e-11)
    np.testing.assert_allclose(dv, rv, atol=1e-11)


def test_finite_differences(oracle):
    """Central differences of L = <dO, O> in float64 on a tiny case."""
    rng = np.random.default_rng(21)
    B, H, S, D = 1, 1, 6, 4
    q, k, v, dout = (rng.standard_normal((B, H, S, D)) for _ in range(4))
    seg = np.array([[0, 0, 0, 1, 1, 1]], np.int32)
    pos = np.array([[0, 1, 2, 0, 1, 2]], np.int32)
    theta = 100.0
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, seg, pos, theta=theta)

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd(q_, k_, v_, seg, pos, theta=theta)
        return float(np.sum(o * dout))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_constant_values_give_zero_qk_gradients(oracle):
    """v_j = c for all j: O = c whatever P is, so dq = dk = 0."""
    rng = np.random.default_rng(22)
    B, H, S, D = 1, 2, 50, 16
    q, k, dout = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    v = np.broadcast_to(rng.standard_normal(D), (B, H, S, D)).copy()
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, None, None, theta=1e6)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)
    # the value gradients still sum over rows the probabilities: sum_j dv_j = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=2), dout.sum(axis=2), atol=1e-12)


def test_zero_queries_closed_form(oracle):
    """q = 0: P_ij = 1/count_i, dk = 0, dv_j = sum_{i>=j} dO_i / count_i."""
    rng = np.random.default_rng(23)
    B, H, S, D = 1, 2, 80, 16
    q = np.zeros((B, H, S, D))
    k, v, dout = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, None, None, theta=1e6)
    np.testing.assert_allclose(dk, 0, atol=1e-13)
    cnt = np.arange(1, S + 1)[None, None, :, None]
    np.testing.assert_allclose(dv, np.cumsum((dout / cnt)[:, :, ::-1], axis=2)[:, :, ::-1], atol=1e-12)


def test_key_gradients_sum_to_zero_without_rope(oracle):
    """Each row's dS sums to zero (softmax is shift invariant), so without RoPE
    the key gradients of a segment sum to zero."""
    rng = np.random.default_rng(24)
    B, H, S, D = 1, 2, 60, 16
    q, k, v, dout = (rng.standard_normal((B, H, S, D)) for _ in range(4))
    seg = np.repeat(np.arange(3, dtype=np.int32), 20)[None]
    _, dk, _ = oracle.attn_bwd(q, k, v, dout, seg, None, theta=0.0)
    for d in range(3):
        np.testing.assert_allclose(dk[:, :, 20 * d:20 * d + 20].sum(axis=2), 0, atol=1e-12)


def test_row_and_column_windows(oracle):
    """dq of listed rows equals the full result; dk/dv of the last columns
    need only the rows that see them."""
    rng = np.random.default_rng(25)
    B, H, S, D = 1, 2, 90, 16
    q, k, v, dout = (rng.standard_normal((B, H, S, D)) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, None, None, theta=1e4)
    rows = np.array([0, 89, 45])
    dqs, _, _ = oracle.attn_bwd(q, k, v, dout, None, None, theta=1e4, rows=rows, col_begin=0, col_end=0)
    np.testing.assert_allclose(dqs, dq[:, :, rows], atol=1e-13)
    tail = np.arange(60, 90)
    _, dkt, dvt = oracle.attn_bwd(q, k, v, dout, None, None, theta=1e4, rows=tail, col_begin=60, col_end=90)
    np.testing.assert_allclose(dkt, dk[:, :, 60:], atol=1e-13)
    np.testing.assert_allclose(dvt, dv[:, :, 60:], atol=1e-13)


@pytest.mark.parametrize("n_docs,causal,theta", [(0, True, 1e6), (3, True, 1e7), (2, False, 0.0)])
def test_probability_matrices_against_the_backward(oracle, n_docs, causal, theta):
    """attn_probs (numpy) against the C oracle: P v = O, rows of P sum to 1,
    rows of dS sum to 0, dv = P^T dO, dq = R(-a) scale dS k' and
    dk = R(-a) scale dS^T q'."""
    from long_context_blockwise_attn_amd.inputs import random_case

    S, D = 150, 32
    (q, k, v, do), seg, pos = random_case(1, 2, S, D, seed=19 + n_docs, n_docs=n_docs, dtype="fp32")
    q, k, v, do = (x.double().numpy() for x in (q, k, v, do))
    P, dS, qr, kr = oracle.attn_probs(q, k, v, do, seg, pos, theta=theta, causal=causal)
    o, _ = oracle.attn_fwd(q, k, v, seg, pos, theta=theta, causal=causal)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, seg, pos, theta=theta, causal=causal)
    np.testing.assert_allclose(P @ v, o, atol=1e-12)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-13)
    np.testing.assert_allclose(dS.sum(-1), 0.0, atol=1e-11)
    np.testing.assert_allclose(np.swapaxes(P, -1, -2) @ do, dv, atol=1e-12)
    tau = 1.0 / np.sqrt(D)
    back = (lambda x: oracle.rope(x, pos, theta, inverse=True)) if theta > 0 else (lambda x: x)
    np.testing.assert_allclose(back(tau * dS @ kr), dq, atol=1e-11)
    np.testing.assert_allclose(back(tau * np.swapaxes(dS, -1, -2) @ qr), dk, atol=1e-11)
