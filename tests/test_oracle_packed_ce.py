"""Pins of the packed-loss oracle (oracle.packed_ce) against what the pages
and the mathematics fix, independently of the oracle's own code.

Masked sequence packing re-weights the loss so that packed training computes
what unpacked training (one example per padded row) computes (zhao9797 page
"LWM (Large World Model)", 数据 and 训练方法 with its ablation table).  The
unpacked objective is written here with torch's own cross_entropy and
autograd on each example separately."""
import math

import numpy as np
import pytest


def _case(rng, B, S, V, n_docs, ignore_frac=0.3):
    x = rng.standard_normal((B * S, V)) * 2.0
    cuts = np.sort(rng.choice(np.arange(1, S), size=n_docs - 1, replace=False))
    seg_row = np.zeros(S, dtype=np.int32)
    for c in cuts:
        seg_row[c:] += 1
    seg = np.tile(seg_row, (B, 1))
    tg = rng.integers(0, V, size=B * S)
    tg[rng.random(B * S) < ignore_frac] = -100
    return x, tg, seg


def unpacked_reference(x, tg, seg, num_segments, grad_scale=1.0):
    """Each example alone: torch cross_entropy (mean over its loss rows, with
    ignore_index), then the mean over examples with a loss row; gradient by
    autograd."""
    import torch

    B, S = seg.shape
    V = x.shape[1]
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tgt = torch.tensor(np.where((tg >= 0) & (tg < V), tg, -100), dtype=torch.int64)
    losses = []
    for b in range(B):
        for e in range(num_segments):
            rows = [b * S + s for s in range(S) if seg[b, s] == e and tgt[b * S + s] >= 0]
            if rows:
                r = torch.tensor(rows)
                losses.append(torch.nn.functional.cross_entropy(xt[r], tgt[r], reduction="mean"))
    if not losses:
        return 0.0, np.zeros_like(x)
    loss = torch.stack(losses).mean()
    (grad_scale * loss).backward()
    return float(loss.detach()), xt.grad.numpy()


@pytest.mark.parametrize("B,S,V,n_docs", [(1, 40, 7, 4), (2, 33, 11, 5), (1, 64, 3, 1), (3, 20, 9, 6)])
def test_packed_equals_unpacked_torch(oracle, B, S, V, n_docs):
    rng = np.random.default_rng(B * 100 + S + V)
    x, tg, seg = _case(rng, B, S, V, n_docs)
    loss, ce, dl = oracle.packed_ce(x, tg, seg, n_docs, grad_scale=0.75)
    rl, rg = unpacked_reference(x, tg, seg, n_docs, grad_scale=0.75)
    assert abs(loss - rl) <= 1e-12 * max(1.0, abs(rl))
    np.testing.assert_allclose(dl, rg, rtol=0, atol=1e-14)


def test_hand_example(oracle):
    """V = 3, a row (0, 0, ln 2) has logsumexp ln 4: target 2 costs ln 2 and
    target 0 costs ln 4.  Example 0 holds (ln 2, ln 4), example 1 holds
    (ln 4) and one row without loss: loss = ((ln 2 + ln 4) / 2 + ln 4) / 2
    = 1.75 ln 2."""
    row = [0.0, 0.0, math.log(2.0)]
    x = np.array([row, row, row, row])
    tg = np.array([2, 0, 0, -1])
    seg = np.array([[0, 0, 1, 1]])
    loss, ce, dl = oracle.packed_ce(x, tg, seg, 2)
    assert abs(loss - 1.75 * math.log(2.0)) < 1e-15
    np.testing.assert_allclose(ce, [math.log(2), math.log(4), math.log(4), 0.0], atol=1e-15)
    p = np.array([0.25, 0.25, 0.5])
    # weights 1 / (E n_e): E = 2; n_0 = 2, n_1 = 1
    np.testing.assert_allclose(dl[0], (p - [0, 0, 1]) / 4, atol=1e-15)
    np.testing.assert_allclose(dl[1], (p - [1, 0, 0]) / 4, atol=1e-15)
    np.testing.assert_allclose(dl[2], (p - [1, 0, 0]) / 2, atol=1e-15)
    assert not dl[3].any()


def test_uniform_logits_closed_form(oracle):
    """Equal logits: every loss row costs ln V, so the loss is ln V whatever
    the packing, and the gradient is (1/V - onehot) / (E n_e)."""
    rng = np.random.default_rng(3)
    V = 13
    x, tg, seg = _case(rng, 1, 50, V, 5)
    x[:] = 0.7
    loss, ce, dl = oracle.packed_ce(x, tg, seg, 5)
    assert abs(loss - math.log(V)) < 1e-13
    keys = [(seg[0, t], t) for t in range(50) if tg[t] >= 0]
    E = len({k for k, _ in keys})
    for t in range(50):
        if tg[t] < 0:
            assert not dl[t].any()
            continue
        n_e = sum(1 for k, _ in keys if k == seg[0, t])
        want = np.full(V, 1.0 / V)
        want[tg[t]] -= 1.0
        np.testing.assert_allclose(dl[t], want / (E * n_e), atol=1e-15)


def test_gradient_by_central_differences(oracle):
    rng = np.random.default_rng(11)
    x, tg, seg = _case(rng, 1, 24, 6, 3)
    _, _, dl = oracle.packed_ce(x, tg, seg, 3, grad_scale=2.0)
    h = 1e-6
    for t, j in [(0, 0), (5, 3), (11, 5), (17, 1), (23, 2)]:
        xp, xm = x.copy(), x.copy()
        xp[t, j] += h
        xm[t, j] -= h
        fd = (oracle.packed_ce(xp, tg, seg, 3)[0] - oracle.packed_ce(xm, tg, seg, 3)[0]) / (2 * h)
        assert abs(2.0 * fd - dl[t, j]) < 1e-8, (t, j)


def test_rows_without_loss_and_out_of_range_ids(oracle):
    rng = np.random.default_rng(5)
    V = 8
    x, tg, seg = _case(rng, 1, 30, V, 3, ignore_frac=0.0)
    base = oracle.packed_ce(x, tg, seg, 3)
    # a target outside [0, V) or a segment id outside [0, num_segments) removes the row
    tg2, seg2 = tg.copy(), seg.copy()
    tg2[4] = V
    seg2[0, 9] = -1
    seg2[0, 10] = 3
    loss, ce, dl = oracle.packed_ce(x, tg2, seg2, 3)
    for t in (4, 9, 10):
        assert ce[t] == 0.0 and not dl[t].any()
    # same as dropping those rows by marking their targets
    tg3 = tg.copy()
    tg3[[4, 9, 10]] = -1
    loss3 = oracle.packed_ce(x, tg3, seg, 3)[0]
    assert abs(loss - loss3) < 1e-14 and abs(loss - base[0]) > 1e-6
    # no loss row at all: loss 0 and no gradient
    loss0, ce0, dl0 = oracle.packed_ce(x, np.full_like(tg, -1), seg, 3)
    assert loss0 == 0.0 and not ce0.any() and not dl0.any()


def test_batch_rows_are_separate_examples(oracle):
    """The same id in two batch rows names two examples: E counts both."""
    V = 5
    x = np.zeros((4, V))
    x[:, 0] = [1.0, 2.0, 3.0, 4.0]
    tg = np.array([0, 0, 0, 1])
    seg = np.array([[0, 0], [0, 0]])
    loss, ce, _ = oracle.packed_ce(x, tg, seg, 1)
    assert abs(loss - 0.5 * ((ce[0] + ce[1]) / 2 + (ce[2] + ce[3]) / 2)) < 1e-15


def test_naive_packing_differs_only_with_unequal_counts(oracle):
    """Re-weighting matters exactly when examples have different numbers of
    loss rows: with equal counts the token mean of the row is the same loss."""
    rng = np.random.default_rng(9)
    V = 10
    x = rng.standard_normal((24, V))
    tg = rng.integers(0, V, size=24)
    seg_eq = np.array([[0] * 8 + [1] * 8 + [2] * 8])
    loss, ce, _ = oracle.packed_ce(x, tg, seg_eq, 3)
    assert abs(loss - ce.mean()) < 1e-14
    seg_uneq = np.array([[0] * 2 + [1] * 20 + [2] * 2])
    loss_u, ce_u, _ = oracle.packed_ce(x, tg, seg_uneq, 3)
    assert abs(loss_u - ce_u.mean()) > 1e-3


def test_gradient_rows_subset(oracle):
    rng = np.random.default_rng(2)
    x, tg, seg = _case(rng, 2, 16, 6, 3)
    full = oracle.packed_ce(x, tg, seg, 3)[2]
    rows = np.array([31, 0, 7, 16])
    part = oracle.packed_ce(x, tg, seg, 3, grad_rows=rows)[2]
    np.testing.assert_array_equal(part, full[rows])
