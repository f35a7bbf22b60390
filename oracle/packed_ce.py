"""Oracle for the loss side of masked sequence packing, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

Masked sequence packing (zhao9797 page "LWM (Large World Model)", 数据 and
训练方法; its ablation table): short examples are packed into one training
row, attention is masked to each example, and the loss is re-weighted so that
packed training computes what training on the same examples unpacked, one per
padded row, computes.  Naive packing instead averages over all tokens of the
row and so gives a short answer less weight than a long one.  The pages give
no formula; the reading taken here is the usual unpacked objective: each
example's loss is the mean cross-entropy over its own loss tokens, and the
batch loss is the mean of those per-example losses over the examples that
have at least one loss token.

Conventions:
  - logits [N, V] (N = B * S token rows, row t = b * S + s);
  - targets [N] int: the target token of row t; values outside [0, V) mark a
    row without loss (the last token of an example, prompt tokens, padding);
  - segment_ids [B, S] int: example id of each token, an example being the
    pair (b, id) with 0 <= id < num_segments; tokens with ids outside that
    range carry no loss;
  - the cross-entropy of a loss row is logsumexp(logits[t]) - logits[t, y_t].
"""
from __future__ import annotations

import numpy as np


def _examples(targets, segment_ids, num_segments, V):
    """Loss-token mask [N] and example key [N] (b * num_segments + id, -1 for
    rows without loss)."""
    seg = np.asarray(segment_ids, dtype=np.int64)
    B, S = seg.shape
    tg = np.asarray(targets, dtype=np.int64).reshape(B * S)
    b = np.repeat(np.arange(B, dtype=np.int64), S)
    sid = seg.reshape(B * S)
    loss_row = (tg >= 0) & (tg < V) & (sid >= 0) & (sid < num_segments)
    key = np.where(loss_row, b * num_segments + sid, -1)
    return loss_row, key


def token_ce(logits, targets, rows):
    """Cross-entropy logsumexp(x_t) - x_t[y_t] of the given rows, float64."""
    x = np.asarray(logits[rows], dtype=np.float64)
    m = x.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))[:, 0]
    y = np.asarray(targets, dtype=np.int64).reshape(-1)[rows]
    return lse - x[np.arange(len(rows)), y]


def packed_ce(logits, targets, segment_ids, num_segments, grad_scale=1.0, grad_rows=None, chunk=2048):
    """Loss, per-row cross-entropy and gradient of the re-weighted packed loss.

    Returns (loss, ce, dlogits):
      loss     mean over examples e of (mean over e's loss rows of ce_t);
      ce       [N] cross-entropy of each loss row, 0 elsewhere;
      dlogits  grad_scale * d loss / d logits for the rows in grad_rows
               (all rows when None), shape [len(grad_rows), V]: for a loss row
               of example e, (softmax(x_t) - onehot(y_t)) / (E * n_e), where E
               is the number of examples and n_e the loss rows of e; zero for
               rows without loss.
    The per-example sums are formed example by example, as written."""
    logits = np.asarray(logits)
    N, V = logits.shape
    loss_row, key = _examples(targets, segment_ids, num_segments, V)
    ce = np.zeros(N, dtype=np.float64)
    idx = np.nonzero(loss_row)[0]
    for c0 in range(0, len(idx), chunk):
        r = idx[c0:c0 + chunk]
        ce[r] = token_ce(logits, targets, r)
    # per-example mean, then the mean over examples
    keys = np.unique(key[loss_row])
    E = len(keys)
    per_example = []
    n_of = {}
    for k in keys:
        rows_k = np.nonzero(key == k)[0]
        n_of[int(k)] = len(rows_k)
        per_example.append(ce[rows_k].sum() / len(rows_k))
    loss = float(np.mean(per_example)) if E else 0.0
    if grad_rows is None:
        grad_rows = np.arange(N)
    grad_rows = np.asarray(grad_rows, dtype=np.int64)
    dl = np.zeros((len(grad_rows), V), dtype=np.float64)
    tg = np.asarray(targets, dtype=np.int64).reshape(-1)
    for i, t in enumerate(grad_rows):
        if not loss_row[t]:
            continue
        x = np.asarray(logits[t], dtype=np.float64)
        p = np.exp(x - x.max())
        p /= p.sum()
        p[tg[t]] -= 1.0
        dl[i] = grad_scale * p / (E * n_of[int(key[t])])
    return loss, ce, dl
