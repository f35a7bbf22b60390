"""Closed forms of causal attention over one document with q = 0 (every
visible score 0, so row i attends uniformly to its c_i = i + 1 keys), in
float64, row chunk by row chunk:
  O_i = (1/c_i) sum_{j<=i} v_j,   LSE_i = ln c_i,   dk = 0,
  dv_j = sum_{i>=j} dO_i / c_i,
  dq_i = R(-a_i) (scale / c_i) [dO_i^T sum_{j<=i} v_j k'_j^T
                                - Delta_i sum_{j<=i} k'_j],
with Delta_i = <dO_i, O_i> and k'_j the key rotated at position j."""
import numpy as np


def prefix_sums(x, block=256):
    """Inclusive prefix sums of x [n, D] along the rows (blocks of rows summed
    by a product with a lower-triangular matrix of ones; numpy's cumsum
    along the first axis of a row-major array is slow at these sizes)."""
    n, D = x.shape
    out = np.empty_like(x)
    low = np.tril(np.ones((block, block)))
    carry = np.zeros(D)
    for b0 in range(0, n, block):
        b1 = min(n, b0 + block)
        out[b0:b1] = carry + low[:b1 - b0, :b1 - b0] @ x[b0:b1]
        carry = out[b1 - 1]
    return out


def zero_query_closed_forms(oracle, k, v, do, theta, scale, chunk_rows=1 << 16, block=512):
    """k, v, do: float64 [S, D] of one head (positions 0..S-1).  Yields
    (row slice, O, dv, dq) for consecutive row chunks."""
    S, D = v.shape
    cnt = np.arange(1, S + 1, dtype=np.float64)
    kr = oracle.rope(k[None, None], None, theta=theta)[0, 0] if theta > 0 else k
    y = do / cnt[:, None]
    suffix = y.sum(axis=0) - prefix_sums(y) + y  # sum_{i>=j} y_i
    carry_v = np.zeros(D)        # sum_{j < r0} v_j
    carry_m = np.zeros((D, D))   # sum_{j < b0} v_j k'_j^T
    carry_k = np.zeros(D)        # sum_{j < b0} k'_j
    for r0 in range(0, S, chunk_rows):
        r1 = min(S, r0 + chunk_rows)
        sl = slice(r0, r1)
        c = cnt[sl, None]
        o_ref = (carry_v + prefix_sums(v[sl])) / c
        delta = np.sum(do[sl] * o_ref, axis=1)
        dqp = np.empty((r1 - r0, D))
        # earlier rows through the carries, this block through the lower
        # triangle of dO V^T
        for b0 in range(r0, r1, block):
            b1 = min(r1, b0 + block)
            bs = slice(b0, b1)
            a = np.tril(do[bs] @ v[bs].T)
            ks = carry_k + prefix_sums(kr[bs])
            dqp[b0 - r0:b1 - r0] = do[bs] @ carry_m + a @ kr[bs] - delta[b0 - r0:b1 - r0, None] * ks
            carry_m += v[bs].T @ kr[bs]
            carry_k += kr[bs].sum(axis=0)
        dqp *= scale / c
        if theta > 0:
            pos = np.arange(r0, r1, dtype=np.int32)[None]
            dq_ref = oracle.rope(dqp[None, None], pos, theta=theta, inverse=True)[0, 0]
        else:
            dq_ref = dqp
        carry_v += v[sl].sum(axis=0)
        yield sl, o_ref, suffix[sl], dq_ref
