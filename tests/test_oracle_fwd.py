"""Pins of the oracle's forward: hand values, torch's scaled_dot_product_attention
in float64 (a library routine for the same definition), closed forms, and the
invariants the pages state (exactness of the blockwise method independent of
block size and ring order; packed-with-mask equals unpacked)."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from test_oracle_rope import complex_rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def mask_matrix(S, seg_b, causal):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = np.ones((S, S), bool)
    if causal:
        m &= j <= i
    if seg_b is not None:
        m &= seg_b[:, None] == seg_b[None, :]
    return m


def torch_reference(q, k, v, seg, pos, theta, causal, scale=None):
    """float64 SDPA with an explicit boolean mask; RoPE as complex rotation."""
    B, H, S, D = q.shape
    if pos is None:
        pos = np.tile(np.arange(S, dtype=np.int32), (B, 1))
    if theta > 0:
        q = complex_rope(q, pos[:, None, :], theta)
        k = complex_rope(k, pos[:, None, :], theta)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    o = np.empty((B, H, S, D))
    lse = np.empty((B, H, S))
    for b in range(B):
        m = torch.from_numpy(mask_matrix(S, None if seg is None else seg[b], causal))
        qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x[b])) for x in (q, k, v))
        o[b] = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale).numpy()
        s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
        lse[b] = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1).numpy()
    return o, lse


def test_hand_values(oracle):
    g = json.load(open(os.path.join(GOLDEN, "attn_hand.json")))
    q, k, v = (np.array(g[n])[None, None] for n in ("q", "k", "v"))
    for key, causal in (("causal", True), ("noncausal", False)):
        o, lse = oracle.attn_fwd(q, k, v, theta=0.0, causal=causal)
        np.testing.assert_allclose(o[0, 0], g[key]["o"], atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], g[key]["lse"], atol=1e-14)
    cs = g["causal_segments"]
    seg = np.array([cs["segment_ids"]], dtype=np.int32)
    o, lse = oracle.attn_fwd(q, k, v, segment_ids=seg, theta=0.0, causal=True)
    np.testing.assert_allclose(o[0, 0], cs["o"], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], cs["lse"], atol=1e-14)
    # the default scale is 1/sqrt(D): passing it explicitly changes nothing
    o2, _ = oracle.attn_fwd(q, k, v, theta=0.0, scale=g["scale"], causal=True)
    np.testing.assert_allclose(o2[0, 0], g["causal"]["o"], atol=1e-14)


@pytest.mark.parametrize("S,D,n_docs,causal,theta", [
    (1, 8, 0, True, 1e4), (7, 8, 0, True, 0.0), (37, 16, 0, True, 1e6), (64, 64, 3, True, 1e7),
    (50, 32, 4, False, 1e4), (129, 128, 0, False, 5e7), (96, 64, 5, True, 5e7)])
def test_matches_torch_sdpa(oracle, S, D, n_docs, causal, theta):
    rng = np.random.default_rng(S * 1000 + D)
    B, H = 2, 2
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    seg = None
    pos = rng.integers(0, 1 << 20, size=(B, S)).astype(np.int32)
    if n_docs:
        seg = np.sort(rng.integers(0, n_docs, size=(B, S)), axis=1).astype(np.int32)
    o, lse = oracle.attn_fwd(q, k, v, seg, pos, theta=theta, causal=causal)
    ro, rlse = torch_reference(q, k, v, seg, pos, theta, causal)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, atol=1e-12)


def test_noncontiguous_segment_ids(oracle):
    """Equality of ids defines the mask, whether or not a segment is contiguous."""
    rng = np.random.default_rng(9)
    B, H, S, D = 1, 2, 40, 16
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    seg = rng.integers(0, 3, size=(B, S)).astype(np.int32)
    seg[0, 0] = seg[0, 1]
    for causal in (True, False):
        o, lse = oracle.attn_fwd(q, k, v, seg, None, theta=1e4, causal=causal)
        ro, rlse = torch_reference(q, k, v, seg, None, 1e4, causal)
        np.testing.assert_allclose(o, ro, atol=1e-12)
        np.testing.assert_allclose(lse, rlse, atol=1e-12)


def test_zero_queries_give_prefix_means(oracle):
    """q = 0: every visible score is 0, so O_i is the mean of the visible v_j
    and LSE_i = ln(count_i)."""
    rng = np.random.default_rng(10)
    B, H, S, D = 1, 2, 300, 32
    lengths = [100, 1, 150, 49]
    seg = np.concatenate([np.full(L, d, np.int32) for d, L in enumerate(lengths)])[None]
    q = np.zeros((B, H, S, D))
    k, v = rng.standard_normal((B, H, S, D)), rng.standard_normal((B, H, S, D))
    o, lse = oracle.attn_fwd(q, k, v, seg, None, theta=1e6, causal=True)
    start = 0
    for L in lengths:
        csum = np.cumsum(v[:, :, start:start + L], axis=2)
        cnt = np.arange(1, L + 1)[None, None, :, None]
        np.testing.assert_allclose(o[:, :, start:start + L], csum / cnt, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, start:start + L], np.log(cnt[..., 0]) + 0 * lse[:, :, start:start + L],
                                   atol=1e-12)
        start += L


def test_singleton_segments_and_single_token(oracle):
    rng = np.random.default_rng(11)
    B, H, S, D = 1, 2, 20, 16
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    seg = np.arange(S, dtype=np.int32)[None]
    o, lse = oracle.attn_fwd(q, k, v, seg, None, theta=0.0, causal=False)
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse, np.sum(q * k, axis=-1) / np.sqrt(D), atol=1e-12)
    o1, _ = oracle.attn_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], theta=1e4)
    np.testing.assert_allclose(o1, v[:, :, :1], atol=1e-14)


def test_probability_rows_sum_to_one(oracle):
    """With v = identity rows (S = D), O_i is the probability row P_i."""
    rng = np.random.default_rng(12)
    S = D = 64
    q, k = rng.standard_normal((1, 1, S, D)), rng.standard_normal((1, 1, S, D))
    v = np.eye(S)[None, None]
    for causal in (True, False):
        P, _ = oracle.attn_fwd(q, k, v, None, None, theta=1e4, causal=causal)
        np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-13)
        assert np.all(P >= 0)
        if causal:
            assert np.all(np.triu(P[0, 0], 1) == 0)


@pytest.mark.parametrize("block_k", [1, 3, 64, 200])
@pytest.mark.parametrize("kv_chunk", [0, 32, 50])
def test_blocked_matches_naive(oracle, block_k, kv_chunk):
    """The blockwise online softmax reaches the exact result for any block size
    and in ring order (the method is exact: elamur.ai summary; ring of K/V
    blocks: zhao9797 page, 模型架构)."""
    rng = np.random.default_rng(13)
    B, H, S, D = 1, 2, 200, 32
    q, k, v = (rng.standard_normal((B, H, S, D)) * 2 for _ in range(3))
    seg = np.sort(rng.integers(0, 4, size=(B, S)), axis=1).astype(np.int32)
    for causal in (True, False):
        o, lse = oracle.attn_fwd(q, k, v, seg, None, theta=1e6, causal=causal)
        ob, lseb = oracle.attn_fwd_blocked(q, k, v, seg, None, theta=1e6, causal=causal, block_k=block_k,
                                           kv_chunk=kv_chunk)
        np.testing.assert_allclose(ob, o, atol=1e-12)
        np.testing.assert_allclose(lseb, lse, atol=1e-12)


def test_packed_equals_unpacked(oracle):
    """Masked packing is numerically equivalent to running each document alone
    (zhao9797 page, 训练方法, Masked Sequence Packing); positions restart."""
    rng = np.random.default_rng(14)
    lengths = [37, 5, 90, 1, 60]
    S, D, H = sum(lengths), 64, 2
    q, k, v = (rng.standard_normal((1, H, S, D)) for _ in range(3))
    seg = np.concatenate([np.full(L, d, np.int32) for d, L in enumerate(lengths)])[None]
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lengths])[None]
    o, lse = oracle.attn_fwd(q, k, v, seg, pos, theta=1e7, causal=True)
    start = 0
    for L in lengths:
        sl = slice(start, start + L)
        od, lsed = oracle.attn_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], None, None, theta=1e7, causal=True)
        np.testing.assert_allclose(o[:, :, sl], od, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, sl], lsed, atol=1e-12)
        start += L


def test_shifted_positions_change_nothing(oracle):
    """Scores depend only on relative positions, so shifting every position
    by the same amount leaves O and LSE unchanged."""
    rng = np.random.default_rng(15)
    B, H, S, D = 1, 2, 64, 128
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    pos = np.arange(S, dtype=np.int32)[None]
    o0, l0 = oracle.attn_fwd(q, k, v, None, pos, theta=5e7)
    o1, l1 = oracle.attn_fwd(q, k, v, None, pos + 12345, theta=5e7)
    np.testing.assert_allclose(o1, o0, atol=1e-9)
    np.testing.assert_allclose(l1, l0, atol=1e-9)


def test_row_subset_matches_full(oracle):
    rng = np.random.default_rng(16)
    B, H, S, D = 2, 2, 70, 16
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    rows = np.array([0, 69, 33, 34, 5])
    o, lse = oracle.attn_fwd(q, k, v, theta=1e4)
    os_, ls = oracle.attn_fwd(q, k, v, theta=1e4, rows=rows)
    np.testing.assert_array_equal(os_, o[:, :, rows])
    np.testing.assert_array_equal(ls, lse[:, :, rows])
