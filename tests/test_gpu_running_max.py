"""The lazy running max of the online softmax (zhao9797 page "LWM (Large
World Model)", 模型架构: blockwise attention merges each block's partial
result with a running max and sum, exactly).  The kernels raise a row's
running max m only when a tile's max exceeds it by more than 8 in log2
units; a raise rescales O and l and moves the start value of the later
score MFMAs.  Random inputs almost never need a raise after the first tile,
so in these cases every key before S/3 carries a bias of about -12 in log2
units (one dimension: q = C, k = -24): with the forward walking tiles in
increasing order (the decode each chunk so), every row that reaches the
unbiased keys raises its max once, mid-walk.  The bias is large but its
keys' probabilities are tiny, so the scores that matter stay of the usual
size.  Forward and decode (the kernels with a running max) against the
oracle; the backward recomputes P from the forward's LSE, checked here.
(Its gradients are not compared on these inputs: a key element of -24
multiplies the bf16 rounding of dS in dq's bias dimension, where the exact
sum cancels, and that alone exceeds the absolute bar.)"""
import math

import numpy as np
import pytest

from helpers import assert_parity, to64

# the bias sits in the last RoPE pair, which turns by less than 2e-3 rad over
# these positions at theta 1e6


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def bias_query_value(D):
    """A bf16 value C near 4 whose product with the softmax scale times
    log2(e) (the factor the kernels fold into the query rows before rounding
    them to bf16) rounds to bf16 with a relative error below 1e-4, so the
    bias term C * k / sqrt(D) loses next to nothing in the kernels' rounding
    and the small scores stay comparable to the oracle's."""
    import torch

    sl2 = np.float32(np.float32(1.0 / math.sqrt(D)) * np.float32(1.4426950408889634))
    exact = math.log2(math.e) / math.sqrt(D)
    cand = torch.arange(3.0, 5.0, 2.0 ** -6).to(torch.bfloat16).unique().double().numpy()
    y = (cand.astype(np.float32) * sl2).astype(np.float32)
    yb = torch.from_numpy(y).to(torch.bfloat16).double().numpy()
    rel = np.abs(yb / (cand * exact) - 1.0)
    i = int(np.argmin(rel))
    assert rel[i] < 1e-4, rel[i]
    return float(cand[i])


def rising_case(S, D, seed):
    from long_context_blockwise_attn_amd.inputs import random_case

    (q, k, v, _), _, pos = random_case(1, 2, S, D, seed)
    bd = D - 2
    q[..., bd] = bias_query_value(D)
    q[..., bd + 1] = 0.0
    k[..., bd + 1] = 0.0
    k[..., : S // 3, bd] = -24.0
    k[..., S // 3:, bd] = 0.0
    return q, k, v, pos


def raises_per_row(q, k, causal):
    """How often the lazy rule raises each row's running max after its first
    tile, tiles of 64 keys walked in increasing order (head 0, no RoPE,
    scores in fp64 from the bf16 inputs)."""
    s = to64(q)[0, 0] @ to64(k)[0, 0].T * (math.log2(math.e) / math.sqrt(q.shape[-1]))
    S = s.shape[0]
    out = np.zeros(S, dtype=np.int64)
    for i in range(S):
        last = i if causal else S - 1
        m = -np.inf
        for t0 in range(0, last + 1, 64):
            mx = s[i, t0:min(last + 1, t0 + 64)].max()
            if m == -np.inf:
                m = mx
            elif mx > m + 8.0:
                m = mx
                out[i] += 1
    return out


def test_inputs_raise_the_running_max():
    """The inputs do what the GPU cases need (CPU only)."""
    for D in (128, 64):
        q, k, _, _ = rising_case(1000, D, seed=5)
        r = raises_per_row(q, k, causal=True)
        # every row that reaches the unbiased keys raises once; none before
        assert (r[: 1000 // 3] == 0).all()
        assert (r[1000 // 3 + 64:] >= 1).mean() > 0.9


@pytest.mark.gpu
@pytest.mark.parametrize("D,theta,causal,kv_chunk", [
    (128, 0.0, True, 0), (128, 1e6, True, 0), (128, 0.0, False, 0), (128, 1e6, True, 256), (64, 1e6, True, 0)])
def test_fwd_with_raised_max(oracle, torch_cuda, D, theta, causal, kv_chunk):
    import long_context_blockwise_attn_amd as bw

    torch = torch_cuda
    S = 1000
    q, k, v, pos = rising_case(S, D, seed=5)
    print("rising keys S%d D%d theta %g causal %d chunk %d" % (S, D, theta, causal, kv_chunk), flush=True)
    dpos = torch.from_numpy(pos).cuda()
    o, lse = bw.attn_fwd(q.cuda(), k.cuda(), v.cuda(), None, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), None, pos, theta=theta, causal=causal)
    assert_parity(to64(o), ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")


@pytest.mark.gpu
@pytest.mark.parametrize("theta", [0.0, 1e6])
def test_decode_with_raised_max(oracle, torch_cuda, theta):
    import long_context_blockwise_attn_amd as bw

    torch = torch_cuda
    S, nq = 4096, 4
    q, k, v, pos = rising_case(S, 128, seed=7)
    print("decode rising keys S%d n_q %d theta %g" % (S, nq, theta), flush=True)
    dpos = torch.from_numpy(pos).cuda()
    kc, vc = k.cuda(), v.cuda()
    kcache = bw.rope_apply(kc, dpos, theta=theta) if theta > 0 else kc
    o, lse = bw.attn_decode(q[:, :, S - nq:].contiguous().cuda(), kcache, vc, None, theta=theta)
    torch.cuda.synchronize()
    rows = np.arange(S - nq, S, dtype=np.int64)
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), None, pos, theta=theta, causal=True, rows=rows)
    assert_parity(to64(o), ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")
