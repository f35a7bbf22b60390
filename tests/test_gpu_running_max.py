"""The lazy running max of the online softmax (zhao9797 page "LWM (Large
World Model)", 模型架构: blockwise attention merges each block's partial
result with a running max and sum, exactly).  The kernels raise a row's
running max m only when a tile's max exceeds it by more than 8 in log2
units; a raise rescales O and l and moves the start value of the later
score MFMAs.  Random inputs almost never need a raise after the first tile,
so in these cases every key before S/3 carries a bias of about -12 in log2
units (one dimension: q = C, k = -24): with the forward walking tiles in
increasing order (the decode each chunk so), every row that reaches the
unbiased keys raises its max once, mid-walk; in a second set the keys fall
in four equal runs biased by about -36, -24, -12 and 0, so a row raises its
max up to three times.  The bias is large but its
keys' probabilities are tiny, so the scores that matter stay of the usual
size.  Forward and decode (the kernels with a running max) against the
oracle, and the backward, which recomputes P from the forward's LSE.

The gradients of these inputs carry the rounding of the bf16 MFMA operands
magnified by the bias: dq_i = scale sum_j dS_ij k'_j takes each dS_ij
rounded to bf16 (relative error up to 2^-9) times a key element of -24, and
in the bias dimension the exact sum cancels (rows of dS sum to zero), so the
rounding alone can exceed the absolute bar.  dS_ij = P_ij (dP_ij - Delta_i)
also inherits the relative error of P_ij, which the bf16 rounding of the
rotated rows q'' = q' scale log2(e) and k' puts into the score: at most
e_ij = 2^-8 scale sum_d |q'_i[d]| |k'_j[d]| (natural-log units; each
operand rounded once).  Their bar is therefore the absolute one plus the
bound of these roundings, per element:
  dq_i[d]: scale sum_j |dS_ij| |k'_j[d]| (2^-8 + e_ij)  (dS, k' rounded once),
  dk_j[d]: scale sum_i |dS_ij| |q'_i[d]| (2^-8 + e_ij),
  dv_j[d]: sum_i P_ij |dO_i[d]| (2^-9 + e_ij)           (P rounded once),
with P, dS, q' and k' from the oracle (attn_probs).  The mean-abs bar stays
2e-3."""
import math

import numpy as np
import pytest

from helpers import MAX_ABS, assert_parity, to64

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


def rising_case(S, D, seed, with_grad_out=False, stairs=1):
    """stairs = 1: keys before S/3 biased by about -12 (log2 units), the rest
    not.  stairs = n > 1: n + 1 equal runs of keys biased by -12n, ..., -12,
    0, so that a row raises its max once on entering each later run."""
    from long_context_blockwise_attn_amd.inputs import random_case

    (q, k, v, do), _, pos = random_case(1, 2, S, D, seed)
    bd = D - 2
    q[..., bd] = bias_query_value(D)
    q[..., bd + 1] = 0.0
    k[..., bd + 1] = 0.0
    if stairs == 1:
        k[..., : S // 3, bd] = -24.0
        k[..., S // 3:, bd] = 0.0
    else:
        edges = [S * r // (stairs + 1) for r in range(stairs + 2)]
        for r in range(stairs + 1):
            k[..., edges[r]:edges[r + 1], bd] = -24.0 * (stairs - r)
    return (q, k, v, pos, do) if with_grad_out else (q, k, v, pos)


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
        q, k, _, _ = rising_case(2000, D, seed=6, stairs=3)
        r = raises_per_row(q, k, causal=True)
        # a row raises on entering each later run of keys: up to three times
        for n in range(4):
            lo = 500 * n
            assert (r[lo:lo + 500] <= n).all()
            assert (r[lo + 64:lo + 500] == n).mean() > 0.9


@pytest.mark.gpu
@pytest.mark.parametrize("D,theta,causal,kv_chunk", [
    (128, 0.0, True, 0), (128, 1e6, True, 0), (128, 0.0, False, 0), (128, 1e6, True, 256), (64, 1e6, True, 0)])
def test_fwd_with_raised_max(oracle, torch_cuda, D, theta, causal, kv_chunk):
    import long_context_blockwise_attn_amd as bw

    torch = torch_cuda
    S = 1000
    q, k, v, pos, do = rising_case(S, D, seed=5, with_grad_out=True)
    print("rising keys S%d D%d theta %g causal %d chunk %d" % (S, D, theta, causal, kv_chunk), flush=True)
    dpos = torch.from_numpy(pos).cuda()
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bw.attn_fwd(qc, kc, vc, None, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    dq, dk, dv = bw.attn_bwd(qc, kc, vc, o, lse, dc, None, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), None, pos, theta=theta, causal=causal)
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), None, pos, theta=theta, causal=causal)
    P, dS, qr, kr = oracle.attn_probs(to64(q), to64(k), to64(v), to64(do), None, pos, theta=theta, causal=causal)
    scale, u = 1.0 / math.sqrt(D), 2.0 ** -8
    e = u * scale * (np.abs(qr) @ np.swapaxes(np.abs(kr), -1, -2))  # score rounding bound per pair
    tr = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
    bar_dq = MAX_ABS + scale * ((np.abs(dS) * (u + e)) @ np.abs(kr))
    bar_dk = MAX_ABS + scale * (tr(np.abs(dS) * (u + e)) @ np.abs(qr))
    bar_dv = MAX_ABS + tr(P * (u / 2 + e)) @ np.abs(to64(do))
    print("  rounding bound on top of the bar: dq up to %.3g, dk up to %.3g, dv up to %.3g" % (
        bar_dq.max() - MAX_ABS, bar_dk.max() - MAX_ABS, bar_dv.max() - MAX_ABS), flush=True)
    assert_parity(dq, rdq, "dq", max_abs=bar_dq)
    assert_parity(dk, rdk, "dk", max_abs=bar_dk)
    assert_parity(dv, rdv, "dv", max_abs=bar_dv)


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
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")


@pytest.mark.gpu
@pytest.mark.parametrize("D,theta,kv_chunk", [(128, 0.0, 0), (128, 1e6, 0), (64, 1e6, 0), (128, 1e6, 512)])
def test_fwd_with_several_raises(oracle, torch_cuda, D, theta, kv_chunk):
    """Rows that raise their running max up to three times in one walk (the
    forward is the kernel with a running max; the backward recomputes P from
    the LSE and has none)."""
    import long_context_blockwise_attn_amd as bw

    torch = torch_cuda
    S = 2000
    q, k, v, pos = rising_case(S, D, seed=6, stairs=3)
    print("stair keys S%d D%d theta %g chunk %d" % (S, D, theta, kv_chunk), flush=True)
    dpos = torch.from_numpy(pos).cuda()
    o, lse = bw.attn_fwd(q.cuda(), k.cuda(), v.cuda(), None, dpos, theta=theta, causal=True, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), None, pos, theta=theta, causal=True)
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")


@pytest.mark.gpu
def test_decode_with_several_raises(oracle, torch_cuda):
    import long_context_blockwise_attn_amd as bw

    torch = torch_cuda
    S, nq, theta = 8192, 4, 1e6
    q, k, v, pos = rising_case(S, 128, seed=8, stairs=3)
    print("decode stair keys S%d n_q %d theta %g" % (S, nq, theta), flush=True)
    dpos = torch.from_numpy(pos).cuda()
    kcache = bw.rope_apply(k.cuda(), dpos, theta=theta)
    o, lse = bw.attn_decode(q[:, :, S - nq:].contiguous().cuda(), kcache, v.cuda(), None, theta=theta)
    torch.cuda.synchronize()
    rows = np.arange(S - nq, S, dtype=np.int64)
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), None, pos, theta=theta, causal=True, rows=rows)
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")
