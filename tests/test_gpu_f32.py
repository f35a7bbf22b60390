"""The fp32 entry points (attn_fwd_f32, attn_bwd_f32, rope_apply_f32) on the
GPU against the fp64 oracle, element by element.

The paper trains and runs its models in full precision (arXiv 2402.08268,
training and inference setup); these cases take float32 N(0,1) inputs as they
are, so the oracle sees exactly the values the GPU sees.

Tolerance (fp32 arithmetic, fp64 oracle): the inputs are exact, and every
step rounds to fp32 (unit roundoff u = 2^-24) or uses the hardware's fp32
exp2, sine and cosine (relative errors of a few u).  A score is a 128-term
fp32 dot product of O(1) values scaled to O(1), an output is a sum of at most
S ~ 1e3 products with weights summing to 1, and a gradient is a sum of S such
products of O(1) factors; the rounding bound n u sum|terms| is 1e3 * 6e-8 ~
6e-5 for sums of O(1) magnitude.  The bar is max-abs 2e-4 and mean-abs 2e-5
on O, LSE, dq, dk and dv (100x tighter than the bf16 path's).
"""
import numpy as np
import pytest

from helpers import assert_parity, to64

pytestmark = pytest.mark.gpu

F32_MAX_ABS = 2e-4
F32_MEAN_ABS = 2e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def check(got, ref, name):
    err = assert_parity(got, ref, name, max_abs=F32_MAX_ABS, mean_abs=F32_MEAN_ABS)
    print("  %s (max, mean) abs error %.2e %.2e" % (name, err[0], err[1]), flush=True)


@pytest.mark.parametrize("theta", [1e4, 1e6, 5e7])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_f32_matches_oracle(oracle, torch_cuda, theta, D):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    rng = np.random.default_rng(int(theta) % 1000 + D + 7)
    B, H, S = 2, 3, 300
    x = torch.from_numpy(rng.standard_normal((B, H, S, D), dtype=np.float32))
    pos = rng.integers(0, 1 << 20, size=(B, S)).astype(np.int32)
    pos[0, :5] = [0, 1, (1 << 20) - 1, 12345, 999999]
    print("rope_f32 D%d theta %g" % (D, theta), flush=True)
    y = bw.rope_apply_f32(x.cuda(), torch.from_numpy(pos).cuda(), theta=theta)
    torch.cuda.synchronize()
    ref = oracle.rope(to64(x), pos, theta)
    err = np.abs(to64(y) - ref)
    print("  max abs error %.2e" % float(err.max()), flush=True)
    # fp32 rotation with an fp64-reduced angle: a few ulp of the pair's norm
    norm = np.sqrt(to64(x).reshape(B, H, S, D // 2, 2).__pow__(2).sum(-1)).repeat(2, axis=-1)
    assert np.all(err <= 4e-6 * norm + 1e-7), "max excess %.3e" % float(np.max(err - 4e-6 * norm))
    back = bw.rope_apply_f32(y, torch.from_numpy(pos).cuda(), theta=theta, inverse=True)
    torch.cuda.synchronize()
    assert np.max(np.abs(to64(back) - to64(x))) <= 1e-5


F32_CASES = [
    (2, 3, 1000, 128, 0, True, 1e6, 0),      # several tiles and a ragged tail
    (1, 2, 777, 128, 5, True, 1e7, 0),       # packed documents
    (1, 2, 600, 64, 4, False, 1e4, 0),       # packing without the causal term
    (1, 1, 300, 128, 0, False, 5e7, 0),      # dense
    (1, 2, 1, 128, 0, True, 1e6, 0),         # a single token
    (1, 2, 65, 64, 0, True, 1e6, 0),
    (1, 2, 300, 128, 3, True, 1e6, 0),       # more query tiles than the dQ kernel's 128 rows
    (1, 2, 1024, 128, 0, True, 5e7, 256),    # ring order over 4 chunks
    (1, 2, 1024, 128, 6, False, 1e7, 128),   # ring order, non-causal, packed
    (2, 2, 513, 128, 0, True, 0.0, 0),       # no RoPE
]


def f32_case(torch, B, H, S, D, n_docs, seed):
    from long_context_blockwise_attn_amd.inputs import random_case

    (q, k, v, do), seg, pos = random_case(B, H, S, D, seed, n_docs=n_docs, dtype="fp32")
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    return (q, k, v, do), seg, pos, dseg, torch.from_numpy(pos).cuda()


@pytest.mark.parametrize("B,H,S,D,n_docs,causal,theta,kv_chunk", F32_CASES)
def test_fwd_f32_matches_oracle(oracle, torch_cuda, B, H, S, D, n_docs, causal, theta, kv_chunk):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    print("fwd_f32 B%d H%d S%d D%d docs %d causal %d theta %g chunk %d" % (B, H, S, D, n_docs, causal, theta,
                                                                        kv_chunk), flush=True)
    (q, k, v, _), seg, pos, dseg, dpos = f32_case(torch, B, H, S, D, n_docs, seed=S + D + n_docs + 11)
    o, lse = bw.attn_fwd_f32(q.cuda(), k.cuda(), v.cuda(), dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=theta, causal=causal)
    check(to64(o), ro, "O")
    check(lse.cpu().numpy(), rlse, "LSE")


@pytest.mark.parametrize("B,H,S,D,n_docs,causal,theta,kv_chunk", F32_CASES)
def test_bwd_f32_matches_oracle(oracle, torch_cuda, B, H, S, D, n_docs, causal, theta, kv_chunk):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    print("bwd_f32 B%d H%d S%d D%d docs %d causal %d theta %g chunk %d" % (B, H, S, D, n_docs, causal, theta,
                                                                        kv_chunk), flush=True)
    (q, k, v, do), seg, pos, dseg, dpos = f32_case(torch, B, H, S, D, n_docs, seed=S + 3 * D + n_docs + 13)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bw.attn_fwd_f32(qc, kc, vc, dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    dq, dk, dv = bw.attn_bwd_f32(qc, kc, vc, o, lse, doc, dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=theta, causal=causal)
    check(to64(dq), rdq, "dq")
    check(to64(dk), rdk, "dk")
    check(to64(dv), rdv, "dv")


@pytest.mark.parametrize("B,H,S,D,n_docs,causal,kv_chunk", [
    (1, 2, 1024, 128, 0, True, 0),
    (1, 2, 1024, 128, 6, False, 128),
    (2, 4, 2048, 128, 0, True, 0),
    (1, 1, 64, 128, 0, False, 0),
    (1, 2, 1024, 64, 6, False, 128),
])
def test_f32_bwd_bitwise_reproducible(torch_cuda, B, H, S, D, n_docs, causal, kv_chunk):
    """Repeated calls on the same inputs give the same bits (no atomics, and
    every kernel's result depends on its inputs alone)."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case
    torch = torch_cuda
    print("f32 repeat B%d H%d S%d D%d docs %d causal %d chunk %d" % (B, H, S, D, n_docs, causal, kv_chunk),
          flush=True)
    (q, k, v, do), seg, pos = random_case(B, H, S, D, S + 5, n_docs=n_docs, dtype="fp32")
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    kw = dict(theta=1e6, causal=causal, kv_chunk=kv_chunk)
    o, lse = bw.attn_fwd_f32(qc, kc, vc, dseg, dpos, **kw)
    runs = [bw.attn_bwd_f32(qc, kc, vc, o, lse, doc, dseg, dpos, **kw) for _ in range(4)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for x, y in zip(r, runs[0]):
            assert torch.equal(x, y)


def test_f32_deterministic_and_causal_exact(torch_cuda):
    """Two runs agree bitwise, and values after position t do not reach
    outputs or gradients of rows up to t."""
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    g = torch.Generator(device="cuda").manual_seed(21)
    B, H, S, D = 1, 2, 700, 128
    q, k, v, do = (torch.randn(B, H, S, D, generator=g, device="cuda") for _ in range(4))
    print("f32 determinism B%d H%d S%d D%d" % (B, H, S, D), flush=True)
    o, lse = bw.attn_fwd_f32(q, k, v, None, None, theta=1e6)
    o2, lse2 = bw.attn_fwd_f32(q, k, v, None, None, theta=1e6)
    a = bw.attn_bwd_f32(q, k, v, o, lse, do, None, None, theta=1e6)
    b = bw.attn_bwd_f32(q, k, v, o, lse, do, None, None, theta=1e6)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    t = 300
    k2, v2 = k.clone(), v.clone()
    k2[:, :, t + 1:] = 1e4
    v2[:, :, t + 1:] = -1e4
    o3, lse3 = bw.attn_fwd_f32(q, k2, v2, None, None, theta=1e6)
    c = bw.attn_bwd_f32(q, k2, v2, o3, lse3, do, None, None, theta=1e6)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, :t + 1], o3[:, :, :t + 1])
    assert torch.equal(c[0][:, :, :t + 1], a[0][:, :, :t + 1])


def test_f32_rejects_bf16_tensors(torch_cuda):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    x = torch.zeros(1, 1, 64, 128, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(bw.AttnError):
        bw.attn_fwd_f32(x, x, x)
