"""Forward and backward (bf16, and the fp32 entry points) on seeded random
shapes against the oracle: batch, heads, length, head size, packing, causal
or not, RoPE base and ring chunk drawn together, so that combinations the
hand-picked cases do not name (a packed batch of two with a ring chunk that
is not a whole number of tiles, a length just past a tile edge with D = 64,
...) meet the same bars."""
import numpy as np
import pytest

from helpers import assert_parity, to64

pytestmark = pytest.mark.gpu


def draw_cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        # lengths around tile edges (64, 128, 256) and in between
        S = int(rng.choice([int(rng.integers(1, 1400)), 64 * int(rng.integers(1, 20)) + int(rng.integers(-2, 3))]))
        S = max(S, 1)
        n_docs = int(rng.choice([0, 0, int(rng.integers(2, 8))]))
        n_docs = min(n_docs, S) if n_docs else 0
        causal = bool(rng.random() < 0.75)
        theta = float(rng.choice([0.0, 1e4, 1e6, 5e7]))
        kv_chunk = int(rng.choice([0, 0, 64, 128, 192, 320]))
        cases.append((i, B, H, S, D, n_docs, causal, theta, kv_chunk))
    return cases


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("i,B,H,S,D,n_docs,causal,theta,kv_chunk", draw_cases(16))
def test_random_shape_fwd_bwd(oracle, torch_cuda, i, B, H, S, D, n_docs, causal, theta, kv_chunk):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case
    torch = torch_cuda
    (q, k, v, do), seg, pos = random_case(B, H, S, D, seed=1000 + i, n_docs=n_docs)
    print("case %d: B%d H%d S%d D%d docs %d causal %d theta %g chunk %d" % (i, B, H, S, D, n_docs, causal, theta,
                                                                            kv_chunk), flush=True)
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bw.attn_fwd(qc, kc, vc, dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    dq, dk, dv = bw.attn_bwd(qc, kc, vc, o, lse, doc, dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    ro, rlse = oracle.attn_fwd(q64, k64, v64, seg, pos, theta=theta, causal=causal)
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")
    rdq, rdk, rdv = oracle.attn_bwd(q64, k64, v64, to64(do), seg, pos, theta=theta, causal=causal)
    assert_parity(dq, rdq, "dq")
    assert_parity(dk, rdk, "dk")
    assert_parity(dv, rdv, "dv")


# fp32 entry points: the same draws (another seed) at the fp32 path's bar
# (max-abs 2e-4, mean-abs 2e-5; its derivation is in test_gpu_f32.py)
F32_MAX_ABS = 2e-4
F32_MEAN_ABS = 2e-5


@pytest.mark.parametrize("i,B,H,S,D,n_docs,causal,theta,kv_chunk", draw_cases(8, seed=20261204))
def test_random_shape_fwd_bwd_f32(oracle, torch_cuda, i, B, H, S, D, n_docs, causal, theta, kv_chunk):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case
    torch = torch_cuda
    (q, k, v, do), seg, pos = random_case(B, H, S, D, seed=2000 + i, n_docs=n_docs, dtype="fp32")
    print("f32 case %d: B%d H%d S%d D%d docs %d causal %d theta %g chunk %d" % (i, B, H, S, D, n_docs, causal,
                                                                                theta, kv_chunk), flush=True)
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bw.attn_fwd_f32(qc, kc, vc, dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    dq, dk, dv = bw.attn_bwd_f32(qc, kc, vc, o, lse, doc, dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    ro, rlse = oracle.attn_fwd(q64, k64, v64, seg, pos, theta=theta, causal=causal)
    rdq, rdk, rdv = oracle.attn_bwd(q64, k64, v64, to64(do), seg, pos, theta=theta, causal=causal)
    for got, ref, name in [(o, ro, "O"), (lse.cpu().numpy(), rlse, "LSE"), (dq, rdq, "dq"), (dk, rdk, "dk"),
                           (dv, rdv, "dv")]:
        assert_parity(got, ref, name, max_abs=F32_MAX_ABS, mean_abs=F32_MEAN_ABS)
