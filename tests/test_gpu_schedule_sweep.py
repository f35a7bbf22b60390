"""The order in which the kernels visit key/value (and query) tiles changes
the result only by rounding: the blockwise method is exact in any visiting
order (elamur.ai summary page, Summary; the ring order is the order in
which a ring of devices hands the blocks over: zhao9797 page "LWM (Large
World Model)", 模型架构 and Infra).  The kernels have one tile shape each, so
the sweep runs over the ring chunk instead: one case with chunks from one
64-row tile up to longer than the sequence, each against the oracle, and
the LSE against the natural order's within the rounding of the order-
dependent bf16 P."""
import numpy as np
import pytest

from helpers import assert_parity, to64

pytestmark = pytest.mark.gpu

CHUNKS = [64, 128, 192, 320, 512, 1024, 4096]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("n_docs", [0, 4])
def test_ring_chunk_sweep(oracle, torch_cuda, n_docs):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    torch = torch_cuda
    B, H, S, D, theta = 1, 2, 1600, 128, 1e6
    (q, k, v, do), seg, pos = random_case(B, H, S, D, seed=300 + n_docs, n_docs=n_docs)
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=theta)
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=theta)
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    _, lse0 = bw.attn_fwd(qc, kc, vc, dseg, dpos, theta=theta)
    torch.cuda.synchronize()
    lse0 = lse0.cpu().numpy()
    for chunk in CHUNKS:
        print("ring chunk %d, %d documents" % (chunk, n_docs), flush=True)
        o, lse = bw.attn_fwd(qc, kc, vc, dseg, dpos, theta=theta, kv_chunk=chunk)
        dq, dk, dv = bw.attn_bwd(qc, kc, vc, o, lse, doc, dseg, dpos, theta=theta, kv_chunk=chunk)
        torch.cuda.synchronize()
        assert_parity(o, ro, "O chunk %d" % chunk)
        assert_parity(lse.cpu().numpy(), rlse, "LSE chunk %d" % chunk)
        assert_parity(dq, rdq, "dq chunk %d" % chunk)
        assert_parity(dk, rdk, "dk chunk %d" % chunk)
        assert_parity(dv, rdv, "dv chunk %d" % chunk)
        # the same sums in another order.  The row sum adds the bf16-rounded
        # p = 2^(s - m) that the PV product uses, and m, the running max when
        # a tile is visited, depends on the order: each order's sum is within
        # 2^-9 (relative) of the exact one, so the two LSEs differ by at most
        # 2^-8 (plus fp32 rounding)
        assert np.abs(lse.cpu().numpy() - lse0).max() < 2.0 ** -8 + 1e-5
