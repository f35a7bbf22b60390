"""A softmax scale other than 1/sqrt(D), which the entry points take as a
parameter: the bf16 kernels fold scale * log2(e) into the query rows and
store dK times scale / (scale * log2(e)), so the scale reaches every kernel.
Forward, backward, decode and the fp32 path against the oracle with the same
scale (exact attention: zhao9797 page "LWM (Large World Model)", 模型架构)."""
import numpy as np
import pytest

from helpers import assert_parity, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("path,D,scale,theta,causal", [
    ("bf16", 128, 0.05, 1e6, True),
    ("bf16", 128, 0.15, 0.0, True),
    ("bf16", 64, 0.2, 1e4, False),
    ("f32", 128, 0.15, 1e6, True),
])
def test_fwd_bwd_with_scale(oracle, torch_cuda, path, D, scale, theta, causal):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    torch = torch_cuda
    B, H, S = 1, 2, 700
    f32 = path == "f32"
    (q, k, v, do), seg, pos = random_case(B, H, S, D, seed=int(1000 * scale) + D, n_docs=3,
                                           dtype="fp32" if f32 else "bf16")
    print("scale %g %s D%d theta %g causal %d" % (scale, path, D, theta, causal), flush=True)
    fwd, bwd = (bw.attn_fwd_f32, bw.attn_bwd_f32) if f32 else (bw.attn_fwd, bw.attn_bwd)
    dseg, dpos = torch.from_numpy(seg).cuda(), torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fwd(qc, kc, vc, dseg, dpos, theta=theta, causal=causal, scale=scale)
    dq, dk, dv = bwd(qc, kc, vc, o, lse, doc, dseg, dpos, theta=theta, causal=causal, scale=scale)
    torch.cuda.synchronize()
    bars = dict(max_abs=2e-4, mean_abs=2e-5) if f32 else {}
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=theta, scale=scale, causal=causal)
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=theta, scale=scale,
                                    causal=causal)
    assert_parity(o, ro, "O", **bars)
    assert_parity(lse.cpu().numpy(), rlse, "LSE", **bars)
    assert_parity(dq, rdq, "dq", **bars)
    assert_parity(dk, rdk, "dk", **bars)
    assert_parity(dv, rdv, "dv", **bars)


def test_decode_with_scale(oracle, torch_cuda):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    torch = torch_cuda
    S, nq, scale, theta = 3000, 6, 0.15, 1e6
    (q, k, v, _), _, pos = random_case(1, 2, S, 128, seed=31)
    print("decode scale %g S%d n_q %d" % (scale, S, nq), flush=True)
    dpos = torch.from_numpy(pos).cuda()
    kcache = bw.rope_apply(k.cuda(), dpos, theta=theta)
    o, lse = bw.attn_decode(q[:, :, S - nq:].contiguous().cuda(), kcache, v.cuda(), None, theta=theta, scale=scale)
    torch.cuda.synchronize()
    rows = np.arange(S - nq, S, dtype=np.int64)
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), None, pos, theta=theta, scale=scale, causal=True, rows=rows)
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")
