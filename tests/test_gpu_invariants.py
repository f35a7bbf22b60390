"""Properties of exact attention that hold at any size, on the GPU path:
  - RoPE makes scores depend only on relative positions (RoFormer's rotation,
    the "standard RoPE" of the zhao9797 page "LWM (Large World Model)",
    模型架构), so shifting every position by the same amount leaves the
    attention output and its gradients unchanged;
  - a document of one token attends only to itself (the packing mask,
    训练方法, Masked Sequence Packing): its output is its own value row,
    bitwise, and its dv is its own dO;
  - softmax rows sum to one, so v = 1 everywhere gives O = 1 and, dS being
    P (dP - Delta) = 0 for a constant v, dq = dk = 0 for any dO.
Each case is compared with the oracle (or with the closed form) under the
same bar as every parity test."""
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


@pytest.mark.parametrize("n_docs,causal,kv_chunk", [(0, True, 0), (3, True, 0), (0, False, 256)])
def test_position_shift_invariance(oracle, torch_cuda, n_docs, causal, kv_chunk):
    """Positions p and p + 12345 give the same attention, forward and
    backward: the GPU at shifted positions against the oracle at the
    original ones."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    torch = torch_cuda
    B, H, S, D = 1, 2, 900, 128
    (q, k, v, do), seg, pos = random_case(B, H, S, D, seed=77 + n_docs, n_docs=n_docs)
    shifted = (pos + 12345).astype(np.int32)
    print("position shift docs %d causal %d chunk %d" % (n_docs, causal, kv_chunk), flush=True)
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(shifted).cuda()
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bw.attn_fwd(qc, kc, vc, dseg, dpos, theta=1e6, causal=causal, kv_chunk=kv_chunk)
    dq, dk, dv = bw.attn_bwd(qc, kc, vc, o, lse, dc, dseg, dpos, theta=1e6, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=1e6, causal=causal)
    # the gradient of q and k is rotated back at their own positions, so only
    # dv and the attention itself are shift-invariant; dq and dk are checked
    # at the shifted positions
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, shifted, theta=1e6, causal=causal)
    assert_parity(o, ro, "O (shifted positions vs original)")
    assert_parity(lse.cpu().numpy(), rlse, "LSE (shifted positions vs original)")
    _, _, rdv0 = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=1e6, causal=causal)
    assert_parity(dv, rdv0, "dv (shifted positions vs original)")
    assert_parity(dq, rdq, "dq")
    assert_parity(dk, rdk, "dk")


@pytest.mark.parametrize("causal", [True, False])
def test_single_token_documents(oracle, torch_cuda, causal):
    """Every document one token long: O = v bitwise, LSE = the row's own
    score, dv = dO, dq = dk = 0 (within the bar: dS = P (dP - Delta) with
    P = 1 and Delta = dP up to the order of the kernel's sums)."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    torch = torch_cuda
    B, H, S, D = 1, 2, 777, 128
    (q, k, v, do), _, _ = random_case(B, H, S, D, seed=91)
    seg = np.arange(S, dtype=np.int32)[None]
    pos = np.zeros((1, S), dtype=np.int32)
    print("single-token documents causal %d" % causal, flush=True)
    dseg, dpos = torch.from_numpy(seg).cuda(), torch.from_numpy(pos).cuda()
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bw.attn_fwd(qc, kc, vc, dseg, dpos, theta=1e7, causal=causal)
    dq, dk, dv = bw.attn_bwd(qc, kc, vc, o, lse, dc, dseg, dpos, theta=1e7, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, vc), "O = v"
    _, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=1e7, causal=causal)
    # position 0: no rotation, so the own score is scale <q_i, k_i>
    own = (to64(q) * to64(k)).sum(-1) / np.sqrt(D)
    assert np.allclose(rlse, own, rtol=0, atol=1e-12)
    assert_parity(lse.cpu().numpy(), own, "LSE = own score")
    assert_parity(dv, to64(do), "dv = dO")
    zero = np.zeros((B, H, S, D))
    assert_parity(dq, zero, "dq = 0")
    assert_parity(dk, zero, "dk = 0")


@pytest.mark.parametrize("n_docs,kv_chunk", [(0, 0), (4, 0), (0, 128)])
def test_constant_values(oracle, torch_cuda, n_docs, kv_chunk):
    """v = 1: O = 1 (rows of P sum to one, up to the bf16 rounding of P,
    which the kernel's row sums share) and dq = dk = 0 for any dO; dv
    against the oracle."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    torch = torch_cuda
    B, H, S, D = 1, 2, 1100, 128
    (q, k, _, do), seg, pos = random_case(B, H, S, D, seed=55 + n_docs, n_docs=n_docs)
    v = torch.ones_like(q)
    print("constant values docs %d chunk %d" % (n_docs, kv_chunk), flush=True)
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bw.attn_fwd(qc, kc, vc, dseg, dpos, theta=1e6, kv_chunk=kv_chunk)
    dq, dk, dv = bw.attn_bwd(qc, kc, vc, o, lse, dc, dseg, dpos, theta=1e6, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    one = np.ones((B, H, S, D))
    assert_parity(o, one, "O = 1", max_abs=2e-3, mean_abs=2e-4)
    zero = np.zeros((B, H, S, D))
    assert_parity(dq, zero, "dq = 0")
    assert_parity(dk, zero, "dk = 0")
    _, _, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=1e6)
    assert_parity(dv, rdv, "dv")
