"""attn_fwd on the GPU against the oracle, element by element, plus the
mask-exactness, determinism and packing invariants.

Exact attention computed blockwise (elamur.ai summary: no approximation;
zhao9797 page, 模型架构), causal, with the packing mask of 训练方法."""
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


def run_case(oracle, torch, B, H, S, D, seed, n_docs=0, causal=True, theta=1e6, kv_chunk=0, restart_pos=True,
             pos_offset=0):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    (q, k, v, _), seg, pos = random_case(B, H, S, D, seed, n_docs=n_docs)
    if not restart_pos:
        pos = np.tile(np.arange(S, dtype=np.int32), (B, 1))
    pos = pos + pos_offset
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    print("case B%d H%d S%d D%d seed %d docs %d causal %d theta %g chunk %d" % (B, H, S, D, seed, n_docs, causal,
                                                                               theta, kv_chunk), flush=True)
    o, lse = bw.attn_fwd(q.cuda(), k.cuda(), v.cuda(), dseg, dpos, theta=theta, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=theta, causal=causal)
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")
    return o, lse


@pytest.mark.parametrize("B,H,S,D,n_docs,causal,theta,kv_chunk", [
    (2, 3, 1000, 128, 0, True, 1e6, 0),      # several tiles and a ragged tail
    (1, 2, 777, 128, 5, True, 1e7, 0),       # packed documents
    (1, 2, 600, 64, 4, False, 1e4, 0),       # packing without the causal term
    (1, 1, 300, 128, 0, False, 5e7, 0),      # dense
    (1, 2, 1, 128, 0, True, 1e6, 0),         # a single token
    (1, 2, 63, 128, 0, True, 1e6, 0),
    (1, 2, 65, 64, 0, True, 1e6, 0),
    (1, 2, 150, 128, 0, True, 1e6, 0),       # three key tiles: an odd count through the two-step barrier
    (1, 2, 200, 64, 2, False, 1e6, 0),       # four key tiles, D = 64
    (1, 2, 257, 128, 3, True, 1e6, 0),
    (1, 2, 1024, 128, 0, True, 5e7, 256),    # ring order over 4 chunks
    (1, 2, 1024, 128, 6, False, 1e7, 128),   # ring order, non-causal, packed
    (2, 2, 513, 128, 0, True, 0.0, 0),       # no RoPE
])
def test_fwd_matches_oracle(oracle, torch_cuda, B, H, S, D, n_docs, causal, theta, kv_chunk):
    run_case(oracle, torch_cuda, B, H, S, D, seed=S + D + n_docs, n_docs=n_docs, causal=causal, theta=theta,
             kv_chunk=kv_chunk)


def test_fwd_tiny_workload(oracle, torch_cuda):
    """B1 H2 D64 S1024, fp32 N(0,1) draws rounded to bf16, theta 1e4, causal."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import WORKLOADS, make_qkv
    torch = torch_cuda
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w)
    o, lse = bw.attn_fwd(q.cuda(), k.cuda(), v.cuda(), None, None, theta=w.theta)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), None, None, theta=w.theta)
    assert_parity(o, ro, "O")
    assert_parity(lse.cpu().numpy(), rlse, "LSE")


def test_fwd_large_positions(oracle, torch_cuda):
    run_case(oracle, torch_cuda, 1, 2, 500, 128, seed=7, theta=5e7, restart_pos=False, pos_offset=(1 << 20) - 600)


def test_fwd_noncontiguous_segments(oracle, torch_cuda):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    rng = np.random.default_rng(5)
    B, H, S, D = 1, 2, 400, 128
    q, k, v = (torch.from_numpy(rng.standard_normal((B, H, S, D), dtype=np.float32)).to(torch.bfloat16)
               for _ in range(3))
    seg = rng.integers(0, 3, size=(B, S)).astype(np.int32)
    for causal in (True, False):
        o, lse = bw.attn_fwd(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(seg).cuda(), None, theta=1e6,
                             causal=causal)
        torch.cuda.synchronize()
        ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, None, theta=1e6, causal=causal)
        assert_parity(o, ro, "O")
        assert_parity(lse.cpu().numpy(), rlse, "LSE")


def test_fwd_masked_keys_are_exactly_excluded(torch_cuda):
    """Poisoning masked-out K/V with large finite values leaves every
    unaffected output bitwise unchanged (future keys; other documents)."""
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    g = torch.Generator(device="cuda").manual_seed(3)
    B, H, S, D = 1, 2, 1500, 128
    q, k, v = (torch.randn(B, H, S, D, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    o0, l0 = bw.attn_fwd(q, k, v, None, None, theta=1e6)
    t = 700
    k2, v2 = k.clone(), v.clone()
    k2[:, :, t + 1:] = 1e4
    v2[:, :, t + 1:] = -1e4
    o1, l1 = bw.attn_fwd(q, k2, v2, None, None, theta=1e6)
    torch.cuda.synchronize()
    assert torch.equal(o0[:, :, :t + 1], o1[:, :, :t + 1])
    assert torch.equal(l0[:, :, :t + 1], l1[:, :, :t + 1])
    # packing: change the other documents
    lengths = [300, 500, 700]
    seg = torch.from_numpy(np.repeat(np.arange(3, dtype=np.int32), lengths)[None]).cuda()
    o0, l0 = bw.attn_fwd(q, k, v, seg, None, theta=1e6)
    k3, v3 = k.clone(), v.clone()
    k3[:, :, :300] = -1e4
    k3[:, :, 800:] = 1e4
    v3[:, :, :300] = 1e4
    v3[:, :, 800:] = 1e4
    o1, l1 = bw.attn_fwd(q, k3, v3, seg, None, theta=1e6)
    torch.cuda.synchronize()
    assert torch.equal(o0[:, :, 300:800], o1[:, :, 300:800])
    assert torch.equal(l0[:, :, 300:800], l1[:, :, 300:800])


def test_fwd_deterministic(torch_cuda):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    g = torch.Generator(device="cuda").manual_seed(4)
    q, k, v = (torch.randn(1, 4, 2048, 128, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    a = bw.attn_fwd(q, k, v, None, None, theta=1e6)
    b = bw.attn_fwd(q, k, v, None, None, theta=1e6)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fwd_packed_equals_unpacked(torch_cuda):
    """Each document's rows of a packed sequence equal that document run alone
    (zhao9797 page, 训练方法, Masked Sequence Packing)."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import segments_from_lengths
    torch = torch_cuda
    lengths = [200, 37, 700, 1, 300]
    S = sum(lengths)
    seg, pos = segments_from_lengths(lengths)
    g = torch.Generator(device="cuda").manual_seed(6)
    q, k, v = (torch.randn(1, 2, S, 128, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    o, lse = bw.attn_fwd(q, k, v, torch.from_numpy(seg).cuda(), torch.from_numpy(pos).cuda(), theta=1e7)
    start = 0
    for L in lengths:
        sl = slice(start, start + L)
        od, ld = bw.attn_fwd(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), None,
                             None, theta=1e7)
        torch.cuda.synchronize()
        assert_parity(o[:, :, sl], to64(od), "O doc")
        assert_parity(lse[:, :, sl].cpu().numpy(), ld.cpu().numpy(), "LSE doc")
        start += L
