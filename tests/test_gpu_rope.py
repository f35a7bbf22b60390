"""rope_apply on the GPU against the oracle's RoPE ("standard RoPE" with a
context-scaled base theta: zhao9797 page, 模型架构 and the Stage I table of
训练方法)."""
import numpy as np
import pytest

from helpers import to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("theta", [1e4, 1e6, 1e7, 5e7])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_matches_oracle(oracle, torch_cuda, theta, D):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    rng = np.random.default_rng(int(theta) % 1000 + D)
    B, H, S = 2, 3, 300
    x = torch.from_numpy(rng.standard_normal((B, H, S, D), dtype=np.float32)).to(torch.bfloat16)
    pos = rng.integers(0, 1 << 20, size=(B, S)).astype(np.int32)
    pos[0, :5] = [0, 1, (1 << 20) - 1, 12345, 999999]
    y = bw.rope_apply(x.cuda(), torch.from_numpy(pos).cuda(), theta=theta)
    torch.cuda.synchronize()
    ref = oracle.rope(to64(x), pos, theta)
    err = np.abs(to64(y) - ref)
    # bf16 output: half an ulp (2^-9 relative) plus fp32 rotation error
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    assert np.all(err <= bound), "max excess %.3e" % float(np.max(err - bound))
    # inverse undoes the rotation up to two bf16 roundings
    back = bw.rope_apply(y, torch.from_numpy(pos).cuda(), theta=theta, inverse=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to64(back), to64(x), atol=2e-2, rtol=2e-2)


def test_rope_position_zero_is_bitwise_identity(torch_cuda):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    x = torch.randn(1, 4, 64, 128, device="cuda").to(torch.bfloat16)
    pos = torch.zeros(1, 64, dtype=torch.int32, device="cuda")
    for inv in (False, True):
        y = bw.rope_apply(x, pos, theta=5e7, inverse=inv)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), x.view(torch.int16))


def test_rope_default_positions_and_in_place(oracle, torch_cuda):
    import long_context_blockwise_attn_amd as bw
    torch = torch_cuda
    x = torch.randn(1, 2, 100, 64, device="cuda").to(torch.bfloat16)
    ref = oracle.rope(to64(x), None, 1e6)
    y = bw.rope_apply(x.clone(), None, theta=1e6)
    xi = x.clone()
    bw.rope_apply(xi, None, theta=1e6, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(y, xi)
    assert np.max(np.abs(to64(y) - ref) - (2.0 ** -8 * np.abs(ref) + 1e-5)) <= 0
