"""attn_decode_noalloc (the decode entry point that allocates nothing: its
workspace is the library's static device array) against attn_decode (the
same kernels with a caller-provided workspace): two calls in a row, the
second smaller than the first, so the second runs on what the first left
in the shared array.  Results must be the same bits."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


CASES = [  # B, H, S, D, n_q, theta, causal: the second smaller than the first
    (1, 8, 100000, 128, 8, 5e7, True),
    (1, 2, 3000, 64, 3, 0.0, False),
]


def test_decode_noalloc_matches_decode_on_consecutive_calls(torch_cuda):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import randn_bf16

    torch = torch_cuda
    dev = torch.device("cuda")
    for i, (B, H, S, D, nq, theta, causal) in enumerate(CASES):
        print("no-alloc decode call %d: B%d H%d S%d D%d n_q %d theta %g causal %d" % (
            i, B, H, S, D, nq, theta, causal), flush=True)
        p = bw.make_params(B, H, S, D, theta=theta, causal=causal)
        assert bw.decode_workspace_bytes(p, nq) <= bw.load().attn_decode_noalloc_max_bytes()
        q = randn_bf16((B, H, nq, D), 100 + i, dev)
        k = randn_bf16((B, H, S, D), 200 + i, dev)
        v = randn_bf16((B, H, S, D), 300 + i, dev)
        kc = bw.rope_apply(k, None, theta=theta) if theta > 0 else k
        o_ref, lse_ref = bw.attn_decode(q, kc, v, None, theta=theta, causal=causal)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, nq), float("nan"), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        bw.attn_decode_noalloc(q, kc, v, None, theta=theta, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(o, o_ref), "o"
        assert torch.equal(lse, lse_ref), "lse"
