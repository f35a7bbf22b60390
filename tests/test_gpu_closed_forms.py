"""Closed forms at full length: the 1M-token workload on every row.

With q = 0 every visible score is 0, so each query row attends uniformly to
the keys it sees, whatever the keys are.  For the causal single document of
the 1M stage (zhao9797 page "LWM (Large World Model)", 训练方法, Stage I
table: 2^20 tokens, theta 5e7), with c_i = i + 1 visible keys:
  - O_i = (1/c_i) sum_{j<=i} v_j (prefix means) and LSE_i = ln c_i;
  - dk = 0 exactly (every dS_ij multiplies a zero query row);
  - dv_j = sum_{i>=j} dO_i / c_i (suffix sums);
  - dq_i = R(-a_i) (scale / c_i) [dO_i^T sum_{j<=i} v_j k'_j^T - Delta_i
    sum_{j<=i} k'_j], Delta_i = <dO_i, O_i>, k'_j the rotated keys (prefix
    sums of the outer products v_j k'_j^T, formed chunk by chunk).
Attention is exact (elamur.ai summary page, Summary: no approximation), so
the blockwise ring-order walk must reproduce these on all 2^20 rows (the
closed forms: tests/closed_forms.py, pinned against the oracle on the CPU).  The GPU
runs 2 of the 32 heads (heads are independent and take the same kernel path)
with the workload's sequence length, theta, chunking and ring order; every
row of both heads is checked in float64 against the closed forms."""
import numpy as np
import pytest

from closed_forms import zero_query_closed_forms
from helpers import assert_parity

pytestmark = pytest.mark.gpu

HEADS = 2
CHUNK_ROWS = 1 << 16  # host-side comparison in row chunks


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_1m_ring_order_zero_queries_closed_forms(oracle, torch_cuda):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import WORKLOADS, randn_bf16

    torch = torch_cuda
    w = WORKLOADS["full_1m"]
    B, H, S, D = 1, HEADS, w.seqlen, w.head_dim
    print("1M closed forms: B%d H%d S%d D%d theta %g chunk %d, q = 0" % (B, H, S, D, w.theta, w.kv_chunk), flush=True)
    dev = torch.device("cuda")
    q = torch.zeros((B, H, S, D), dtype=torch.bfloat16, device=dev)
    k = randn_bf16((B, H, S, D), w.seed * 16 + 1, dev)
    v = randn_bf16((B, H, S, D), w.seed * 16 + 2, dev)
    do = randn_bf16((B, H, S, D), w.seed * 16 + 3, dev)
    o, lse = bw.attn_fwd(q, k, v, None, None, theta=w.theta, causal=True, kv_chunk=w.kv_chunk)
    dq, dk, dv = bw.attn_bwd(q, k, v, o, lse, do, None, None, theta=w.theta, causal=True, kv_chunk=w.kv_chunk)
    torch.cuda.synchronize()
    print("  GPU done", flush=True)
    assert bool((dk == 0).all()), "dk must be exactly zero"

    scale = 1.0 / np.sqrt(D)
    cnt = np.arange(1, S + 1, dtype=np.float64)
    assert_parity(lse.cpu().numpy(), np.log(cnt)[None, None].repeat(H, 1), "LSE = ln(i + 1)")
    for h in range(H):
        vh = v[0, h].double().cpu().numpy()
        doh = do[0, h].double().cpu().numpy()
        kh = k[0, h].double().cpu().numpy()
        for sl, o_ref, dv_ref, dq_ref in zero_query_closed_forms(oracle, kh, vh, doh, w.theta, scale, CHUNK_ROWS):
            rr = "rows [%d, %d)" % (sl.start, sl.stop)
            assert_parity(o[0, h, sl], o_ref, "h%d O %s" % (h, rr))
            assert_parity(dv[0, h, sl], dv_ref, "h%d dv %s" % (h, rr))
            assert_parity(dq[0, h, sl], dq_ref, "h%d dq %s" % (h, rr))
        print("  head %d: O, dv, dq on all %d rows match the closed forms" % (h, S), flush=True)
