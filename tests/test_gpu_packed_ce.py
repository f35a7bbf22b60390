"""packed_ce_loss on the GPU against the oracle (oracle.packed_ce): the
re-weighted cross-entropy of packed rows, its per-row values and its
gradient (loss side of masked sequence packing: zhao9797 page "LWM (Large
World Model)", 数据 and 训练方法).

Tolerances: logits are bf16 and reach the oracle exactly.  The GPU forms each
row's logsumexp in fp32 (exp2 and log of the hardware, sums over <= 65536
terms), so ce_t carries an absolute error of a few 1e-6 on values ~10: bar
5e-5 per row, and the loss (a weighted mean of ce_t, summed in fp64) the
same.  Gradients are written as bf16 (round to nearest even, relative error
<= 2^-9) from fp32 values with relative error ~1e-6: bar 2^-8 |ref|
elementwise."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CE_ABS = 5e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def run_gpu(torch, x, tg, seg, num_segments, grad_scale=1.0, with_grad=True, use_seg=True):
    import long_context_blockwise_attn_amd as bw

    logits = torch.from_numpy(x).to(torch.bfloat16).cuda()
    targets = torch.from_numpy(np.ascontiguousarray(tg, dtype=np.int32)).cuda()
    dseg = torch.from_numpy(np.ascontiguousarray(seg, dtype=np.int32)).cuda() if use_seg else None
    loss, dl, tce = bw.packed_ce_loss(logits, targets, dseg, num_segments, grad_scale, with_grad=with_grad,
                                      with_token_ce=True)
    torch.cuda.synchronize()
    xb = logits.float().cpu().numpy()  # the exact bf16 values the GPU read
    return float(loss.item()), (dl.float().cpu().numpy() if dl is not None else None), tce.cpu().numpy(), xb


def check_against_oracle(oracle, got, x, tg, seg, num_segments, grad_scale=1.0):
    loss, dl, tce, xb = got
    B, S, V = xb.shape
    rl, rce, rdl = oracle.packed_ce(xb.reshape(B * S, V), tg.reshape(-1), seg, num_segments, grad_scale)
    assert abs(loss - rl) <= CE_ABS, (loss, rl)
    err_ce = np.abs(tce.reshape(-1) - rce).max()
    assert err_ce <= CE_ABS, err_ce
    if dl is not None:
        d = dl.reshape(B * S, V)
        excess = np.abs(d - rdl) - 2.0 ** -8 * np.abs(rdl)
        assert np.all(np.isfinite(d)) and excess.max() <= 1e-30, float(excess.max())
    print("  loss %.6f (oracle %.6f), max ce error %.2e" % (loss, rl, err_ce), flush=True)


@pytest.mark.parametrize("B,S,V,n_docs", [
    (1, 700, 40192, 5),     # the workload's vocabulary, ragged examples
    (2, 300, 32000, 3),     # two batch rows: examples keyed by (row, id)
    (1, 257, 8, 4),         # smallest vocabulary
    (3, 100, 1000, 2),      # vocabulary not a multiple of the threads' span
    (1, 64, 65536, 2),      # largest vocabulary
    (1, 33, 4104, 33),      # one-token examples
])
def test_packed_ce_matches_oracle(oracle, torch_cuda, B, S, V, n_docs):
    from long_context_blockwise_attn_amd.inputs import random_ce_case

    print("packed_ce B%d S%d V%d docs %d" % (B, S, V, n_docs), flush=True)
    x, tg, seg = random_ce_case(B, S, V, seed=B * 1000 + S + V + n_docs, n_docs=n_docs)
    got = run_gpu(torch_cuda, x, tg, seg, n_docs, grad_scale=1.0)
    check_against_oracle(oracle, got, x, tg, seg, n_docs)


def test_packed_ce_without_segments_is_one_example_per_row(oracle, torch_cuda):
    from long_context_blockwise_attn_amd.inputs import random_ce_case

    x, tg, seg = random_ce_case(2, 200, 512, seed=3, n_docs=4)
    got = run_gpu(torch_cuda, x, tg, seg, 1, use_seg=False)
    check_against_oracle(oracle, got, x, tg, np.zeros_like(seg), 1)


@pytest.mark.parametrize("grad_scale", [-2.5, 0.0, 1e-3])
def test_packed_ce_grad_scale(oracle, torch_cuda, grad_scale):
    from long_context_blockwise_attn_amd.inputs import random_ce_case

    x, tg, seg = random_ce_case(1, 300, 2048, seed=17, n_docs=3)
    got = run_gpu(torch_cuda, x, tg, seg, 3, grad_scale=grad_scale)
    check_against_oracle(oracle, got, x, tg, seg, 3, grad_scale=grad_scale)
    if grad_scale == 0.0:
        assert not got[1].any()


def test_packed_ce_rows_without_loss(oracle, torch_cuda):
    """Targets outside [0, V) and ids outside [0, num_segments) carry no loss
    and get zero gradient rows; with no loss row at all the loss is 0."""
    from long_context_blockwise_attn_amd.inputs import random_ce_case

    V = 1024
    x, tg, seg = random_ce_case(1, 200, V, seed=23, n_docs=4, ignore_frac=0.0)
    tg[0, 5] = V
    tg[0, 6] = -7
    seg = seg.copy()
    seg[0, 7] = -1
    seg[0, 8] = 4  # == num_segments
    got = run_gpu(torch_cuda, x, tg, seg, 4)
    check_against_oracle(oracle, got, x, tg, seg, 4)
    for t in (5, 6, 7, 8):
        assert got[2][0, t] == 0.0 and not got[1][0, t].any()
    none = run_gpu(torch_cuda, x, np.full_like(tg, -1), seg, 4)
    assert none[0] == 0.0 and not none[1].any() and not none[2].any()


def test_packed_ce_loss_only_and_reproducible(torch_cuda):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_ce_case

    torch = torch_cuda
    x, tg, seg = random_ce_case(2, 500, 40192, seed=29, n_docs=6)
    logits = torch.from_numpy(x).to(torch.bfloat16).cuda()
    targets, dseg = torch.from_numpy(tg).cuda(), torch.from_numpy(seg).cuda()
    runs = [bw.packed_ce_loss(logits, targets, dseg, 6) for _ in range(3)]
    only = bw.packed_ce_loss(logits, targets, dseg, 6, with_grad=False)
    torch.cuda.synchronize()
    assert only[1] is None and torch.equal(only[0], runs[0][0])
    for r in runs[1:]:
        assert torch.equal(r[0], runs[0][0]) and torch.equal(r[1], runs[0][1])


def test_packed_ce_full_workload(oracle, torch_cuda):
    """The packed_ce_32k workload whole (32768 rows x 40192 logits): the loss
    and every row's cross-entropy against the oracle, the gradient on
    sampled rows (loss and no-loss rows, the first and last rows)."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import WORKLOADS, packed_ce_case

    torch = torch_cuda
    w = WORKLOADS["packed_ce_32k"]
    logits, targets, seg, ne = packed_ce_case(w, device="cuda")
    print("packed_ce_32k: S%d V%d examples %d" % (w.seqlen, w.extra["vocab"], ne), flush=True)
    loss, dl, tce = bw.packed_ce_loss(logits, targets, seg, ne, with_token_ce=True)
    torch.cuda.synchronize()
    B, S, V = logits.shape
    tg = targets.cpu().numpy().reshape(-1)
    rng = np.random.default_rng(1)
    loss_rows = np.nonzero(tg >= 0)[0]
    rows = np.unique(np.concatenate([[0, S - 1], rng.choice(loss_rows, 12, replace=False),
                                     rng.choice(np.nonzero(tg < 0)[0], 4, replace=False)]))
    xf = logits.float().cpu().numpy().reshape(B * S, V)  # exact bf16 values as float32
    del logits
    rl, rce, rdl = oracle.packed_ce(xf, tg, seg.cpu().numpy(), ne, grad_rows=rows)
    assert abs(float(loss.item()) - rl) <= CE_ABS, (float(loss.item()), rl)
    err_ce = np.abs(tce.cpu().numpy().reshape(-1) - rce).max()
    assert err_ce <= CE_ABS, err_ce
    d = dl.reshape(B * S, V)[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    excess = np.abs(d - rdl) - 2.0 ** -8 * np.abs(rdl)
    assert excess.max() <= 1e-30, float(excess.max())
    print("  loss %.6f (oracle %.6f), max ce error %.2e over %d rows" % (float(loss.item()), rl, err_ce, S),
          flush=True)


def test_packed_ce_rows_packed_differently(oracle, torch_cuda):
    """Two batch rows with different example boundaries: an example is
    (batch row, segment id), so the counts and weights are per row."""
    from long_context_blockwise_attn_amd.inputs import ce_targets

    rows = [[100, 150, 50], [20, 200, 80]]
    V = 4096
    parts = [ce_targets(r, V, seed=53 + i) for i, r in enumerate(rows)]
    tg = np.concatenate([p[0] for p in parts])
    seg = np.concatenate([p[1] for p in parts])
    x = np.random.default_rng(59).standard_normal((len(rows), seg.shape[1], V), dtype=np.float32) * 3
    got = run_gpu(torch_cuda, x, tg, seg, 3)
    check_against_oracle(oracle, got, x, tg, seg, 3)
