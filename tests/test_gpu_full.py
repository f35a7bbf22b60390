"""Parity at the full workload sizes.

The GPU path runs each workload whole, with the parameters the benchmark
uses: 32K single document; 128K of log-uniform packed documents; 256K of
video-text records (forward only); 1M in ring order over 64 chunks of 16384.
The oracle cannot produce every output at these sizes, so it is evaluated on
samples it computes one by one:
  - O, LSE and dq on sampled query rows (tile edges, document edges, the last
    rows, random rows);
  - dk and dv on windows of key columns together with every query row that
    sees them (the last 32 keys of a document, and one whole short document
    of a packed row), so those columns are complete sums, not partial ones.
For the 1M workload the GPU runs 8 of the 32 heads: heads are independent and
each takes the same kernel path, while the sequence length, the chunking and
the ring order are the workload's.  The fp32 path (attn_fwd_f32 /
attn_bwd_f32 on fp32 draws of the same workloads) runs the 32K and the 128K
packed workloads whole, held to the fp32 bars.
"""
import numpy as np
import pytest

from helpers import assert_parity

pytestmark = pytest.mark.gpu

# workload, heads run on the GPU (None: all of the workload's), heads checked,
# path (bf16, or fp32 tensors through attn_fwd_f32 / attn_bwd_f32 with the
# fp32 bars of test_gpu_f32.py)
FULL = [
    ("llama7b_32k", None, (0, 31), "bf16"),
    ("packing_128k", None, (7,), "bf16"),
    ("video_text_256k", None, (12,), "bf16"),
    ("full_1m", 8, (3,), "bf16"),
    ("llama7b_32k", None, (5,), "f32"),
    ("packing_128k", None, (20,), "f32"),
]
F32_BARS = dict(max_abs=2e-4, mean_abs=2e-5)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def doc_bounds(lengths):
    ends = np.cumsum(lengths)
    return np.concatenate([[0], ends[:-1]]).astype(np.int64), ends.astype(np.int64)


def sample_rows(S, lengths, rng, n_random=24, n_docs=6):
    """Tile edges, the last rows, the first and last rows of a few documents
    and random rows."""
    rows = {0, 1, 31, 32, 63, 64, 255, 256, 257, S - 33, S - 2, S - 1}
    starts, ends = doc_bounds(lengths)
    pick = rng.choice(len(lengths), size=min(n_docs, len(lengths)), replace=False)
    for d in pick:
        rows.update({int(starts[d]), int(starts[d]) + 1, int(ends[d]) - 1})
    rows.update(int(x) for x in rng.integers(0, S, size=n_random))
    return np.array(sorted(r for r in rows if 0 <= r < S), dtype=np.int64)


def key_windows(S, lengths, rng):
    """Key-column windows [c0, c1) whose every viewing query row lies in
    [c0, c_last_row]: the last 32 keys of a document (rows that see key j
    are j .. end of its document) and, for packed rows, one whole document
    of at most 1024 tokens."""
    starts, ends = doc_bounds(lengths)
    wins = []
    d = int(rng.integers(0, len(lengths))) if len(lengths) > 1 else 0
    e = int(ends[d])
    wins.append((max(int(starts[d]), e - 32), e))
    if len(lengths) > 1:
        short = [i for i in range(len(lengths)) if lengths[i] <= 1024 and i != d]
        if short:
            i = short[len(short) // 2]
            wins.append((int(starts[i]), int(ends[i])))
    if e != S:
        wins.append((S - 32, S))
    return wins


def head64(t, h):
    return t[:, h:h + 1].float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name,gpu_heads,check_heads,path", FULL)
def test_full_size_sampled_parity(oracle, torch_cuda, name, gpu_heads, check_heads, path):
    import functools

    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import WORKLOADS, make_qkv, packing

    torch = torch_cuda
    w = WORKLOADS[name]
    H = w.heads if gpu_heads is None else gpu_heads
    S = w.seqlen
    f32 = path == "f32"
    bars = F32_BARS if f32 else {}
    assert_parity_ = functools.partial(assert_parity, **bars)
    fwd, bwd = (bw.attn_fwd_f32, bw.attn_bwd_f32) if f32 else (bw.attn_fwd, bw.attn_bwd)
    seg, pos, lengths = packing(w)
    q, k, v, do = make_qkv(w, device="cuda", with_grad_out=True, heads=gpu_heads, dtype="fp32" if f32 else "bf16")
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    print("workload %s (%s): B%d H%d S%d D%d theta %g chunk %d docs %d backward %d" % (
        name, path, w.batch, H, S, w.head_dim, w.theta, w.kv_chunk, len(lengths), w.backward), flush=True)
    o, lse = fwd(q, k, v, dseg, dpos, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk)
    grads = None
    if w.backward:
        grads = bwd(q, k, v, o, lse, do, dseg, dpos, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk)
    torch.cuda.synchronize()
    print("  GPU done", flush=True)

    rng = np.random.Generator(np.random.PCG64(S + len(lengths)))
    rows = sample_rows(S, lengths, rng)
    wins = key_windows(S, lengths, rng) if w.backward else []
    for h in check_heads:
        qh, kh, vh = head64(q, h), head64(k, h), head64(v, h)
        ro, rlse = oracle.attn_fwd(qh, kh, vh, seg, pos, theta=w.theta, causal=w.causal, rows=rows)
        eo = assert_parity_(o[:, h:h + 1, rows], ro, "%s h%d O" % (name, h))
        el = assert_parity_(lse[:, h:h + 1, rows].cpu().numpy(), rlse, "%s h%d LSE" % (name, h))
        print("  head %d: O, LSE on %d rows, (max, mean) abs errors %s %s" % (h, len(rows), eo, el), flush=True)
        if grads is None:
            continue
        dq, dk, dv = grads
        doh = head64(do, h)
        rdq, _, _ = oracle.attn_bwd(qh, kh, vh, doh, seg, pos, theta=w.theta, causal=w.causal, rows=rows,
                                    col_begin=0, col_end=0)
        eq = assert_parity_(dq[:, h:h + 1, rows], rdq, "%s h%d dq" % (name, h))
        print("  head %d: dq on %d rows, (max, mean) abs error %s" % (h, len(rows), eq), flush=True)
        for c0, c1 in wins:
            wrows = np.arange(c0, c1, dtype=np.int64)
            rdq, rdk, rdv = oracle.attn_bwd(qh, kh, vh, doh, seg, pos, theta=w.theta, causal=w.causal, rows=wrows,
                                            col_begin=c0, col_end=c1)
            assert_parity_(dq[:, h:h + 1, c0:c1], rdq, "%s h%d dq [%d,%d)" % (name, h, c0, c1))
            ek = assert_parity_(dk[:, h:h + 1, c0:c1], rdk, "%s h%d dk [%d,%d)" % (name, h, c0, c1))
            ev = assert_parity_(dv[:, h:h + 1, c0:c1], rdv, "%s h%d dv [%d,%d)" % (name, h, c0, c1))
            print("  head %d: keys [%d, %d): dk %s dv %s" % (h, c0, c1, ek, ev), flush=True)
    del q, k, v, do, o, lse, grads
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama7b_32k", "packing_128k"])
def test_full_size_bitwise_reproducible(torch_cuda, name):
    """Two forward + backward passes over the whole workload give the same
    bits in o, lse, dq, dk and dv: no atomics, and every kernel's result
    depends on its inputs alone (not on the order in which workgroups run)."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import WORKLOADS, make_qkv, packing

    torch = torch_cuda
    w = WORKLOADS[name]
    seg, pos, lengths = packing(w)
    q, k, v, do = make_qkv(w, device="cuda", with_grad_out=True)
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    print("bitwise reproducibility %s: B%d H%d S%d D%d" % (name, w.batch, w.heads, w.seqlen, w.head_dim), flush=True)
    runs = []
    for _ in range(2):
        o, lse = bw.attn_fwd(q, k, v, dseg, dpos, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk)
        runs.append((o, lse) + bw.attn_bwd(q, k, v, o, lse, do, dseg, dpos, theta=w.theta, causal=w.causal,
                                           kv_chunk=w.kv_chunk))
        torch.cuda.synchronize()
    for n, x, y in zip(("o", "lse", "dq", "dk", "dv"), runs[0], runs[1]):
        assert torch.equal(x, y), n
    del q, k, v, do, runs
    torch.cuda.empty_cache()


# workload, heads compared on every row for the forward, heads for the backward
EVERY_ROW = [
    ("llama7b_32k", (0, 17), (9,)),
    ("packing_128k", (3, 30), (14,)),
    ("video_text_256k", (6, 25), ()),
]


@pytest.mark.parametrize("name,fwd_heads,bwd_heads", EVERY_ROW)
def test_full_size_every_row(oracle, torch_cuda, name, fwd_heads, bwd_heads):
    """The whole workload on the GPU, and whole heads against the oracle:
    O and LSE on every row of two heads, and dq, dk, dv on every row of one
    head (the bf16 path, the benchmark's parameters)."""
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import WORKLOADS, make_qkv, packing

    torch = torch_cuda
    w = WORKLOADS[name]
    seg, pos, lengths = packing(w)
    q, k, v, do = make_qkv(w, device="cuda", with_grad_out=True)
    dseg = None if seg is None else torch.from_numpy(seg).cuda()
    dpos = torch.from_numpy(pos).cuda()
    print("every row %s: B%d H%d S%d D%d, forward heads %s, backward heads %s" % (
        name, w.batch, w.heads, w.seqlen, w.head_dim, fwd_heads, bwd_heads), flush=True)
    o, lse = bw.attn_fwd(q, k, v, dseg, dpos, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk)
    grads = None
    if bwd_heads:
        grads = bw.attn_bwd(q, k, v, o, lse, do, dseg, dpos, theta=w.theta, causal=w.causal, kv_chunk=w.kv_chunk)
    torch.cuda.synchronize()
    for h in fwd_heads:
        qh, kh, vh = head64(q, h), head64(k, h), head64(v, h)
        ro, rlse = oracle.attn_fwd(qh, kh, vh, seg, pos, theta=w.theta, causal=w.causal)
        eo = assert_parity(o[:, h:h + 1], ro, "%s h%d O" % (name, h))
        el = assert_parity(lse[:, h:h + 1].cpu().numpy(), rlse, "%s h%d LSE" % (name, h))
        print("  head %d: O, LSE on all %d rows, (max, mean) abs errors %s %s" % (h, w.seqlen, eo, el), flush=True)
    for h in bwd_heads:
        dq, dk, dv = grads
        rdq, rdk, rdv = oracle.attn_bwd(head64(q, h), head64(k, h), head64(v, h), head64(do, h), seg, pos,
                                        theta=w.theta, causal=w.causal)
        e = [assert_parity(g[:, h:h + 1], r, "%s h%d %s" % (name, h, n))
             for n, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv))]
        print("  head %d: dq, dk, dv on all %d rows, (max, mean) abs errors %s" % (h, w.seqlen, e), flush=True)
    del q, k, v, do, o, lse, grads
    torch.cuda.empty_cache()
