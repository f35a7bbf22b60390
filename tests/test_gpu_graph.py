"""The library's calls captured in a HIP graph (through torch.cuda.graph) and
replayed: the library allocates nothing, never synchronizes and clears its
counters with a kernel rather than a memset, so a captured sequence must give
the eager results on every replay.  Each replay is separated by eager work
and a synchronization, and every replay is compared bitwise with the eager
result."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_graph_replays_match_eager(torch_cuda):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case, random_ce_case

    torch = torch_cuda
    B, H, S, D = 1, 4, 1500, 128
    (q, k, v, do), seg, pos = random_case(B, H, S, D, seed=31, n_docs=4)
    q, k, v, do = (t.cuda() for t in (q, k, v, do))
    dseg, dpos = torch.from_numpy(seg).cuda(), torch.from_numpy(pos).cuda()
    theta = 1e6
    p = bw.make_params(B, H, S, D, theta=theta)
    ws_f = torch.empty(bw.workspace_bytes(p, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(bw.workspace_bytes(p, 1), dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    # decode rows against a rotated cache
    kc = bw.rope_apply(k, dpos, theta=theta)
    nq = 4
    qd = q[:, :, S - nq:].contiguous()
    pd = bw.make_params(B, H, S, D, theta=theta)
    ws_d = torch.empty(bw.decode_workspace_bytes(pd, nq), dtype=torch.uint8, device="cuda")
    od, lsed = torch.empty_like(qd), torch.empty((B, H, nq), dtype=torch.float32, device="cuda")
    # packed cross-entropy
    x, tg, sg = random_ce_case(1, 700, 4096, seed=37, n_docs=5)
    logits = torch.from_numpy(x).to(torch.bfloat16).cuda()
    targets, cseg = torch.from_numpy(tg).cuda(), torch.from_numpy(sg).cuda()
    ws_c = torch.empty(bw.packed_ce_workspace_bytes(bw.make_ce_params(1, 700, 4096, 5)), dtype=torch.uint8,
                       device="cuda")
    dl = torch.empty_like(logits)
    ce_out = {}

    def body():
        bw.attn_fwd(q, k, v, dseg, dpos, theta=theta, out=o, lse=lse, workspace=ws_f)
        bw.attn_bwd(q, k, v, o, lse, do, dseg, dpos, theta=theta, dq=dq, dk=dk, dv=dv, workspace=ws_b)
        bw.attn_decode(qd, kc, v, dpos[:, S - nq:].contiguous(), theta=theta, out=od, lse=lsed, workspace=ws_d)
        ce_out["loss"] = bw.packed_ce_loss(logits, targets, cseg, 5, dlogits=dl, workspace=ws_c)[0]

    outs = (o, lse, dq, dk, dv, od, lsed, dl)
    body()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs] + [ce_out["loss"].clone()]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the allocator on the capture stream
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    graph_loss = ce_out["loss"]
    print("graph captured", flush=True)
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays; the replay must overwrite it
        graph_loss.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(list(outs) + [graph_loss], eager)):
            assert torch.equal(t, e), "replay %d: output %d differs from the eager result" % (rep, i)
        print("  replay %d matches" % rep, flush=True)
    del g
