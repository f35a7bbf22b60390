"""Segment ids that are not contiguous (the packing mask is equality of ids:
zhao9797 page "LWM (Large World Model)", 训练方法).  Ids change per 64-row
tile so that a block's range of candidate tiles contains tiles of other
segments: the walks must test each tile there, while for contiguous
segments every tile in the range is useful.  Also two batch rows packed
differently, and many documents shorter than a tile.  Forward and backward,
bf16 and fp32 paths, against the oracle."""
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


# segment id of each 64-row tile
TILE_IDS = [0, 0, 0, 0, 7, 7, 0, 0, 3, 3, 0, 0, 7, 7, 0, 3, 3, 7]


@pytest.mark.parametrize("path", ["bf16", "f32"])
@pytest.mark.parametrize("causal,kv_chunk", [(False, 0), (True, 0), (False, 256)])
def test_interleaved_segments(oracle, torch_cuda, path, causal, kv_chunk):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case

    torch = torch_cuda
    S = 64 * len(TILE_IDS) - 17  # ragged last tile
    B, H, D = 1, 2, 128
    f32 = path == "f32"
    (q, k, v, do), _, pos = random_case(B, H, S, D, seed=S + causal, dtype="fp32" if f32 else "bf16")
    seg = np.repeat(np.array(TILE_IDS, dtype=np.int32), 64)[:S][None]
    print("interleaved segments %s S%d causal %d chunk %d" % (path, S, causal, kv_chunk), flush=True)
    fwd, bwd = (bw.attn_fwd_f32, bw.attn_bwd_f32) if f32 else (bw.attn_fwd, bw.attn_bwd)
    dseg, dpos = torch.from_numpy(seg).cuda(), torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fwd(qc, kc, vc, dseg, dpos, theta=1e6, causal=causal, kv_chunk=kv_chunk)
    dq, dk, dv = bwd(qc, kc, vc, o, lse, doc, dseg, dpos, theta=1e6, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    bars = dict(max_abs=2e-4, mean_abs=2e-5) if f32 else {}
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=1e6, causal=causal)
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=1e6, causal=causal)
    assert_parity(o, ro, "O", **bars)
    assert_parity(lse.cpu().numpy(), rlse, "LSE", **bars)
    assert_parity(dq, rdq, "dq", **bars)
    assert_parity(dk, rdk, "dk", **bars)
    assert_parity(dv, rdv, "dv", **bars)


# Two batch rows packed differently: every per-row table (segment block
# ranges, tile ranges, segment ids read by the kernels) is indexed by the row.
ROW_LENGTHS = [[100, 250, 350], [30, 400, 20, 131, 119]]


@pytest.mark.parametrize("path", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_batch_rows_with_different_packings(oracle, torch_cuda, path, causal):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case, segments_from_lengths

    torch = torch_cuda
    S = sum(ROW_LENGTHS[0])
    assert all(sum(r) == S for r in ROW_LENGTHS)
    B, H, D = len(ROW_LENGTHS), 2, 128
    f32 = path == "f32"
    (q, k, v, do), _, _ = random_case(B, H, S, D, seed=41 + causal, dtype="fp32" if f32 else "bf16")
    rows = [segments_from_lengths(r, 1) for r in ROW_LENGTHS]
    seg = np.concatenate([r[0] for r in rows])
    pos = np.concatenate([r[1] for r in rows])
    print("batch rows with different packings %s causal %d" % (path, causal), flush=True)
    fwd, bwd = (bw.attn_fwd_f32, bw.attn_bwd_f32) if f32 else (bw.attn_fwd, bw.attn_bwd)
    dseg, dpos = torch.from_numpy(seg).cuda(), torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fwd(qc, kc, vc, dseg, dpos, theta=1e6, causal=causal)
    dq, dk, dv = bwd(qc, kc, vc, o, lse, doc, dseg, dpos, theta=1e6, causal=causal)
    torch.cuda.synchronize()
    bars = dict(max_abs=2e-4, mean_abs=2e-5) if f32 else {}
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=1e6, causal=causal)
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=1e6, causal=causal)
    assert_parity(o, ro, "O", **bars)
    assert_parity(lse.cpu().numpy(), rlse, "LSE", **bars)
    assert_parity(dq, rdq, "dq", **bars)
    assert_parity(dk, rdk, "dk", **bars)
    assert_parity(dv, rdv, "dv", **bars)


# Many documents shorter than a tile: every 32-row block and every tile holds
# several segments, so masks take the segment test (alone off the diagonal,
# with the position limit on it) in every tile of a document edge.
TINY_LENGTHS = [1, 2, 3, 5, 8, 13, 31, 33, 64, 65, 1, 1, 127, 2, 40, 7, 100, 1, 19, 250, 3]


@pytest.mark.parametrize("path", ["bf16", "f32"])
@pytest.mark.parametrize("causal,kv_chunk", [(True, 0), (False, 0), (True, 128)])
def test_many_tiny_documents(oracle, torch_cuda, path, causal, kv_chunk):
    import long_context_blockwise_attn_amd as bw
    from long_context_blockwise_attn_amd.inputs import random_case, segments_from_lengths

    torch = torch_cuda
    S = sum(TINY_LENGTHS)
    B, H, D = 1, 2, 128
    f32 = path == "f32"
    (q, k, v, do), _, _ = random_case(B, H, S, D, seed=S + causal + kv_chunk, dtype="fp32" if f32 else "bf16")
    seg, pos = segments_from_lengths(TINY_LENGTHS, B)
    print("tiny documents %s S%d causal %d chunk %d" % (path, S, causal, kv_chunk), flush=True)
    fwd, bwd = (bw.attn_fwd_f32, bw.attn_bwd_f32) if f32 else (bw.attn_fwd, bw.attn_bwd)
    dseg, dpos = torch.from_numpy(seg).cuda(), torch.from_numpy(pos).cuda()
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fwd(qc, kc, vc, dseg, dpos, theta=1e6, causal=causal, kv_chunk=kv_chunk)
    dq, dk, dv = bwd(qc, kc, vc, o, lse, doc, dseg, dpos, theta=1e6, causal=causal, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    bars = dict(max_abs=2e-4, mean_abs=2e-5) if f32 else {}
    ro, rlse = oracle.attn_fwd(to64(q), to64(k), to64(v), seg, pos, theta=1e6, causal=causal)
    rdq, rdk, rdv = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), seg, pos, theta=1e6, causal=causal)
    assert_parity(o, ro, "O", **bars)
    assert_parity(lse.cpu().numpy(), rlse, "LSE", **bars)
    assert_parity(dq, rdq, "dq", **bars)
    assert_parity(dk, rdk, "dk", **bars)
    assert_parity(dv, rdv, "dv", **bars)
