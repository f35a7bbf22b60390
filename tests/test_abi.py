"""The C-ABI library loads, exports every entry point of include/bwattn.h, and
rejects bad arguments before touching the GPU (no compute call here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import long_context_blockwise_attn_amd as bw

    if not os.path.exists(bw.library_path):
        from long_context_blockwise_attn_amd import build

        build.build()
    return bw.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bwattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "rope_apply", "attn_workspace_bytes", "attn_status_string",
            "attn_last_error", "attn_profile_events", "attn_profile_count", "attn_decode",
            "attn_decode_workspace_bytes", "attn_fwd_f32", "attn_bwd_f32", "rope_apply_f32", "packed_ce_loss",
            "packed_ce_workspace_bytes", "attn_decode_noalloc", "attn_decode_noalloc_max_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_params_layout_matches_header():
    import long_context_blockwise_attn_amd as bw

    # int32 x5, float, int32, (pad), double, int32 x2 -> 48 bytes with 8-byte alignment
    assert ctypes.sizeof(bw.Params) == 48
    assert bw.Params.rope_theta.offset == 32


def call_fwd(lib, p, q=16, k=32, v=48, seg=None, pos=None, o=64, lse=80, ws=None, nbytes=0):
    V = ctypes.c_void_p
    return lib.attn_fwd(ctypes.byref(p) if p is not None else None, V(q) if q else None, V(k) if k else None,
                        V(v) if v else None, V(seg) if seg else None, V(pos) if pos else None, V(o) if o else None,
                        V(lse) if lse else None, V(ws) if ws else None, nbytes, None)


def test_argument_errors_before_any_hip_call(lib):
    import long_context_blockwise_attn_amd as bw

    ok = bw.make_params(1, 2, 1024, 128, theta=1e6)
    assert call_fwd(lib, None) == 1
    bad = bw.make_params(1, 2, 1024, 128)
    bad.struct_size = 40
    assert call_fwd(lib, bad) == 1 and b"struct_size" in lib.attn_last_error()
    assert call_fwd(lib, bw.make_params(0, 2, 1024, 128)) == 1
    assert call_fwd(lib, bw.make_params(1, 2, 0, 128)) == 1
    assert call_fwd(lib, bw.make_params(1, 2, 1024, 96)) == 2
    assert call_fwd(lib, bw.make_params(1, 2, 1024, 128, kv_chunk=100)) == 1
    assert call_fwd(lib, bw.make_params(1, 2, 1024, 128, theta=float("nan"))) == 1
    p = bw.make_params(1, 2, 1024, 128)
    p.causal = 2
    assert call_fwd(lib, p) == 1
    assert call_fwd(lib, ok, q=0) == 1
    assert call_fwd(lib, ok, q=18) == 1 and b"aligned" in lib.attn_last_error()
    assert call_fwd(lib, ok, ws=None) == 3
    assert call_fwd(lib, ok, ws=4096, nbytes=16) == 3
    assert lib.attn_status_string(3) == b"ATTN_ERR_WORKSPACE"
    V = ctypes.c_void_p
    assert lib.rope_apply(ctypes.byref(bw.make_params(1, 1, 8, 64, theta=0.0)), V(16), V(16), None, 0, None) == 1
    assert lib.rope_apply(ctypes.byref(ok), V(16), V(16), None, 2, None) == 1
    # attn_bwd(p, q, k, v, o, lse, d_o, seg, pos, dq, dk, dv, ws, ws_bytes, stream)
    args = [ctypes.byref(ok)] + [V(16 * (i + 1)) for i in range(12)] + [0, None]
    args[7] = None  # segment_ids may be NULL
    args[8] = None  # positions may be NULL
    args[12] = None
    assert lib.attn_bwd(*args) == 3  # no workspace
    args[5] = None  # lse is required
    assert lib.attn_bwd(*args) == 1


def test_f32_argument_errors_before_any_hip_call(lib):
    import long_context_blockwise_attn_amd as bw

    V = ctypes.c_void_p
    ok = bw.make_params(1, 2, 1024, 128, theta=1e6)

    def fwd(p=ok, q=16, ws=None, nbytes=0):
        return lib.attn_fwd_f32(ctypes.byref(p), V(q) if q else None, V(32), V(48), None, None, V(64), V(80),
                                V(ws) if ws else None, nbytes, None)

    assert fwd(q=0) == 1
    assert fwd(q=20) == 1 and b"aligned" in lib.attn_last_error()
    assert fwd(p=bw.make_params(1, 2, 1024, 80)) == 2
    assert fwd() == 3
    assert fwd(ws=4096, nbytes=bw.workspace_bytes(ok, 2) - 1) == 3
    args = [ctypes.byref(ok)] + [V(16 * (i + 1)) for i in range(12)] + [0, None]
    args[7] = args[8] = args[12] = None
    assert lib.attn_bwd_f32(*args) == 3
    args[10] = None  # dk is required
    assert lib.attn_bwd_f32(*args) == 1
    assert lib.rope_apply_f32(ctypes.byref(bw.make_params(1, 1, 8, 64, theta=0.0)), V(16), V(16), None, 0, None) == 1
    assert lib.rope_apply_f32(ctypes.byref(ok), V(16), V(16), None, 3, None) == 1


def test_f32_workspace_holds_fp32_rotated_rows(lib):
    import long_context_blockwise_attn_amd as bw

    p = bw.make_params(1, 32, 32768, 128, theta=1e6)
    n = 32 * 32768 * 128
    f, b = bw.workspace_bytes(p, 2), bw.workspace_bytes(p, 3)
    assert f >= 2 * n * 4 and b >= 2 * n * 4 + 2 * 32 * 32768 * 4
    # the same layout with bf16 rows (no transposed copies on either path); the
    # bf16 forward keeps only k' (it rotates its query rows as it loads them)
    assert bw.workspace_bytes(p, 0) == n * 2 + (f - 2 * n * 4)
    p0 = bw.make_params(1, 32, 32768, 128, theta=0.0)
    assert bw.workspace_bytes(p0, 2) == f - 2 * n * 4


def test_workspace_size_depends_only_on_params(lib):
    import long_context_blockwise_attn_amd as bw

    p = bw.make_params(1, 32, 32768, 128, theta=1e6)
    f, b = bw.workspace_bytes(p, 0), bw.workspace_bytes(p, 1)
    n = 32 * 32768 * 128
    assert f >= n * 2 and b >= 2 * n * 2 + 32 * 32768 * 4
    p0 = bw.make_params(1, 32, 32768, 128, theta=0.0)
    assert bw.workspace_bytes(p0, 0) < f
    assert lib.attn_workspace_bytes(ctypes.byref(p), 7) == 0


def test_profile_hook_arguments(lib):
    assert lib.attn_profile_events(10, None, None, 0) == 1
    assert lib.attn_profile_events(1, None, None, -1) == 1
    assert lib.attn_profile_events(1, None, None, 3) == 1
    assert lib.attn_profile_events(1, None, None, 0) == 0
    assert lib.attn_profile_count(1) == 0
    assert lib.attn_profile_count(17) == -1


def test_decode_argument_errors_before_any_hip_call(lib):
    import long_context_blockwise_attn_amd as bw

    V = ctypes.c_void_p
    p = bw.make_params(1, 2, 4096, 128, theta=1e6)

    def call(n_q=4, q=16, k=32, v=48, pos=None, o=64, lse=80, ws=None, nbytes=0, params=p):
        return lib.attn_decode(ctypes.byref(params), n_q, V(q) if q else None, V(k) if k else None,
                               V(v) if v else None, V(pos) if pos else None, V(o) if o else None,
                               V(lse) if lse else None, V(ws) if ws else None, nbytes, None)

    assert call(n_q=0) == 1 and b"n_q" in lib.attn_last_error()
    assert call(n_q=33) == 1
    assert call(n_q=5, params=bw.make_params(1, 2, 4, 128)) == 1  # more rows than cached keys
    assert call(q=0) == 1
    assert call(k=40) == 1 and b"aligned" in lib.attn_last_error()
    assert call(params=bw.make_params(1, 2, 4096, 96)) == 2
    assert call() == 3  # no workspace
    assert call(ws=4096, nbytes=16) == 3
    assert lib.attn_decode_workspace_bytes(ctypes.byref(p), 0) == 0
    n1 = bw.decode_workspace_bytes(p, 1)
    n32 = bw.decode_workspace_bytes(p, 32)
    assert 0 < n1 < n32


def test_decode_split_is_chunks_of_tiles(lib):
    """The workspace holds one partial state per chunk and row: its size pins
    the chunk count the plan chose (about 2048 chunks in all, at least 256
    keys and at most 2^20 keys each)."""
    import long_context_blockwise_attn_amd as bw

    for B, H, S in ((1, 32, 1 << 20), (1, 2, 1000), (2, 1, 300), (1, 32, 32), (16, 64, 1 << 22)):
        p = bw.make_params(B, H, S, 128, theta=0.0)
        n = bw.decode_workspace_bytes(p, 1)
        # the scaled query row (bf16), partial O (D floats) + (m, l), each 256-byte aligned
        q_rows, per_chunk_o, per_chunk_ml = B * H * 128 * 2, B * H * 128 * 4, B * H * 2 * 4
        al = lambda x: (x + 255) // 256 * 256
        # ... and at most 2^20 keys per chunk
        want = max(min(max(1, -(-2048 // (B * H))), max(1, -(-S // 256))), -(-S // (1 << 20)))
        chunk = -(-(-(-S // want)) // 32) * 32
        nc = -(-S // chunk)
        assert n == al(q_rows) + al(nc * per_chunk_o) + al(nc * per_chunk_ml), (B, H, S, n, nc)


def test_packed_ce_argument_errors_before_any_hip_call(lib):
    import long_context_blockwise_attn_amd as bw

    V = ctypes.c_void_p
    ok = bw.make_ce_params(1, 1024, 40192, num_segments=64)
    assert ctypes.sizeof(bw.CeParams) == 24

    def call(p=ok, logits=16, targets=32, seg=None, loss=48, dl=64, tce=None, ws=None, nbytes=0):
        return lib.packed_ce_loss(ctypes.byref(p), V(logits) if logits else None, V(targets) if targets else None,
                                  V(seg) if seg else None, V(loss) if loss else None, V(dl) if dl else None,
                                  V(tce) if tce else None, V(ws) if ws else None, nbytes, None)

    assert call(logits=0) == 1 and call(targets=0) == 1 and call(loss=0) == 1
    assert call(logits=24) == 1 and b"aligned" in lib.attn_last_error()
    assert call(targets=34) == 1
    assert call(p=bw.make_ce_params(1, 1024, 40190)) == 1  # not a multiple of 8
    assert call(p=bw.make_ce_params(1, 1024, 65544)) == 2  # above the largest vocabulary
    assert call(p=bw.make_ce_params(1, 1024, 4096, num_segments=0)) == 1
    assert call(p=bw.make_ce_params(1, 1024, 4096, grad_scale=float("inf"))) == 1
    bad = bw.make_ce_params(1, 1024, 4096)
    bad.struct_size = 20
    assert call(p=bad) == 1
    assert call() == 3  # no workspace
    n = bw.packed_ce_workspace_bytes(ok)
    assert n == 256 + 256 + 1024 * 4  # counts, weights (64 each, 256-byte aligned), one float per row
    assert call(ws=4096, nbytes=n - 1) == 3
    assert lib.packed_ce_workspace_bytes(ctypes.byref(bw.make_ce_params(1, 8, 7))) == 0


class FakeTensor:
    """Stands in for a torch tensor in the binding's argument checks (no
    device memory is touched: every case below is refused before the
    library is called)."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True):
        import torch

        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contiguous = contiguous

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contiguous

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        import torch

        return {torch.bfloat16: 2, torch.float32: 4, torch.int32: 4, torch.uint8: 1}[self.dtype]

    def data_ptr(self):
        raise AssertionError("the binding passed a refused tensor to the library")


def test_binding_refuses_bad_lse_and_workspace():
    """lse and the workspace are checked for dtype, shape, contiguity and
    device before any pointer reaches the library (a host pointer or a short
    buffer would otherwise be handed to the kernels)."""
    import torch

    import long_context_blockwise_attn_amd as bw

    B, H, S, D = 1, 2, 64, 128
    bf = torch.bfloat16

    def t(shape=(B, H, S, D), dtype=bf, device="cuda:0", contiguous=True):
        return FakeTensor(shape, dtype, device, contiguous)

    q, k, v, o, do = t(), t(), t(), t(), t()
    good_lse = t((B, H, S), torch.float32)
    bad_lses = [t((B, H, S), torch.float32, device="cpu"), t((B, H, S - 1), torch.float32),
                t((B, H, S), bf), t((B, H, S), torch.float32, contiguous=False),
                t((B, H, S), torch.float32, device="cuda:1")]
    for lse in bad_lses:
        with pytest.raises(bw.AttnError, match="lse"):
            bw.attn_fwd(q, k, v, lse=lse, out=o)
        with pytest.raises(bw.AttnError, match="lse"):
            bw.attn_bwd(q, k, v, o, lse, do, dq=t(), dk=t(), dv=t())
    for ws in [t((1 << 20,), torch.uint8, device="cpu"), t((1 << 20,), torch.uint8, device="cuda:1"),
               t((16,), torch.uint8)]:
        with pytest.raises(bw.AttnError, match="workspace"):
            bw.attn_fwd(q, k, v, lse=good_lse, out=o, workspace=ws)
        with pytest.raises(bw.AttnError, match="workspace"):
            bw.attn_bwd(q, k, v, o, good_lse, do, dq=t(), dk=t(), dv=t(), workspace=ws)
    # every tensor on q's device
    with pytest.raises(bw.AttnError, match="k is on"):
        bw.attn_fwd(q, t(device="cuda:1"), v, lse=good_lse, out=o)
    with pytest.raises(bw.AttnError, match="dv is on"):
        bw.attn_bwd(q, k, v, o, good_lse, do, dq=t(), dk=t(), dv=t(device="cuda:1"))
    with pytest.raises(bw.AttnError, match="segment_ids is on"):
        bw.attn_fwd(q, k, v, FakeTensor((B, S), torch.int32, "cuda:1"), lse=good_lse, out=o)
    with pytest.raises(bw.AttnError, match="segment_ids"):
        bw.attn_fwd(q, k, v, FakeTensor((B, S), torch.int32, "cpu"), lse=good_lse, out=o)
    # decode: lse, out and workspace alike
    qd = t((B, H, 4, D))
    with pytest.raises(bw.AttnError, match="lse"):
        bw.attn_decode(qd, k, v, out=t((B, H, 4, D)), lse=t((B, H, 4), torch.float32, device="cpu"))
    with pytest.raises(bw.AttnError, match="workspace"):
        bw.attn_decode(qd, k, v, out=t((B, H, 4, D)), lse=t((B, H, 4), torch.float32),
                       workspace=t((1 << 20,), torch.uint8, device="cpu"))
    # packed cross-entropy: dlogits and workspace
    logits = t((B, S, 64))
    tg = FakeTensor((B, S), torch.int32)
    with pytest.raises(bw.AttnError, match="dlogits"):
        bw.packed_ce_loss(logits, tg, dlogits=t((B, S, 64), device="cpu"))
    with pytest.raises(bw.AttnError, match="workspace"):
        bw.packed_ce_loss(logits, tg, dlogits=t((B, S, 64)), workspace=t((8,), torch.uint8))


def test_decode_noalloc_refuses_what_its_static_workspace_cannot_hold(lib):
    """attn_decode_noalloc takes no workspace: parameters that need more than
    its static array are refused with ATTN_ERR_WORKSPACE before any HIP
    call; the largest decode shapes of the workloads fit."""
    import long_context_blockwise_attn_amd as bw

    V = ctypes.c_void_p
    cap = lib.attn_decode_noalloc_max_bytes()
    assert cap == 64 << 20
    wide = bw.make_params(64, 64, 1024, 128)
    assert bw.decode_workspace_bytes(wide, 32) > cap
    rc = lib.attn_decode_noalloc(ctypes.byref(wide), 32, V(16), V(32), V(48), None, V(64), V(80), None)
    assert rc == 3 and b"attn_decode_noalloc" in lib.attn_last_error()
    for B, H, S, nq in ((1, 32, 1 << 20, 32), (1, 32, 1 << 20, 1), (8, 32, 1 << 16, 32), (1, 2048, 4096, 32)):
        assert bw.decode_workspace_bytes(bw.make_params(B, H, S, 128), nq) <= cap, (B, H, S, nq)
