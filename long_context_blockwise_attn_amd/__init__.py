"""Blockwise exact causal attention with RoPE and a packing mask for MI355X.

Thin ctypes binding over the C-ABI library ``libbwattn.so`` (include/bwattn.h):
argument checks and marshalling only; every step of the computation runs in
the library's HIP kernels.  PyTorch provides device memory and the stream.
Importing this package does not load the library; the first call does, and
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["attn_fwd", "attn_bwd", "attn_decode", "attn_decode_noalloc", "rope_apply", "attn_fwd_f32", "attn_bwd_f32", "rope_apply_f32",
           "packed_ce_loss", "workspace_bytes", "decode_workspace_bytes", "packed_ce_workspace_bytes", "AttnError",
           "library_path", "Params", "CeParams"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libbwattn.so")
_lib = None


class AttnError(RuntimeError):
    pass


class Params(ctypes.Structure):
    """attn_params of include/bwattn.h."""

    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("kv_chunk", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
    ]


class CeParams(ctypes.Structure):
    """packed_ce_params of include/bwattn.h."""

    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("grad_scale", ctypes.c_float),
    ]


def make_ce_params(B, S, V, num_segments=1, grad_scale=1.0) -> CeParams:
    return CeParams(ctypes.sizeof(CeParams), B, S, V, int(num_segments), float(grad_scale))


def make_params(B, H, S, D, theta=0.0, causal=True, scale=0.0, kv_chunk=0, deterministic=False) -> Params:
    return Params(ctypes.sizeof(Params), B, H, S, D, float(scale), int(bool(causal)), float(theta), int(kv_chunk),
                  int(bool(deterministic)))


def load():
    """Load libbwattn.so (raises AttnError if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise AttnError("HIP library %s is not built; run long_context_blockwise_attn_amd/build.py" % library_path)
        lib = ctypes.CDLL(library_path)
        P, V = ctypes.POINTER(Params), ctypes.c_void_p
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [ctypes.c_int]
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_workspace_bytes.argtypes = [P, ctypes.c_int32]
        lib.rope_apply.restype = ctypes.c_int
        lib.rope_apply.argtypes = [P, V, V, V, ctypes.c_int32, V]
        lib.attn_fwd.restype = ctypes.c_int
        lib.attn_fwd.argtypes = [P, V, V, V, V, V, V, V, V, ctypes.c_size_t, V]
        lib.attn_bwd.restype = ctypes.c_int
        lib.attn_bwd.argtypes = [P, V, V, V, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V]
        lib.rope_apply_f32.restype = ctypes.c_int
        lib.rope_apply_f32.argtypes = [P, V, V, V, ctypes.c_int32, V]
        lib.attn_fwd_f32.restype = ctypes.c_int
        lib.attn_fwd_f32.argtypes = [P, V, V, V, V, V, V, V, V, ctypes.c_size_t, V]
        lib.attn_bwd_f32.restype = ctypes.c_int
        lib.attn_bwd_f32.argtypes = [P, V, V, V, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V]
        lib.attn_decode.restype = ctypes.c_int
        lib.attn_decode.argtypes = [P, ctypes.c_int32, V, V, V, V, V, V, V, ctypes.c_size_t, V]
        lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_decode_workspace_bytes.argtypes = [P, ctypes.c_int32]
        lib.attn_decode_noalloc.restype = ctypes.c_int
        lib.attn_decode_noalloc.argtypes = [P, ctypes.c_int32, V, V, V, V, V, V, V]
        lib.attn_decode_noalloc_max_bytes.restype = ctypes.c_size_t
        lib.attn_decode_noalloc_max_bytes.argtypes = []
        CP = ctypes.POINTER(CeParams)
        lib.packed_ce_workspace_bytes.restype = ctypes.c_size_t
        lib.packed_ce_workspace_bytes.argtypes = [CP]
        lib.packed_ce_loss.restype = ctypes.c_int
        lib.packed_ce_loss.argtypes = [CP, V, V, V, V, V, V, V, ctypes.c_size_t, V]
        lib.attn_profile_events.restype = ctypes.c_int
        lib.attn_profile_events.argtypes = [ctypes.c_int32, V, V, ctypes.c_int32]
        lib.attn_profile_count.restype = ctypes.c_int32
        lib.attn_profile_count.argtypes = [ctypes.c_int32]
        _lib = lib
    return _lib


def _raise(rc):
    if rc != 0:
        lib = load()
        raise AttnError("%s: %s" % (lib.attn_status_string(rc).decode(), lib.attn_last_error().decode()))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_bhsd(name, t, shape=None, f32=False, device=None):
    import torch

    dt = torch.float32 if f32 else torch.bfloat16
    if t.dtype != dt or t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
        raise AttnError("%s must be a contiguous %s CUDA tensor [B,H,S,D]" % (name, "fp32" if f32 else "bf16"))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise AttnError("%s has shape %r, expected %r" % (name, tuple(t.shape), tuple(shape)))
    _check_device(name, t, device)


def _check_device(name, t, device):
    if device is not None and t.device != device:
        raise AttnError("%s is on %s, the other tensors on %s" % (name, t.device, device))


def _check_bs(name, t, B, S, device=None):
    import torch

    if t is None:
        return None
    if t.dtype != torch.int32 or tuple(t.shape) != (B, S) or not t.is_contiguous() or not t.is_cuda:
        raise AttnError("%s must be a contiguous int32 CUDA tensor [B,S]" % name)
    _check_device(name, t, device)
    return t


def _check_lse(lse, shape, device):
    """lse: a contiguous fp32 CUDA tensor of the given shape on `device`."""
    import torch

    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous() or not lse.is_cuda:
        raise AttnError("lse must be a contiguous fp32 CUDA tensor %r" % (list(shape),))
    _check_device("lse", lse, device)


def _check_workspace(workspace, need, device):
    """A caller-supplied workspace: a contiguous CUDA tensor on `device` of
    at least `need` bytes.  Returns its size in bytes."""
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise AttnError("workspace must be a contiguous CUDA tensor")
    _check_device("workspace", workspace, device)
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise AttnError("workspace of %d bytes needed, %d given" % (need, nbytes))
    return nbytes


def workspace_bytes(params: Params, which: int) -> int:
    n = load().attn_workspace_bytes(ctypes.byref(params), which)
    if n == 0:
        _raise(1)
    return int(n)


def _workspace(params, which, workspace, device):
    import torch

    need = workspace_bytes(params, which)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, _check_workspace(workspace, need, device)


def _rope(fn, f32, x, positions, theta, inverse, out):
    import torch

    _check_bhsd("x", x, f32=f32)
    B, H, S, D = x.shape
    _check_bs("positions", positions, B, S, x.device)
    if out is not None:
        _check_bhsd("out", out, x.shape, f32=f32, device=x.device)
    else:
        out = torch.empty_like(x)
    p = make_params(B, H, S, D, theta=theta)
    _raise(fn(ctypes.byref(p), _ptr(x), _ptr(out), _ptr(positions), int(bool(inverse)), _stream()))
    return out


def rope_apply(x, positions=None, theta=1e4, inverse=False, out=None):
    """RoPE of x (bf16 [B,H,S,D]) at positions (int32 [B,S] or None)."""
    return _rope(load().rope_apply, False, x, positions, theta, inverse, out)


def rope_apply_f32(x, positions=None, theta=1e4, inverse=False, out=None):
    """RoPE of x (fp32 [B,H,S,D]) at positions (int32 [B,S] or None)."""
    return _rope(load().rope_apply_f32, True, x, positions, theta, inverse, out)


def _fwd(fn, f32, q, k, v, segment_ids, positions, theta, causal, scale, kv_chunk, out, lse, workspace):
    import torch

    _check_bhsd("q", q, f32=f32)
    B, H, S, D = q.shape
    dev = q.device
    _check_bhsd("k", k, q.shape, f32=f32, device=dev)
    _check_bhsd("v", v, q.shape, f32=f32, device=dev)
    _check_bs("segment_ids", segment_ids, B, S, dev)
    _check_bs("positions", positions, B, S, dev)
    if out is not None:
        _check_bhsd("out", out, q.shape, f32=f32, device=dev)
    if lse is not None:
        _check_lse(lse, (B, H, S), dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    p = make_params(B, H, S, D, theta=theta, causal=causal, scale=scale, kv_chunk=kv_chunk)
    ws, nbytes = _workspace(p, 2 if f32 else 0, workspace, q.device)
    _raise(fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(segment_ids), _ptr(positions), _ptr(out), _ptr(lse),
              _ptr(ws), nbytes, _stream()))
    return out, lse


def attn_fwd(q, k, v, segment_ids=None, positions=None, theta=0.0, causal=True, scale=0.0, kv_chunk=0, out=None,
             lse=None, workspace=None):
    """Blockwise exact attention forward; returns (o bf16 [B,H,S,D], lse fp32 [B,H,S])."""
    return _fwd(load().attn_fwd, False, q, k, v, segment_ids, positions, theta, causal, scale, kv_chunk, out, lse,
                workspace)


def attn_fwd_f32(q, k, v, segment_ids=None, positions=None, theta=0.0, causal=True, scale=0.0, kv_chunk=0, out=None,
                 lse=None, workspace=None):
    """attn_fwd on fp32 tensors; returns (o fp32 [B,H,S,D], lse fp32 [B,H,S])."""
    return _fwd(load().attn_fwd_f32, True, q, k, v, segment_ids, positions, theta, causal, scale, kv_chunk, out, lse,
                workspace)


def _bwd(fn, f32, q, k, v, o, lse, dout, segment_ids, positions, theta, causal, scale, kv_chunk, dq, dk, dv,
         workspace):
    import torch

    _check_bhsd("q", q, f32=f32)
    B, H, S, D = q.shape
    dev = q.device
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_bhsd(name, t, q.shape, f32=f32, device=dev)
    _check_lse(lse, (B, H, S), dev)
    _check_bs("segment_ids", segment_ids, B, S, dev)
    _check_bs("positions", positions, B, S, dev)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _check_bhsd(name, t, q.shape, f32=f32, device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    p = make_params(B, H, S, D, theta=theta, causal=causal, scale=scale, kv_chunk=kv_chunk)
    ws, nbytes = _workspace(p, 3 if f32 else 1, workspace, q.device)
    _raise(fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(segment_ids),
              _ptr(positions), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nbytes, _stream()))
    return dq, dk, dv


def attn_bwd(q, k, v, o, lse, dout, segment_ids=None, positions=None, theta=0.0, causal=True, scale=0.0, kv_chunk=0,
             dq=None, dk=None, dv=None, workspace=None):
    """Backward of attn_fwd; returns (dq, dk, dv) bf16 [B,H,S,D] with respect to
    the un-rotated q and k and to v."""
    return _bwd(load().attn_bwd, False, q, k, v, o, lse, dout, segment_ids, positions, theta, causal, scale, kv_chunk,
                dq, dk, dv, workspace)


def attn_bwd_f32(q, k, v, o, lse, dout, segment_ids=None, positions=None, theta=0.0, causal=True, scale=0.0,
                 kv_chunk=0, dq=None, dk=None, dv=None, workspace=None):
    """Backward of attn_fwd_f32; returns fp32 (dq, dk, dv) [B,H,S,D]."""
    return _bwd(load().attn_bwd_f32, True, q, k, v, o, lse, dout, segment_ids, positions, theta, causal, scale,
                kv_chunk, dq, dk, dv, workspace)


def decode_workspace_bytes(params: Params, n_q: int) -> int:
    n = load().attn_decode_workspace_bytes(ctypes.byref(params), int(n_q))
    if n == 0:
        _raise(1)
    return int(n)


def attn_decode(q, k_cache, v_cache, q_positions=None, theta=0.0, causal=True, scale=0.0, out=None, lse=None,
                workspace=None):
    """Decode attention of the n_q query rows q (bf16 [B,H,n_q,D], un-rotated;
    row r is the token at sequence index S - n_q + r) against the cache
    (k_cache rotated, v_cache; bf16 [B,H,S,D]).  Returns (o bf16 [B,H,n_q,D],
    lse fp32 [B,H,n_q])."""
    import torch

    _check_bhsd("q", q)
    B, H, nq, D = q.shape
    dev = q.device
    _check_bhsd("k_cache", k_cache, device=dev)
    S = k_cache.shape[2]
    _check_bhsd("k_cache", k_cache, (B, H, S, D))
    _check_bhsd("v_cache", v_cache, (B, H, S, D), device=dev)
    _check_bs("q_positions", q_positions, B, nq, dev)
    if out is not None:
        _check_bhsd("out", out, q.shape, device=dev)
    if lse is not None:
        _check_lse(lse, (B, H, nq), dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    p = make_params(B, H, S, D, theta=theta, causal=causal, scale=scale)
    need = decode_workspace_bytes(p, nq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    nbytes = _check_workspace(workspace, need, dev)
    _raise(load().attn_decode(ctypes.byref(p), int(nq), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(q_positions),
                              _ptr(out), _ptr(lse), _ptr(workspace), nbytes, _stream()))
    return out, lse


def attn_decode_noalloc(q, k_cache, v_cache, q_positions=None, theta=0.0, causal=True, scale=0.0, out=None,
                        lse=None):
    """attn_decode through the entry point that allocates nothing: the
    library's static device workspace stands in for the caller's (calls that
    overlap in time on one GPU race).  out and lse, when given, are written
    in place, so a caller that must not allocate passes both."""
    import torch

    _check_bhsd("q", q)
    B, H, nq, D = q.shape
    dev = q.device
    _check_bhsd("k_cache", k_cache, device=dev)
    S = k_cache.shape[2]
    _check_bhsd("k_cache", k_cache, (B, H, S, D))
    _check_bhsd("v_cache", v_cache, (B, H, S, D), device=dev)
    _check_bs("q_positions", q_positions, B, nq, dev)
    if out is not None:
        _check_bhsd("out", out, q.shape, device=dev)
    if lse is not None:
        _check_lse(lse, (B, H, nq), dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    p = make_params(B, H, S, D, theta=theta, causal=causal, scale=scale)
    _raise(load().attn_decode_noalloc(ctypes.byref(p), int(nq), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(q_positions), _ptr(out), _ptr(lse), _stream()))
    return out, lse


def packed_ce_workspace_bytes(params: CeParams) -> int:
    n = load().packed_ce_workspace_bytes(ctypes.byref(params))
    if n == 0:
        _raise(1)
    return int(n)


def packed_ce_loss(logits, targets, segment_ids=None, num_segments=1, grad_scale=1.0, with_grad=True,
                   with_token_ce=False, dlogits=None, workspace=None):
    """Re-weighted cross-entropy of packed rows (loss side of masked sequence
    packing): logits bf16 [B,S,V], targets int32 [B,S] (outside [0, V): no
    loss), segment_ids int32 [B,S] example ids in [0, num_segments) or None.
    Returns (loss fp32 [1], dlogits bf16 [B,S,V] or None, token_ce fp32 [B,S]
    or None)."""
    import torch

    if logits.dtype != torch.bfloat16 or logits.dim() != 3 or not logits.is_contiguous() or not logits.is_cuda:
        raise AttnError("logits must be a contiguous bf16 CUDA tensor [B,S,V]")
    B, S, V = logits.shape
    dev = logits.device
    if targets is None:
        raise AttnError("targets are required")
    _check_bs("targets", targets, B, S, dev)
    _check_bs("segment_ids", segment_ids, B, S, dev)
    if not with_grad:
        dlogits = None
    elif dlogits is not None:
        if (tuple(dlogits.shape) != tuple(logits.shape) or dlogits.dtype != torch.bfloat16
                or not dlogits.is_contiguous() or not dlogits.is_cuda):
            raise AttnError("dlogits must be a contiguous bf16 CUDA tensor shaped like logits")
        _check_device("dlogits", dlogits, dev)
    p = make_ce_params(B, S, V, num_segments, grad_scale)
    need = packed_ce_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    nbytes = _check_workspace(workspace, need, dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    if with_grad and dlogits is None:
        dlogits = torch.empty_like(logits)
    tce = torch.empty((B, S), dtype=torch.float32, device=dev) if with_token_ce else None
    _raise(load().packed_ce_loss(ctypes.byref(p), _ptr(logits), _ptr(targets), _ptr(segment_ids), _ptr(loss),
                                 _ptr(dlogits), _ptr(tce), _ptr(workspace), nbytes, _stream()))
    return loss, dlogits, tce
