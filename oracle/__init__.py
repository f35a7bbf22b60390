"""Oracle: plain CPU definition of blockwise causal attention with RoPE and a
packing mask, in float64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it and
shares no code with it.

The attention arithmetic lives in ``oracle.c`` (built to ``liboracle.so`` by
``build()``); this module marshals numpy arrays, except for ``attn_probs``
(the full probability and dS matrices of small cases, in numpy) and the loss
of ``packed_ce.py``.  Each function states the passage of the pages it
follows; see the header of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc and OpenMP into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_num_threads.restype = i32
        lib.oracle_rope.argtypes = [i32, i32, i32, i32, P, P, f64, i32, P]
        lib.oracle_attn_fwd.argtypes = [i32, i32, i32, i32, P, P, P, P, P, f64, f64, i32, P, i64, P, P]
        lib.oracle_attn_fwd_blocked.argtypes = [i32, i32, i32, i32, P, P, P, P, P, f64, f64, i32, i32, i32, P, P]
        lib.oracle_attn_bwd.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, f64, f64, i32, P, i64, i32, i32, P, P, P]
        for f in (lib.oracle_rope, lib.oracle_attn_fwd, lib.oracle_attn_fwd_blocked, lib.oracle_attn_bwd):
            f.restype = i32
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x, B, S):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    if a.shape != (B, S):
        raise ValueError("expected int32 [B,S], got %r" % (a.shape,))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle call failed with code %d" % rc)


def rope(x, positions=None, theta=1e4, inverse=False):
    """RoPE on [B,H,S,D]: rotate pair (x[2i], x[2i+1]) by pos * theta^(-2i/D)
    ("standard RoPE" with scaled theta: zhao9797 page, 模型架构; RoFormer)."""
    x = _f64(x)
    B, H, S, D = x.shape
    pos = _i32(positions, B, S)
    y = np.empty_like(x)
    _check(_load().oracle_rope(B, H, S, D, _ptr(x), _ptr(pos), float(theta), int(bool(inverse)), _ptr(y)))
    return y


def attn_fwd(q, k, v, segment_ids=None, positions=None, theta=0.0, scale=0.0, causal=True, rows=None):
    """Exact softmax attention (the paper's blockwise method is exact:
    elamur.ai summary page, Summary) with causal and packing masks
    (zhao9797 page, 模型架构 and 训练方法).  theta <= 0: no RoPE.

    Returns (o [B,H,n,D], lse [B,H,n]) with n = S, or len(rows) if rows given.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, S, D = q.shape
    seg, pos = _i32(segment_ids, B, S), _i32(positions, B, S)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = S if r is None else len(r)
    o = np.zeros((B, H, n, D))
    lse = np.zeros((B, H, n))
    _check(_load().oracle_attn_fwd(B, H, S, D, _ptr(q), _ptr(k), _ptr(v), _ptr(seg), _ptr(pos), float(theta),
                                   float(scale), int(bool(causal)), _ptr(r), n, _ptr(o), _ptr(lse)))
    return o, lse


def attn_fwd_blocked(q, k, v, segment_ids=None, positions=None, theta=0.0, scale=0.0, causal=True,
                     block_k=64, kv_chunk=0):
    """The blockwise online-softmax algorithm (paper: blockwise ring attention
    fused with FlashAttention; zhao9797 page, 模型架构), optionally visiting
    K/V chunks in ring order.  For block-size and order independence checks."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, S, D = q.shape
    seg, pos = _i32(segment_ids, B, S), _i32(positions, B, S)
    o = np.zeros((B, H, S, D))
    lse = np.zeros((B, H, S))
    _check(_load().oracle_attn_fwd_blocked(B, H, S, D, _ptr(q), _ptr(k), _ptr(v), _ptr(seg), _ptr(pos),
                                           float(theta), float(scale), int(bool(causal)), int(block_k),
                                           int(kv_chunk), _ptr(o), _ptr(lse)))
    return o, lse


def attn_bwd(q, k, v, dout, segment_ids=None, positions=None, theta=0.0, scale=0.0, causal=True, rows=None,
             col_begin=0, col_end=None):
    """Exact gradient of attn_fwd with respect to the un-rotated q, k and v.

    Only the listed query rows contribute (all rows if None).  Returns
    (dq [B,H,n,D] for the listed rows, dk, dv [B,H,col_end-col_begin,D]).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, S, D = q.shape
    seg, pos = _i32(segment_ids, B, S), _i32(positions, B, S)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = S if r is None else len(r)
    if col_end is None:
        col_end = S
    ncol = col_end - col_begin
    dq = np.zeros((B, H, n, D))
    dk = np.zeros((B, H, ncol, D))
    dv = np.zeros((B, H, ncol, D))
    _check(_load().oracle_attn_bwd(B, H, S, D, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(seg), _ptr(pos),
                                   float(theta), float(scale), int(bool(causal)), _ptr(r), n, int(col_begin),
                                   int(col_end), _ptr(dq), _ptr(dk), _ptr(dv)))
    return dq, dk, dv


def attn_probs(q, k, v, dout, segment_ids=None, positions=None, theta=0.0, scale=0.0, causal=True):
    """The intermediate matrices of the exact backward, for small S (numpy,
    float64, full S x S matrices per head).  With q', k' the rotated rows
    (RoPE as in rope()), s_ij = scale <q'_i, k'_j> over the visible pairs
    (causal: j <= i; packing: equal segment ids), P = softmax_j(s),
    O = P v, Delta_i = <dO_i, O_i>, dP_ij = <dO_i, v_j> and
    dS_ij = P_ij (dP_ij - Delta_i) (zhao9797 page, 训练方法: training takes
    gradient steps through the exact attention of 模型架构).

    Returns (P, dS, q', k'), P and dS [B,H,S,S] (zero off the mask), q' and
    k' [B,H,S,D].  For bounds on the rounding of these operands in the
    tests; the outputs themselves come from attn_fwd / attn_bwd."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, S, D = q.shape
    seg, pos = _i32(segment_ids, B, S), _i32(positions, B, S)
    if S > 4096:
        raise ValueError("attn_probs keeps S x S matrices; S %d is too large" % S)
    tau = scale if scale > 0 else 1.0 / np.sqrt(D)
    qr = rope(q, pos, theta) if theta > 0 else q
    kr = rope(k, pos, theta) if theta > 0 else k
    P = np.zeros((B, H, S, S))
    dS = np.zeros((B, H, S, S))
    idx = np.arange(S)
    for b in range(B):
        vis = np.ones((S, S), dtype=bool) if seg is None else seg[b][:, None] == seg[b][None, :]
        if causal:
            vis &= idx[None, :] <= idx[:, None]
        for h in range(H):
            s = np.where(vis, tau * (qr[b, h] @ kr[b, h].T), -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ v[b, h]
            delta = np.sum(dout[b, h] * o, axis=1)
            dp = dout[b, h] @ v[b, h].T
            P[b, h] = p
            dS[b, h] = np.where(vis, p * (dp - delta[:, None]), 0.0)
    return P, dS, qr, kr


# loss side of masked sequence packing (numpy, float64)
from .packed_ce import packed_ce, token_ce  # noqa: E402,F401
