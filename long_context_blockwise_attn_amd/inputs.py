"""Seeded synthetic inputs shaped like the workloads on the pages.

This module holds no attention arithmetic: it only draws random tensors and
the packing structure (segment ids and per-document positions).  Both the GPU
path and the oracle take their inputs from here, so the tests and the
benchmark see the same values on both sides.

Workloads (B batch, H heads, D head dim, S sequence length):

tiny
    B1 H2 D64 S1024, q/k/v float32 N(0,1) from numpy PCG64(seed), cast to
    bf16 (round to nearest even) for the GPU; theta 1e4; one document; causal.
llama7b_32k
    B1 H32 D128 S32768 (a LLaMA-2-7B attention layer; zhao9797 page, 模型架构),
    bf16 N(0,1); theta 1e6 (the 32K stage, 训练方法 Stage I table); one
    document; causal.
packing_128k
    B1 H32 D128 S131072, theta 1e7 (the 128K stage); documents with lengths
    log-uniform in [512, 32768] packed into one row (masked sequence packing,
    训练方法), positions restart per document; causal + segment mask.
video_text_256k
    B1 H32 D128 S262144, theta 1e7; records of a text span (uniform 64..2048
    tokens) and a 30-frame clip of 256 vision tokens per frame (数据: video
    sampled at 30 frames; 模型架构: 256 tokens per 256x256 frame, <eof> after
    every frame but the last, <eov> after the last, <vision>...</vision>
    around the clip), one record per segment, order of text and clip drawn at
    random (数据: modality order swapped at random); causal + segment mask.
full_1m
    B1 H32 D128 S1048576, theta 5e7 (the 1M stage); one document; causal; the
    sequence is cut into 64 chunks of 16384 and K/V are visited in ring order.
decode_1m
    B1 H32 D128, a cache of S = 1048576 keys and values, theta 5e7, and n_q = 1
    new query row per (b,h) (token-by-token generation at 1M context); bf16
    N(0,1) q [B,H,n_q,D], k, v [B,H,S,D]; causal.
packed_ce_32k
    the loss side of masked sequence packing: B1 S32768 token rows of bf16
    logits over V = 40192 (LLaMA-2's 32000 BPE tokens plus the 8192 codes of
    the image tokenizer's VQGAN codebook), N(0, 2^2); short-context examples
    (数据: image and video chat data packed to the context length) with
    lengths log-uniform in [128, 8192], the last one cut; in each example of
    length L the last round(U(0.2, 0.8) L) rows are the answer and carry a
    uniform random target, except the example's last row (its next token
    belongs to the next example); all other rows carry no loss (-1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# tokens of one 30-frame clip: 30 frames x 256 tokens, 29 <eof>, 1 <eov>,
# <vision> and </vision>
FRAMES_PER_CLIP = 30
TOKENS_PER_FRAME = 256
CLIP_TOKENS = FRAMES_PER_CLIP * TOKENS_PER_FRAME + (FRAMES_PER_CLIP - 1) + 1 + 2


@dataclass
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    seqlen: int
    theta: float
    causal: bool = True
    packing: str = "none"  # none | loguniform | video_text
    kv_chunk: int = 0
    backward: bool = True
    seed: int = 0
    input_dtype: str = "bf16"  # bf16, or fp32 drawn then rounded to bf16
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 1024, 1e4, backward=False, seed=1, input_dtype="fp32"),
    "llama7b_32k": Workload("llama7b_32k", 1, 32, 128, 32768, 1e6, seed=2),
    "packing_128k": Workload("packing_128k", 1, 32, 128, 131072, 1e7, packing="loguniform", seed=3),
    "video_text_256k": Workload("video_text_256k", 1, 32, 128, 262144, 1e7, packing="video_text",
                                backward=False, seed=4),
    "full_1m": Workload("full_1m", 1, 32, 128, 1048576, 5e7, kv_chunk=16384, seed=5),
    "decode_1m": Workload("decode_1m", 1, 32, 128, 1048576, 5e7, backward=False, seed=6, extra={"n_q": 1}),
    "packed_ce_32k": Workload("packed_ce_32k", 1, 0, 0, 32768, 0.0, packing="loguniform", backward=False, seed=7,
                              extra={"vocab": 40192, "lengths": (128, 8192)}),
}


def loguniform_lengths(total: int, lo: int, hi: int, seed: int) -> list[int]:
    """Document lengths L = round(exp(U(ln lo, ln hi))) drawn until they cover
    `total` tokens; the last one is cut so the lengths sum to `total`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out, acc = [], 0
    while acc < total:
        L = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = min(L, total - acc)
        out.append(L)
        acc += L
    return out


def video_text_lengths(total: int, seed: int) -> list[int]:
    """Record lengths: a text span of U{64..2048} tokens plus one clip of
    CLIP_TOKENS tokens; one record per segment, last record cut to fit.  The
    text-first or clip-first order is drawn too but does not change a record's
    length, so only the length is returned."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out, acc = [], 0
    while acc < total:
        text = int(rng.integers(64, 2049))
        _text_first = bool(rng.integers(0, 2))
        L = min(text + CLIP_TOKENS, total - acc)
        out.append(L)
        acc += L
    return out


def segments_from_lengths(lengths, batch: int = 1):
    """int32 [B,S] segment ids (document index) and positions restarting at 0
    in every document; the same packing for every batch row."""
    seg = np.concatenate([np.full(L, i, dtype=np.int32) for i, L in enumerate(lengths)])
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lengths])
    return np.tile(seg, (batch, 1)), np.tile(pos, (batch, 1))


def packing(w: Workload):
    """(segment_ids, positions, lengths) as int32 numpy [B,S]; segment_ids is
    None for a single document (positions are then 0..S-1)."""
    S = w.seqlen
    if w.packing == "none":
        return None, np.tile(np.arange(S, dtype=np.int32), (w.batch, 1)), [S]
    if w.packing == "loguniform":
        lengths = loguniform_lengths(S, 512, 32768, w.seed)
    elif w.packing == "video_text":
        lengths = video_text_lengths(S, w.seed)
    else:
        raise ValueError(w.packing)
    seg, pos = segments_from_lengths(lengths, w.batch)
    return seg, pos, lengths


def randn_bf16(shape, seed: int, device="cpu", fp32_numpy: bool = False):
    """bf16 N(0,1) tensor.  fp32_numpy=True draws float32 with numpy PCG64 and
    rounds to bf16 (round to nearest even, torch's cast); otherwise torch's
    generator on `device` draws it."""
    import torch

    if fp32_numpy:
        rng = np.random.Generator(np.random.PCG64(seed))
        x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
        return x.to(torch.bfloat16).to(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_qkv(w: Workload, device="cpu", with_grad_out: bool = False, heads: int | None = None, dtype="bf16"):
    """q, k, v (and dO) [B,H,S,D] for workload w: bf16, or with dtype "fp32"
    the float32 N(0,1) draws themselves (torch generator, same seeds).  heads
    overrides H (a subset of a workload's heads for cheaper tests)."""
    H = w.heads if heads is None else heads
    shape = (w.batch, H, w.seqlen, w.head_dim)
    if dtype == "fp32":
        import torch

        out = []
        for i in range(4 if with_grad_out else 3):
            g = torch.Generator(device=device)
            g.manual_seed(w.seed * 16 + i)
            out.append(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
        return tuple(out)
    fp32 = w.input_dtype == "fp32"
    if fp32:
        # one numpy draw for q, k, v in sequence so the seed fixes all three
        rng = np.random.Generator(np.random.PCG64(w.seed))
        import torch

        ts = [torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32)).to(torch.bfloat16).to(device)
              for _ in range(4 if with_grad_out else 3)]
    else:
        ts = [randn_bf16(shape, w.seed * 16 + i, device) for i in range(4 if with_grad_out else 3)]
    return tuple(ts)


def random_case(B, H, S, D, seed, n_docs=0, device="cpu", dtype="bf16"):
    """Small random case for parity tests: q, k, v and dO, float32 N(0,1)
    from numpy PCG64(seed), kept as float32 for dtype "fp32", else rounded to
    bf16; and, if n_docs > 0, n_docs contiguous documents of random lengths
    (positions restart per document); otherwise one document with positions
    0..S-1."""
    import torch

    rng = np.random.Generator(np.random.PCG64(seed))
    if n_docs > 0:
        cuts = np.sort(rng.choice(np.arange(1, S), size=min(n_docs - 1, S - 1), replace=False))
        lengths = np.diff(np.concatenate([[0], cuts, [S]])).astype(int).tolist()
        seg, pos = segments_from_lengths(lengths, B)
    else:
        seg, pos = None, np.tile(np.arange(S, dtype=np.int32), (B, 1))
    shape = (B, H, S, D)
    out_dtype = torch.float32 if dtype == "fp32" else torch.bfloat16
    ts = [torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32)).to(out_dtype).to(device)
          for i in range(4)]
    return ts, seg, pos


def ce_targets(lengths, V, seed, batch=1):
    """int32 [B, S] targets and segment ids for packed examples of the given
    lengths: the last round(U(0.2, 0.8) L) rows of an example of length L are
    its answer and get a uniform random target in [0, V), except the
    example's last row; every other row gets -1 (no loss)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seg, _ = segments_from_lengths(lengths, batch)
    S = int(sum(lengths))
    tg = np.full((batch, S), -1, dtype=np.int32)
    for b in range(batch):
        s0 = 0
        for L in lengths:
            a = max(1, int(round(rng.uniform(0.2, 0.8) * L)))
            lo, hi = s0 + L - a, s0 + L - 1  # answer rows lo .. hi-1 (the last row has no target)
            if hi > lo:
                tg[b, lo:hi] = rng.integers(0, V, size=hi - lo)
            s0 += L
    return tg, seg


def packed_ce_case(w: Workload, device="cpu"):
    """(logits bf16 [B,S,V], targets int32 [B,S], segment ids int32 [B,S],
    num_segments) of a packed cross-entropy workload."""
    import torch

    V = w.extra["vocab"]
    lo, hi = w.extra["lengths"]
    lengths = loguniform_lengths(w.seqlen, lo, hi, w.seed)
    tg, seg = ce_targets(lengths, V, w.seed + 1, w.batch)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 16)
    logits = (2.0 * torch.randn((w.batch, w.seqlen, V), generator=g, device=device, dtype=torch.float32)).to(
        torch.bfloat16)
    return logits, torch.from_numpy(tg).to(device), torch.from_numpy(seg).to(device), len(lengths)


def random_ce_case(B, S, V, seed, n_docs, ignore_frac=0.3):
    """Small packed cross-entropy case (numpy PCG64): bf16 logits N(0, 2^2)
    [B,S,V] (as float32 values), targets with a fraction of rows marked -1,
    and n_docs contiguous examples of random lengths per row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (2.0 * rng.standard_normal((B, S, V))).astype(np.float32)
    cuts = np.sort(rng.choice(np.arange(1, S), size=min(n_docs - 1, S - 1), replace=False)) if n_docs > 1 else []
    lengths = np.diff(np.concatenate([[0], cuts, [S]])).astype(int).tolist()
    seg, _ = segments_from_lengths(lengths, B)
    tg = rng.integers(0, V, size=(B, S)).astype(np.int32)
    tg[rng.random((B, S)) < ignore_frac] = -1
    return x, tg, seg
