/*
 * bwattn.h - blockwise exact causal attention with RoPE and a packing mask,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is the attention core of the Large World Model training
 * stack (arXiv 2402.08268, "World Model on Million-Length Video And Language
 * With Blockwise RingAttention"):
 *   - exact softmax attention computed blockwise (query blocks stream K/V
 *     blocks and merge partial results with an online-softmax running max and
 *     sum), as in the ring/blockwise attention fused with FlashAttention that
 *     the paper trains with (zhao9797 page "LWM (Large World Model)", section
 *     模型架构; elamur.ai summary page, Summary: no approximation);
 *   - causal masking of a decoder-only autoregressive model (zhao9797 page,
 *     模型架构);
 *   - the masked-sequence-packing mask: tokens of one packed example attend
 *     only to tokens of the same example (zhao9797 page, 训练方法, "Masked
 *     Sequence Packing");
 *   - standard RoPE with a context-scaled base theta, 1e6 at 32K up to 5e7 at
 *     1M (zhao9797 page, 模型架构 and the Stage I table of 训练方法).
 * The cross-device K/V ring of the paper becomes an in-HBM loop over K/V
 * blocks on one GPU (kv_chunk below gives the ring's visiting order).
 *
 * Conventions for every entry point
 *   - Tensors are device pointers.  q, k, v, o, dO, dq, dk, dv are bf16
 *     [B,H,S,D] contiguous (D innermost).  segment_ids and positions are int32
 *     [B,S].  lse is fp32 [B,H,S].  All pointers must be 16-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The library never allocates, frees or synchronizes, and keeps
 *     no pointer after returning.  The caller owns every buffer, including the
 *     workspace sized by attn_workspace_bytes, and keeps them alive until the
 *     stream work has finished.  Entry points keep no state (apart from the
 *     thread-local measurement request of attn_profile_events, and the static
 *     workspace of attn_decode_noalloc, below) and are thread-safe (calls of
 *     attn_decode_noalloc that overlap on one GPU excepted).
 *   - Every argument is checked before any HIP call.  The return value is an
 *     attn_status; no exception crosses the ABI and the library never aborts.
 *     Device-side values (segment ids, positions) are not checked: any int32
 *     values are legal.  Faults inside kernels surface at the next stream
 *     synchronisation, as for any HIP kernel.
 *
 * Reading of the pages where they are silent (softmax scale, RoPE pairing,
 * positions under packing) is stated at each field.
 */
#ifndef BWATTN_H
#define BWATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null required pointer, bad size, misalignment, overflow, struct_size */
  ATTN_ERR_UNSUPPORTED = 2, /* head_dim not compiled, or the device is not gfx950 */
  ATTN_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than attn_workspace_bytes */
  ATTN_ERR_HIP = 4          /* a HIP launch or query failed */
} attn_status;

typedef struct {
  int32_t struct_size;   /* must equal sizeof(attn_params): guards against ABI drift          */
  int32_t batch;         /* B >= 1                                                           */
  int32_t heads;         /* H >= 1                                                           */
  int32_t seqlen;        /* S >= 1                                                           */
  int32_t head_dim;      /* D, 64 or 128                                                     */
  float softmax_scale;   /* <= 0 selects 1/sqrt(D) (the pages give no scale)                 */
  int32_t causal;        /* 1: key j visible to query i only if j <= i (sequence index)      */
                         /* 0: no causal term (the packing mask still applies)               */
  double rope_theta;     /* RoPE base; <= 0 disables RoPE (q, k used as given).  Pairs       */
                         /* (x[2i], x[2i+1]) rotate by pos * theta^(-2i/D), angle in fp64.   */
  int32_t kv_chunk;      /* 0: K/V blocks visited in natural order.  > 0: ring order: the    */
                         /* sequence is cut in chunks of kv_chunk keys (a multiple of 64);   */
                         /* queries of chunk r visit chunk r, r-1, ..., 0, C-1, ..., r+1.    */
                         /* (attn_bwd walks tiles of 128 rows or keys: its chunks are        */
                         /* rounded down to whole tiles; the result is the same sum.)        */
  int32_t deterministic; /* must be 0 or 1.  attn_bwd is bitwise reproducible either way:    */
                         /* no path uses float atomics, so both values run the same kernels  */
} attn_params;

/* Name of a status code (static string). */
const char* attn_status_string(int status);

/* Message of the last error returned on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Bytes of device workspace that attn_fwd (which = 0), attn_bwd (1),
 * attn_fwd_f32 (2) or attn_bwd_f32 (3) needs for these parameters; 0 if the
 * parameters are invalid.  rope_apply and rope_apply_f32 need none. */
size_t attn_workspace_bytes(const attn_params* p, int32_t which);

/* RoPE on x (bf16 [B,H,S,D]) into y (same shape; y may equal x): each pair
 * (x[2i], x[2i+1]) of a row at position pos rotates by a = pos * theta^(-2i/D)
 * (inverse != 0: by -a, the transpose of the rotation).  positions NULL means
 * pos = s.  The angle is formed and reduced in fp64; the rotation is done in
 * fp32 and rounded to bf16 (round to nearest even).  Uses p->batch, heads,
 * seqlen, head_dim and rope_theta (which must be > 0).  RoPE as "standard
 * RoPE" with scaled theta: zhao9797 page, 模型架构. */
int rope_apply(const attn_params* p, const void* x, void* y, const int32_t* positions, int32_t inverse,
               void* stream);

/* Forward: o = softmax(scale * q' k'^T + mask) v and lse (natural log) per
 * query row, where q' and k' are q and k after RoPE at `positions`, and the
 * mask allows key j for query i iff segment_ids[j] == segment_ids[i] and
 * (if causal) j <= i.  q and k are passed un-rotated.  segment_ids NULL: one
 * segment per batch row; positions NULL: pos = s.  Exact attention computed
 * blockwise with an online softmax (zhao9797 page, 模型架构; packing mask:
 * 训练方法).  o: bf16 [B,H,S,D]; lse: fp32 [B,H,S], kept for attn_bwd.
 * workspace: attn_workspace_bytes(p, 0) bytes of device memory. */
int attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, const int32_t* segment_ids,
             const int32_t* positions, void* o, float* lse, void* workspace, size_t workspace_bytes,
             void* stream);

/* Backward of attn_fwd: given o and lse from attn_fwd on the same inputs and
 * the output gradient d_o, writes dq, dk, dv (bf16 [B,H,S,D]), the gradients
 * with respect to the un-rotated q and k and to v (the RoPE backward is
 * included).  The attention probabilities are recomputed from lse, so memory
 * stays linear in S.  workspace: attn_workspace_bytes(p, 1) bytes. */
int attn_bwd(const attn_params* p, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* d_o, const int32_t* segment_ids, const int32_t* positions,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* fp32 variant.  The paper trains and runs its models in full precision      */
/* (arXiv 2402.08268, training and inference setup); these entry points take  */
/* the same operation on fp32 tensors and compute it with fp32 matrix         */
/* instructions (fp32 products and sums; exp2 and the RoPE sine and cosine by */
/* the hardware's fp32 approximations).  Conventions as above, with every     */
/* bf16 tensor replaced by fp32 [B,H,S,D] contiguous; lse stays fp32 [B,H,S]. */
/* ------------------------------------------------------------------------ */

/* rope_apply on fp32 rows (fp32 rotation, fp64 angle). */
int rope_apply_f32(const attn_params* p, const float* x, float* y, const int32_t* positions, int32_t inverse,
                   void* stream);

/* attn_fwd on fp32 q, k, v; o fp32 [B,H,S,D].  workspace:
 * attn_workspace_bytes(p, 2) bytes. */
int attn_fwd_f32(const attn_params* p, const float* q, const float* k, const float* v, const int32_t* segment_ids,
                 const int32_t* positions, float* o, float* lse, void* workspace, size_t workspace_bytes,
                 void* stream);

/* attn_bwd on fp32 tensors: o and lse from attn_fwd_f32 on the same inputs,
 * d_o fp32; writes fp32 dq, dk, dv.  workspace: attn_workspace_bytes(p, 3)
 * bytes. */
int attn_bwd_f32(const attn_params* p, const float* q, const float* k, const float* v, const float* o,
                 const float* lse, const float* d_o, const int32_t* segment_ids, const int32_t* positions, float* dq,
                 float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Decode attention against a long key/value cache: the n_q new query rows
 * of each (b, h) against the p->seqlen = S cached keys, as in 1M-token
 * inference with the same exact blockwise attention (zhao9797 page "LWM
 * (Large World Model)", 模型架构).  The keys are split into chunks (split-K);
 * each chunk keeps the online-softmax state (running max, running sum,
 * unnormalised output) of every row, and the chunks are merged with the same
 * rule.
 *   - q: bf16 [B,H,n_q,D], un-rotated.  Query row r is the token at sequence
 *     index S - n_q + r: the cache already holds its key and value.  With
 *     p->causal = 1 it sees keys j <= S - n_q + r, otherwise all S keys.
 *   - k_cache: bf16 [B,H,S,D] keys already rotated (rope_apply at their
 *     positions, done once when a key enters the cache); un-rotated when
 *     rope_theta <= 0.  v_cache: bf16 [B,H,S,D].
 *   - q_positions: int32 [B,n_q] RoPE positions of the query rows; NULL means
 *     S - n_q + r.
 *   - o: bf16 [B,H,n_q,D]; lse: fp32 [B,H,n_q] (natural log).
 *   - 1 <= n_q <= 32; segment masks are not taken (one document per row);
 *     p->kv_chunk and p->deterministic are ignored.  The result does not
 *     depend on the split.
 * workspace: attn_decode_workspace_bytes(p, n_q) bytes of device memory. */
int attn_decode(const attn_params* p, int32_t n_q, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* q_positions, void* o, float* lse, void* workspace, size_t workspace_bytes,
                void* stream);

/* Bytes of device workspace attn_decode needs for these parameters and n_q;
 * 0 if they are invalid. */
size_t attn_decode_workspace_bytes(const attn_params* p, int32_t n_q);

/* attn_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, token-by-token serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results as attn_decode (the same kernels,
 * so the same bits), minus the workspace: the call uses a static device
 * array of attn_decode_noalloc_max_bytes() bytes (64 MiB) that the library
 * holds on every GPU it runs on until the process ends.  It allocates and
 * frees nothing.
 *   - Parameters whose attn_decode_workspace_bytes(p, n_q) exceeds that size
 *     are refused with ATTN_ERR_WORKSPACE before any HIP call (at n_q = 32
 *     and D = 128 every batch x heads up to 2048 fits).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other host threads) race and give
 *     wrong results; calls ordered on one stream do not.  Nothing in the
 *     array needs to start at zero: a call writes every byte it reads.
 *   - The array's device address is looked up once per device, on the
 *     first call with that device current. */
int attn_decode_noalloc(const attn_params* p, int32_t n_q, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* q_positions, void* o, float* lse, void* stream);

/* Size in bytes of the static workspace of attn_decode_noalloc. */
size_t attn_decode_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------ */
/* Loss side of masked sequence packing.  Short examples packed into one row  */
/* attend only to themselves (the segment mask above) and their loss is       */
/* re-weighted so that packed training computes what training the same        */
/* examples unpacked, one per padded row, computes (zhao9797 page "LWM (Large */
/* World Model)", 数据 and 训练方法 with its ablation table).  The pages give  */
/* no formula; the objective taken is the unpacked one: each example's mean   */
/* cross-entropy over its loss tokens, averaged over the examples that have   */
/* loss tokens:  loss = sum_t ce_t / (E n_e(t)).                               */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t struct_size;  /* must equal sizeof(packed_ce_params)                                 */
  int32_t batch;        /* B >= 1                                                             */
  int32_t seqlen;       /* S >= 1; token row t = b * S + s, N = B * S <= 2^31 - 1             */
  int32_t vocab;        /* V: a multiple of 8, 8 <= V <= 65536                                */
  int32_t num_segments; /* example ids of a batch row lie in [0, num_segments); >= 1          */
  float grad_scale;     /* dlogits = grad_scale * d loss / d logits                           */
} packed_ce_params;

/* Bytes of device workspace packed_ce_loss needs; 0 if the parameters are
 * invalid. */
size_t packed_ce_workspace_bytes(const packed_ce_params* p);

/* Re-weighted cross-entropy of packed token rows and its gradient.
 *   - logits: bf16 [N, V] (row t = b * S + s), 16-byte aligned.
 *   - targets: int32 [N], the target token of each row; a value outside
 *     [0, V) marks a row without loss (the last token of an example, prompt
 *     tokens, padding).
 *   - segment_ids: int32 [B, S] example ids (example = (b, id)); NULL means
 *     one example per batch row.  Rows whose id lies outside
 *     [0, num_segments) carry no loss.  Device values are not checked.
 *   - loss: one fp32 in device memory: sum over loss rows t of
 *     ce_t / (E n_e(t)), ce_t = logsumexp(logits[t]) - logits[t][y_t], E the
 *     number of examples with a loss row, n_e their loss rows; 0 if E = 0.
 *   - dlogits: bf16 [N, V] or NULL (loss only): grad_scale * (softmax(logits[t])
 *     - onehot(y_t)) / (E n_e(t)) for loss rows, zero rows elsewhere.
 *   - token_ce: fp32 [N] or NULL: ce_t of loss rows, 0 elsewhere.
 * The result does not depend on the order of work (bitwise reproducible).
 * workspace: packed_ce_workspace_bytes(p) bytes. */
int packed_ce_loss(const packed_ce_params* p, const void* logits, const int32_t* targets,
                   const int32_t* segment_ids, float* loss, void* dlogits, float* token_ce, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Measurement hook (for benchmarks and profilers; not needed to compute).    */
/* ------------------------------------------------------------------------ */
typedef enum {
  ATTN_KERNEL_ROPE = 0,      /* RoPE pre-pass (also used by rope_apply)               */
  ATTN_KERNEL_FWD = 1,       /* forward main kernel                                   */
  ATTN_KERNEL_BWD_DQ = 2,    /* backward: dQ and Delta                                */
  ATTN_KERNEL_BWD_DKDV = 3,  /* backward: dK and dV                                   */
  ATTN_KERNEL_DECODE = 4,    /* decode: per-chunk partial states (split-K)            */
  ATTN_KERNEL_DECODE_MERGE = 5, /* decode: merge of the chunk states                  */
  ATTN_KERNEL_FWD_F32 = 6,   /* fp32 forward main kernel                              */
  ATTN_KERNEL_BWD_DQ_F32 = 7,   /* fp32 backward: dQ and Delta                        */
  ATTN_KERNEL_BWD_DKDV_F32 = 8, /* fp32 backward: dK and dV                           */
  ATTN_KERNEL_PACKED_CE = 9, /* packed cross-entropy: the per-row loss and gradient kernel */
  ATTN_KERNEL_COUNT = 10
} attn_kernel_id;

/* Ask the library to bracket the next n launches of kernel `kernel` made by
 * the calling thread with hipEventRecord(start[i], s) and
 * hipEventRecord(stop[i], s), where s is the stream of the launch and i counts
 * those launches from 0.  start and stop are arrays of n hipEvent_t created by
 * the caller, which keeps them valid until the recorded work has finished.
 * Launches after the n-th record nothing; n = 0 clears the request.  The
 * request is thread-local and changes no result.  Returns ATTN_OK or
 * ATTN_ERR_INVALID_ARG (kernel out of range, n < 0, null arrays with n > 0). */
int attn_profile_events(int32_t kernel, void* const* start, void* const* stop, int32_t n);

/* Number of launches of `kernel` bracketed so far under the current request
 * of the calling thread (-1 if kernel is out of range). */
int32_t attn_profile_count(int32_t kernel);

#ifdef __cplusplus
}
#endif

#endif /* BWATTN_H */
