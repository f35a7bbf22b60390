// C-ABI entry points: argument checks (before any HIP call), workspace plan,
// and the launch sequence of each operation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "bwattn.h"
#include "kernels.hpp"

using namespace bwattn;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

// Measurement hook state (thread-local): events to record around launches.
struct ProfileSlot {
  void* const* start = nullptr;
  void* const* stop = nullptr;
  int32_t n = 0, used = 0;
};
thread_local ProfileSlot g_prof[ATTN_KERNEL_COUNT];

// Launch wrapper: records the requested events around one kernel launch.
template <typename F>
hipError_t timed_launch(int kernel, hipStream_t st, F&& launch) {
  ProfileSlot& ps = g_prof[kernel];
  bool rec = ps.used < ps.n;
  if (rec) {
    hipError_t e = hipEventRecord((hipEvent_t)ps.start[ps.used], st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (rec) {
    e = hipEventRecord((hipEvent_t)ps.stop[ps.used], st);
    if (e != hipSuccess) return e;
    ++ps.used;
  }
  return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxSeq = int64_t(1) << 24;  // per-head offsets stay below 2^32 bytes

int check_params(const attn_params* p) {
  if (p == nullptr) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size != (int32_t)sizeof(attn_params))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %d != sizeof(attn_params) %d", p->struct_size,
                (int)sizeof(attn_params));
  if (p->batch < 1 || p->heads < 1 || p->seqlen < 1 || p->head_dim < 1)
    return fail(ATTN_ERR_INVALID_ARG, "batch, heads, seqlen and head_dim must be >= 1 (got %d, %d, %d, %d)",
                p->batch, p->heads, p->seqlen, p->head_dim);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  if ((int64_t)p->seqlen > kMaxSeq) return fail(ATTN_ERR_INVALID_ARG, "seqlen %d above %lld", p->seqlen, (long long)kMaxSeq);
  int64_t bh = (int64_t)p->batch * p->heads;
  if (bh > (int64_t)1 << 20) return fail(ATTN_ERR_INVALID_ARG, "batch*heads %lld too large", (long long)bh);
  int64_t elems = bh * p->seqlen * p->head_dim;
  if (elems > ((int64_t)1 << 40)) return fail(ATTN_ERR_INVALID_ARG, "tensor of %lld elements too large", (long long)elems);
  int64_t tiles = bh * ((p->seqlen + kFwdBlockQ - 1) / kFwdBlockQ);
  if (tiles > ((int64_t)1 << 31) - 1) return fail(ATTN_ERR_INVALID_ARG, "too many tiles");
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->deterministic != 0 && p->deterministic != 1) return fail(ATTN_ERR_INVALID_ARG, "deterministic must be 0 or 1");
  if (!(std::isfinite(p->softmax_scale))) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (std::isnan(p->rope_theta) || std::isinf(p->rope_theta))
    return fail(ATTN_ERR_INVALID_ARG, "rope_theta is not finite");
  if (p->kv_chunk < 0 || p->kv_chunk % kFwdBlockK != 0)
    return fail(ATTN_ERR_INVALID_ARG, "kv_chunk %d must be 0 or a positive multiple of %d", p->kv_chunk, kFwdBlockK);
  return ATTN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int B, H, S, D;
  bool rope, f32;
  int bq, bkv;  // own rows of the query-stationary and of the key-stationary kernel
  int nblk, n64p, n_qtiles, n_ktiles, n_bkv, n_bq;
  size_t off_qr, off_kr, off_delta, off_blk, off_t64, off_qrange, off_krange, total;
};

// Workspace layout of the forward (which = 0) or backward (which = 1) of the
// bf16 or the fp32 path.  The segment-dependent parts are always reserved so
// that the size depends only on the parameters.
Plan make_plan(const attn_params* p, int which, bool f32) {
  Plan pl{};
  pl.B = p->batch;
  pl.H = p->heads;
  pl.S = p->seqlen;
  pl.D = p->head_dim;
  pl.rope = p->rope_theta > 0.0;
  pl.f32 = f32;
  pl.bq = f32 ? (which == 0 ? kF32FwdBlockQ : kF32DqBlockQ) : kFwdBlockQ;
  pl.bkv = f32 ? kF32BwdBlockK : kBwdBlockK;
  pl.nblk = (pl.S + kSegBlock - 1) / kSegBlock;
  pl.n64p = tile64_pitch(pl.S);
  pl.n_qtiles = (pl.S + pl.bq - 1) / pl.bq;
  pl.n_ktiles = (pl.S + kFwdBlockK - 1) / kFwdBlockK;
  pl.n_bkv = (pl.S + pl.bkv - 1) / pl.bkv;
  const int bqo = f32 ? kF32BwdBlockQ : kBwdBlockQ;
  pl.n_bq = (pl.S + bqo - 1) / bqo;
  const size_t esize = f32 ? 4 : 2;
  size_t n = (size_t)pl.B * pl.H * pl.S * pl.D;
  size_t off = 0;
  // rotated rows; the bf16 backward always keeps its query rows here, rotated
  // or not, times scale * log2(e) (the bf16 forward forms them as it loads)
  if (f32 ? pl.rope : which == 1) {
    pl.off_qr = off;
    off += align256(n * esize);
  }
  if (pl.rope) {
    pl.off_kr = off;
    off += align256(n * esize);
  }
  if (which == 1) {
    pl.off_delta = off;  // -Delta, then -LSE log2(e)
    off += 2 * align256((size_t)pl.B * pl.H * pl.S * 4);
  }
  pl.off_blk = off;
  off += align256((size_t)pl.B * pl.nblk * sizeof(int2));
  pl.off_t64 = off;
  off += align256((size_t)pl.B * pl.n64p * sizeof(int2));
  pl.off_qrange = off;
  off += align256((size_t)pl.B * pl.n_qtiles * sizeof(int2));
  if (which == 1) {
    pl.off_krange = off;
    off += align256((size_t)pl.B * pl.n_bkv * sizeof(int2));
  }
  pl.total = off;
  return pl;
}

// Device check, cached per device: the kernels are built for gfx950 only.
int check_device() {
  static std::mutex mu;
  static int state[64];  // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(ATTN_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDeviceProperties failed");
    state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  if (state[dev] != 1) return fail(ATTN_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return ATTN_OK;
}

void fill_turns(double* turns, int D, double theta) {
  for (int i = 0; i < D / 2; ++i) turns[i] = std::pow(theta, -2.0 * i / D) / (2.0 * M_PI);
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

float scale_of(const attn_params* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : (float)(1.0 / std::sqrt((double)p->head_dim));
}

float scale_log2_of(const attn_params* p) { return scale_of(p) * 1.4426950408889634f; }

// RoPE of q and k into the workspace, and the segment schedule.  The bf16
// backward stores its query rows times scale * log2(e) (rotated or not), so
// the score MFMAs of its kernels leave scores in log2 units; the bf16 forward
// forms those rows itself and needs only the keys.
int prepare(const attn_params* p, const Plan& pl, const void* q, const void* k, const int32_t* seg,
            const int32_t* pos, char* ws, bool bwd, hipStream_t st) {
  const bool q_rows = pl.f32 ? pl.rope : bwd;  // query rows into the workspace
  if (q_rows || pl.rope) {
    RopeArgs r{};
    r.pos = pos;
    r.B = pl.B;
    r.H = pl.H;
    r.S = pl.S;
    r.D = pl.D;
    r.inverse = 0;
    if (pl.rope) fill_turns(r.turns, pl.D, p->rope_theta);  // else all zero: the identity rotation
    const void* src[2] = {q, k};
    const size_t dst[2] = {pl.off_qr, pl.off_kr};
    const float out_scale[2] = {scale_log2_of(p), 1.f};
    const char* what[2] = {"rope(q) launch", "rope(k) launch"};
    for (int i = q_rows ? 0 : 1; i < (pl.rope ? 2 : 1); ++i) {
      int rc = hip_status(timed_launch(ATTN_KERNEL_ROPE, st,
                                       [&] {
                                         if (pl.f32) return launch_rope_f32(r, (const float*)src[i], (float*)(ws + dst[i]), st);
                                         r.x = (const uint16_t*)src[i];
                                         r.y = (uint16_t*)(ws + dst[i]);
                                         r.out_scale = out_scale[i];
                                         return launch_rope(r, st);
                                       }),
                          what[i]);
      if (rc) return rc;
    }
  }
  if (seg) {
    int2* blk = (int2*)(ws + pl.off_blk);
    int rc = hip_status(launch_block_ranges(seg, pl.B, pl.S, pl.nblk, blk, st), "segment ranges launch");
    if (rc) return rc;
    rc = hip_status(launch_tile64_ranges(blk, pl.B, pl.S, pl.nblk, pl.n64p, (int2*)(ws + pl.off_t64), st),
                    "tile ranges (64 rows) launch");
    if (rc) return rc;
    TileRangeArgs t{};
    t.blk = blk;
    t.B = pl.B;
    t.S = pl.S;
    t.nblk = pl.nblk;
    t.causal = p->causal;
    // query tiles -> K/V tile ranges (forward and dQ)
    t.out = (int2*)(ws + pl.off_qrange);
    t.own_rows = pl.bq;
    t.other_rows = kFwdBlockK;
    t.n_own = pl.n_qtiles;
    t.n_other = pl.n_ktiles;
    t.own_is_query = 1;
    rc = hip_status(launch_tile_ranges(t, st), "tile ranges launch");
    if (rc) return rc;
    if (bwd) {
      // key tiles -> query tile ranges (dK/dV)
      t.out = (int2*)(ws + pl.off_krange);
      t.own_rows = pl.bkv;
      t.other_rows = pl.f32 ? kF32BwdBlockQ : kBwdBlockQ;
      t.n_own = pl.n_bkv;
      t.n_other = pl.n_bq;
      t.own_is_query = 0;
      rc = hip_status(launch_tile_ranges(t, st), "key tile ranges launch");
      if (rc) return rc;
    }
  }
  return ATTN_OK;
}

// Arguments shared by the fp32 kernels; the caller sets the per-kernel
// tile counts and range table.
F32Args f32_args(const attn_params* p, const Plan& pl, const void* q, const void* k, const void* v,
                 const int32_t* seg, const int32_t* pos, char* ws) {
  F32Args a{};
  a.q = pl.rope ? (const float*)(ws + pl.off_qr) : (const float*)q;
  a.k = pl.rope ? (const float*)(ws + pl.off_kr) : (const float*)k;
  a.v = (const float*)v;
  a.seg = seg;
  a.pos = pos;
  a.blk = seg ? (const int2*)(ws + pl.off_blk) : nullptr;
  a.B = pl.B;
  a.H = pl.H;
  a.S = pl.S;
  a.nblk = pl.nblk;
  a.scale = scale_of(p);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.causal = p->causal;
  a.chunk_tiles = p->kv_chunk / kFwdBlockK;
  a.rope = pl.rope ? 1 : 0;
  if (pl.rope) fill_turns(a.turns, pl.D, p->rope_theta);
  return a;
}

// Decode workspace: the query rows (rotated or not) times scale * log2(e),
// then the chunk states.  About 2048
// waves (8 per CU) keep enough K/V bytes in flight to cover HBM latency; a
// chunk is a multiple of kDecodeTile keys, at least 256 (unless the cache is
// shorter) and at most kDecodeMaxChunk.
struct DecodePlan {
  int n_chunks, chunk;
  size_t off_qr, off_po, off_ml, total;
};

DecodePlan make_decode_plan(const attn_params* p, int n_q) {
  DecodePlan d{};
  const int64_t bh = (int64_t)p->batch * p->heads;
  const int S = p->seqlen;
  int64_t want = std::max<int64_t>(1, (2048 + bh - 1) / bh);
  int64_t most = std::max(1, (S + 255) / 256);
  int64_t n = std::max(std::min(want, most), (int64_t)(S + kDecodeMaxChunk - 1) / kDecodeMaxChunk);
  int64_t chunk = (S + n - 1) / n;
  chunk = (chunk + kDecodeTile - 1) / kDecodeTile * kDecodeTile;
  d.chunk = (int)chunk;
  d.n_chunks = (int)((S + chunk - 1) / chunk);
  size_t off = 0;
  d.off_qr = off;
  off += align256((size_t)bh * n_q * p->head_dim * 2);
  d.off_po = off;
  off += align256((size_t)bh * d.n_chunks * n_q * p->head_dim * 4);
  d.off_ml = off;
  off += align256((size_t)bh * d.n_chunks * n_q * 2 * 4);
  d.total = off;
  return d;
}

// Packed cross-entropy: parameter checks and workspace layout.
struct CePlan {
  size_t off_counts, off_weights, off_wloss, total;
};

int check_ce_params(const packed_ce_params* p) {
  if (p == nullptr) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size != (int32_t)sizeof(packed_ce_params))
    return fail(ATTN_ERR_INVALID_ARG, "struct_size %d != sizeof(packed_ce_params) %d", p->struct_size,
                (int)sizeof(packed_ce_params));
  if (p->batch < 1 || p->seqlen < 1) return fail(ATTN_ERR_INVALID_ARG, "batch and seqlen must be >= 1");
  if ((int64_t)p->batch * p->seqlen > ((int64_t)1 << 31) - 1)
    return fail(ATTN_ERR_INVALID_ARG, "batch*seqlen above 2^31 - 1");
  if (p->vocab < 8 || p->vocab % 8 != 0)
    return fail(ATTN_ERR_INVALID_ARG, "vocab %d must be a positive multiple of 8", p->vocab);
  if (ce_chunks_per_thread(p->vocab) < 0)
    return fail(ATTN_ERR_UNSUPPORTED, "vocab %d above %d", p->vocab, kCeMaxVocab);
  if (p->num_segments < 1) return fail(ATTN_ERR_INVALID_ARG, "num_segments must be >= 1");
  if ((int64_t)p->batch * p->num_segments > ((int64_t)1 << 26))
    return fail(ATTN_ERR_INVALID_ARG, "batch*num_segments above 2^26");
  if (!std::isfinite(p->grad_scale)) return fail(ATTN_ERR_INVALID_ARG, "grad_scale is not finite");
  return ATTN_OK;
}

CePlan make_ce_plan(const packed_ce_params* p) {
  CePlan c{};
  const size_t ne = (size_t)p->batch * p->num_segments, n = (size_t)p->batch * p->seqlen;
  size_t off = 0;
  c.off_counts = off;
  off += align256(ne * 4);
  c.off_weights = off;
  off += align256(ne * 4);
  c.off_wloss = off;
  off += align256(n * 4);
  c.total = off;
  return c;
}

int check_decode_rows(int32_t n_q, int S) {
  if (n_q < 1 || n_q > kDecodeMaxRows)
    return fail(ATTN_ERR_INVALID_ARG, "n_q %d must be in [1, %d]", n_q, kDecodeMaxRows);
  if (n_q > S) return fail(ATTN_ERR_INVALID_ARG, "n_q %d larger than the cache length %d", n_q, S);
  return ATTN_OK;
}

// Argument checks of the decode entry points (the workspace aside).
int check_decode_args(const attn_params* p, int32_t n_q, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* q_positions, const void* o, const float* lse) {
  int rc = check_params(p);
  if (rc) return rc;
  rc = check_decode_rows(n_q, p->seqlen);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !o || !lse)
    return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, o and lse must not be NULL");
  const void* ptrs[] = {q, k_cache, v_cache, q_positions, o, lse};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  return ATTN_OK;
}

// The decode launch sequence on a workspace laid out by `dp`: every byte the
// merge reads is written earlier in the same sequence (the query rows by the
// RoPE pre-pass, the state of every chunk and row by the partial kernel), so
// the workspace needs no clearing.
int run_decode(const attn_params* p, const DecodePlan& dp, int32_t n_q, const void* q, const void* k_cache,
               const void* v_cache, const int32_t* q_positions, void* o, float* lse, char* ws, hipStream_t st) {
  {
    // query rows times scale * log2(e), as the forward takes them
    RopeArgs r{};
    r.x = (const uint16_t*)q;
    r.y = (uint16_t*)(ws + dp.off_qr);
    r.pos = q_positions;
    r.pos_base = p->seqlen - n_q;
    r.B = p->batch;
    r.H = p->heads;
    r.S = n_q;
    r.D = p->head_dim;
    r.inverse = 0;
    r.out_scale = scale_log2_of(p);
    if (p->rope_theta > 0.0) fill_turns(r.turns, p->head_dim, p->rope_theta);  // else the identity rotation
    int rc = hip_status(timed_launch(ATTN_KERNEL_ROPE, st, [&] { return launch_rope(r, st); }), "rope(q) launch");
    if (rc) return rc;
  }
  DecodeArgs a{};
  a.q = (const uint16_t*)(ws + dp.off_qr);
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.part_o = (float*)(ws + dp.off_po);
  a.part_ml = (float*)(ws + dp.off_ml);
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.B = p->batch;
  a.H = p->heads;
  a.S = p->seqlen;
  a.n_q = n_q;
  a.n_chunks = dp.n_chunks;
  a.chunk = dp.chunk;
  a.causal = p->causal;
  int rc = hip_status(
      timed_launch(ATTN_KERNEL_DECODE, st, [&] { return launch_attn_decode_partial(a, p->head_dim, st); }),
      "attn_decode partial launch");
  if (rc) return rc;
  rc = hip_status(
      timed_launch(ATTN_KERNEL_DECODE_MERGE, st, [&] { return launch_attn_decode_combine(a, p->head_dim, st); }),
      "attn_decode merge launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

const char* attn_last_error(void) { return g_err; }

size_t attn_workspace_bytes(const attn_params* p, int32_t which) {
  if (check_params(p) != ATTN_OK) return 0;
  if (which < 0 || which > 3) {
    fail(ATTN_ERR_INVALID_ARG, "which must be 0 (attn_fwd), 1 (attn_bwd), 2 (attn_fwd_f32) or 3 (attn_bwd_f32)");
    return 0;
  }
  g_err[0] = 0;
  return make_plan(p, which & 1, which >= 2).total;
}

int rope_apply(const attn_params* p, const void* x, void* y, const int32_t* positions, int32_t inverse,
               void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!(p->rope_theta > 0.0)) return fail(ATTN_ERR_INVALID_ARG, "rope_apply needs rope_theta > 0");
  if (x == nullptr || y == nullptr) return fail(ATTN_ERR_INVALID_ARG, "x and y must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(positions))
    return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (inverse != 0 && inverse != 1) return fail(ATTN_ERR_INVALID_ARG, "inverse must be 0 or 1");
  rc = check_device();
  if (rc) return rc;
  RopeArgs r{};
  r.x = (const uint16_t*)x;
  r.y = (uint16_t*)y;
  r.pos = positions;
  r.B = p->batch;
  r.H = p->heads;
  r.S = p->seqlen;
  r.D = p->head_dim;
  r.inverse = inverse;
  r.out_scale = 1.f;
  fill_turns(r.turns, p->head_dim, p->rope_theta);
  hipStream_t st = (hipStream_t)stream;
  rc = hip_status(timed_launch(ATTN_KERNEL_ROPE, st, [&] { return launch_rope(r, st); }), "rope launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

int attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, const int32_t* segment_ids,
             const int32_t* positions, void* o, float* lse, void* workspace, size_t workspace_bytes,
             void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || !o || !lse) return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o and lse must not be NULL");
  const void* ptrs[] = {q, k, v, o, lse, segment_ids, positions, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  Plan pl = make_plan(p, 0, false);
  if (workspace == nullptr || workspace_bytes < pl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", pl.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  rc = prepare(p, pl, q, k, segment_ids, positions, ws, false, st);
  if (rc) return rc;
  FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = pl.rope ? (const uint16_t*)(ws + pl.off_kr) : (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.seg = segment_ids;
  a.blk = segment_ids ? (const int2*)(ws + pl.off_blk) : nullptr;
  a.t64 = segment_ids ? (const int2*)(ws + pl.off_t64) : nullptr;
  a.qrange = segment_ids ? (const int2*)(ws + pl.off_qrange) : nullptr;
  a.B = pl.B;
  a.H = pl.H;
  a.S = pl.S;
  a.n_qtiles = pl.n_qtiles;
  a.n_ktiles = pl.n_ktiles;
  a.nblk = pl.nblk;
  a.n64p = pl.n64p;
  a.causal = p->causal;
  a.chunk_tiles = p->kv_chunk / kFwdBlockK;
  a.pos = positions;
  a.q_scale = scale_log2_of(p);
  if (pl.rope) fill_turns(a.turns, pl.D, p->rope_theta);  // else all zero: the identity rotation
  rc = hip_status(timed_launch(ATTN_KERNEL_FWD, st, [&] { return launch_attn_fwd(a, pl.D, st); }), "attn_fwd launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

int attn_bwd(const attn_params* p, const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* d_o, const int32_t* segment_ids, const int32_t* positions, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv)
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o, lse, d_o, dq, dk and dv must not be NULL");
  const void* ptrs[] = {q, k, v, o, lse, d_o, segment_ids, positions, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  Plan pl = make_plan(p, 1, false);
  if (workspace == nullptr || workspace_bytes < pl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", pl.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  rc = prepare(p, pl, q, k, segment_ids, positions, ws, true, st);
  if (rc) return rc;
  BwdArgs a{};
  a.q = (const uint16_t*)(ws + pl.off_qr);
  a.k = pl.rope ? (const uint16_t*)(ws + pl.off_kr) : (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)d_o;
  a.lse = lse;
  a.ndelta = (float*)(ws + pl.off_delta);
  a.nlse2 = (float*)(ws + pl.off_delta + align256((size_t)pl.B * pl.H * pl.S * 4));
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.seg = segment_ids;
  a.pos = positions;
  a.blk = segment_ids ? (const int2*)(ws + pl.off_blk) : nullptr;
  a.t64 = segment_ids ? (const int2*)(ws + pl.off_t64) : nullptr;
  a.qrange = segment_ids ? (const int2*)(ws + pl.off_qrange) : nullptr;
  a.krange = segment_ids ? (const int2*)(ws + pl.off_krange) : nullptr;
  a.B = pl.B;
  a.H = pl.H;
  a.S = pl.S;
  a.n_qtiles = pl.n_qtiles;
  a.n_ktiles = pl.n_ktiles;
  a.nblk = pl.nblk;
  a.n64p = pl.n64p;
  a.n_bkv = pl.n_bkv;
  a.n_bq = pl.n_bq;
  a.scale = scale_of(p);
  a.dk_scale = (float)((double)a.scale / (double)scale_log2_of(p));
  a.causal = p->causal;
  a.chunk_tiles = p->kv_chunk / kFwdBlockK;
  a.rope = pl.rope ? 1 : 0;
  if (pl.rope) fill_turns(a.turns, pl.D, p->rope_theta);
  // dQ first: it also forms Delta = <dO, O> per row, which dK/dV reads
  rc = hip_status(timed_launch(ATTN_KERNEL_BWD_DQ, st, [&] { return launch_attn_bwd_dq(a, pl.D, st); }), "attn_bwd dq launch");
  if (rc) return rc;
  rc = hip_status(timed_launch(ATTN_KERNEL_BWD_DKDV, st, [&] { return launch_attn_bwd_dkdv(a, pl.D, st); }), "attn_bwd dkdv launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

int rope_apply_f32(const attn_params* p, const float* x, float* y, const int32_t* positions, int32_t inverse,
                   void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!(p->rope_theta > 0.0)) return fail(ATTN_ERR_INVALID_ARG, "rope_apply_f32 needs rope_theta > 0");
  if (x == nullptr || y == nullptr) return fail(ATTN_ERR_INVALID_ARG, "x and y must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(positions))
    return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (inverse != 0 && inverse != 1) return fail(ATTN_ERR_INVALID_ARG, "inverse must be 0 or 1");
  rc = check_device();
  if (rc) return rc;
  RopeArgs r{};
  r.pos = positions;
  r.B = p->batch;
  r.H = p->heads;
  r.S = p->seqlen;
  r.D = p->head_dim;
  r.inverse = inverse;
  fill_turns(r.turns, p->head_dim, p->rope_theta);
  hipStream_t st = (hipStream_t)stream;
  rc = hip_status(timed_launch(ATTN_KERNEL_ROPE, st, [&] { return launch_rope_f32(r, x, y, st); }), "rope launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

int attn_fwd_f32(const attn_params* p, const float* q, const float* k, const float* v, const int32_t* segment_ids,
                 const int32_t* positions, float* o, float* lse, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || !o || !lse) return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o and lse must not be NULL");
  const void* ptrs[] = {q, k, v, o, lse, segment_ids, positions, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  Plan pl = make_plan(p, 0, true);
  if (workspace == nullptr || workspace_bytes < pl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", pl.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  rc = prepare(p, pl, q, k, segment_ids, positions, ws, false, st);
  if (rc) return rc;
  F32Args a = f32_args(p, pl, q, k, v, segment_ids, positions, ws);
  a.out_o = o;
  a.out_lse = lse;
  a.range = segment_ids ? (const int2*)(ws + pl.off_qrange) : nullptr;
  a.n_own = pl.n_qtiles;
  a.n_other = pl.n_ktiles;
  rc = hip_status(timed_launch(ATTN_KERNEL_FWD_F32, st, [&] { return launch_attn_fwd_f32(a, pl.D, st); }),
                  "attn_fwd_f32 launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

int attn_bwd_f32(const attn_params* p, const float* q, const float* k, const float* v, const float* o,
                 const float* lse, const float* d_o, const int32_t* segment_ids, const int32_t* positions, float* dq,
                 float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv)
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o, lse, d_o, dq, dk and dv must not be NULL");
  const void* ptrs[] = {q, k, v, o, lse, d_o, segment_ids, positions, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  Plan pl = make_plan(p, 1, true);
  if (workspace == nullptr || workspace_bytes < pl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", pl.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  rc = prepare(p, pl, q, k, segment_ids, positions, ws, true, st);
  if (rc) return rc;
  F32Args a = f32_args(p, pl, q, k, v, segment_ids, positions, ws);
  a.o = o;
  a.dout = d_o;
  a.lse = lse;
  a.ndelta = (float*)(ws + pl.off_delta);
  a.nlse2 = (float*)(ws + pl.off_delta + align256((size_t)pl.B * pl.H * pl.S * 4));
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  // dQ first: it also forms Delta = <dO, O> per row, which dK/dV reads
  a.range = segment_ids ? (const int2*)(ws + pl.off_qrange) : nullptr;
  a.n_own = pl.n_qtiles;
  a.n_other = pl.n_ktiles;
  rc = hip_status(timed_launch(ATTN_KERNEL_BWD_DQ_F32, st, [&] { return launch_attn_bwd_dq_f32(a, pl.D, st); }),
                  "attn_bwd_f32 dq launch");
  if (rc) return rc;
  a.range = segment_ids ? (const int2*)(ws + pl.off_krange) : nullptr;
  a.n_own = pl.n_bkv;
  a.n_other = pl.n_bq;
  rc = hip_status(timed_launch(ATTN_KERNEL_BWD_DKDV_F32, st, [&] { return launch_attn_bwd_dkdv_f32(a, pl.D, st); }),
                  "attn_bwd_f32 dkdv launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

size_t attn_decode_workspace_bytes(const attn_params* p, int32_t n_q) {
  if (check_params(p) != ATTN_OK) return 0;
  if (check_decode_rows(n_q, p->seqlen) != ATTN_OK) return 0;
  g_err[0] = 0;
  return make_decode_plan(p, n_q).total;
}

int attn_decode(const attn_params* p, int32_t n_q, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* q_positions, void* o, float* lse, void* workspace, size_t workspace_bytes,
                void* stream) {
  int rc = check_decode_args(p, n_q, q, k_cache, v_cache, q_positions, o, lse);
  if (rc) return rc;
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  DecodePlan dp = make_decode_plan(p, n_q);
  if (workspace == nullptr || workspace_bytes < dp.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", dp.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  rc = check_device();
  if (rc) return rc;
  return run_decode(p, dp, n_q, q, k_cache, v_cache, q_positions, o, lse, (char*)workspace, (hipStream_t)stream);
}

int attn_decode_noalloc(const attn_params* p, int32_t n_q, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* q_positions, void* o, float* lse, void* stream) {
  int rc = check_decode_args(p, n_q, q, k_cache, v_cache, q_positions, o, lse);
  if (rc) return rc;
  DecodePlan dp = make_decode_plan(p, n_q);
  if (dp.total > kDecodeScratchBytes)
    return fail(ATTN_ERR_WORKSPACE,
                "attn_decode_noalloc: these parameters need %zu bytes of workspace, above its static %zu bytes; "
                "use attn_decode with a workspace", dp.total, kDecodeScratchBytes);
  rc = check_device();
  if (rc) return rc;
  void* ws = nullptr;
  rc = hip_status(decode_scratch(&ws), "attn_decode_noalloc scratch lookup");
  if (rc) return rc;
  return run_decode(p, dp, n_q, q, k_cache, v_cache, q_positions, o, lse, (char*)ws, (hipStream_t)stream);
}

size_t attn_decode_noalloc_max_bytes(void) { return kDecodeScratchBytes; }

size_t packed_ce_workspace_bytes(const packed_ce_params* p) {
  if (check_ce_params(p) != ATTN_OK) return 0;
  g_err[0] = 0;
  return make_ce_plan(p).total;
}

int packed_ce_loss(const packed_ce_params* p, const void* logits, const int32_t* targets,
                   const int32_t* segment_ids, float* loss, void* dlogits, float* token_ce, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc = check_ce_params(p);
  if (rc) return rc;
  if (!logits || !targets || !loss) return fail(ATTN_ERR_INVALID_ARG, "logits, targets and loss must not be NULL");
  const void* ptrs[] = {logits, dlogits, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "logits, dlogits and workspace must be 16-byte aligned");
  const void* ptrs4[] = {targets, segment_ids, loss, token_ce};
  for (const void* ptr : ptrs4)
    if (((uintptr_t)ptr & 3u) != 0) return fail(ATTN_ERR_INVALID_ARG, "targets, segment_ids, loss and token_ce must be 4-byte aligned");
  CePlan pl = make_ce_plan(p);
  if (workspace == nullptr || workspace_bytes < pl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", pl.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  CeArgs a{};
  a.logits = (const uint16_t*)logits;
  a.targets = targets;
  a.seg = segment_ids;
  a.dlogits = (uint16_t*)dlogits;
  a.token_ce = token_ce;
  a.loss = loss;
  a.counts = (int*)(ws + pl.off_counts);
  a.weights = (float*)(ws + pl.off_weights);
  a.wloss = (float*)(ws + pl.off_wloss);
  a.B = p->batch;
  a.S = p->seqlen;
  a.V = p->vocab;
  a.num_segments = p->num_segments;
  a.grad_scale = p->grad_scale;
  rc = hip_status(launch_packed_ce_prologue(a, st), "packed_ce counts launch");
  if (rc) return rc;
  rc = hip_status(timed_launch(ATTN_KERNEL_PACKED_CE, st, [&] { return launch_packed_ce_rows(a, st); }),
                  "packed_ce rows launch");
  if (rc) return rc;
  rc = hip_status(launch_packed_ce_sum(a, st), "packed_ce sum launch");
  if (rc) return rc;
  g_err[0] = 0;
  return ATTN_OK;
}

int attn_profile_events(int32_t kernel, void* const* start, void* const* stop, int32_t n) {
  if (kernel < 0 || kernel >= ATTN_KERNEL_COUNT) return fail(ATTN_ERR_INVALID_ARG, "kernel id %d out of range", kernel);
  if (n < 0) return fail(ATTN_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && (start == nullptr || stop == nullptr)) return fail(ATTN_ERR_INVALID_ARG, "event arrays must not be NULL");
  g_prof[kernel].start = n > 0 ? start : nullptr;
  g_prof[kernel].stop = n > 0 ? stop : nullptr;
  g_prof[kernel].n = n;
  g_prof[kernel].used = 0;
  g_err[0] = 0;
  return ATTN_OK;
}

int32_t attn_profile_count(int32_t kernel) {
  if (kernel < 0 || kernel >= ATTN_KERNEL_COUNT) return -1;
  return g_prof[kernel].used;
}

}  // extern "C"
