// Kernel argument blocks and launchers of the library (host and device).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bwattn {

// Tile sizes shared by the host schedule and the kernels.
constexpr int kFwdBlockQ = 256;   // query rows per forward / dQ workgroup (8 waves x 32 rows)
constexpr int kFwdBlockK = 64;    // keys per K/V tile streamed by the forward / dQ kernels
constexpr int kBwdBlockK = 256;   // keys per dK/dV workgroup (8 waves x 32 keys)
constexpr int kBwdBlockQ = 128;   // query rows per Q/dO tile streamed by the bf16 dK/dV kernel
constexpr int kF32BwdBlockQ = 64;  // query rows per Q/dO tile streamed by the fp32 dK/dV kernel
constexpr int kSegBlock = 32;     // rows per segment-range block

struct RopeArgs {
  const uint16_t* x;
  uint16_t* y;
  const int32_t* pos;  // [B,S] or null (pos = pos_base + s)
  int pos_base;
  int B, H, S, D;
  int inverse;
  float out_scale;   // y = (R x) * out_scale, rounded once to bf16
  int stream;        // nonzero: the streaming variant for tensors of 512 MiB and more
  double turns[64];  // theta^(-2i/D) / (2 pi), i < D/2
};

// Range tables: per own tile, [lo, hi) over the other side's tiles.  Bit 30
// of lo is set when some tile inside the range cannot hold a visible pair
// (segment ids that are not contiguous), so a walk over it must test each
// tile; for contiguous segments every tile in [lo, hi) is useful.
constexpr int kRangeSparse = 1 << 30;

struct TileRangeArgs {
  const int2* blk;  // [B, nblk] segment ranges or null (no packing mask)
  int2* out;        // [B, n_own] -> [lo | sparse flag, hi) over the other side's tiles
  int B, S, nblk;
  int own_rows, other_rows, n_own, n_other;
  int causal, own_is_query;
};

// Forward and dQ kernels: a workgroup owns kFwdBlockQ query rows of one (b,h)
// and streams K/V tiles of kFwdBlockK keys.
struct FwdArgs {
  const uint16_t* q;  // queries [B,H,S,D] as given (rotated and scaled on load)
  const uint16_t* k;  // rotated keys
  const uint16_t* v;
  uint16_t* o;
  float* lse;          // natural log, [B,H,S]
  const int32_t* seg;  // [B,S] or null
  const int2* blk;     // segment ranges per 32 rows, or null
  const int2* t64;     // segment ranges per 64-row tile, [B, n64p], or null
  const int2* qrange;  // [B, n_qtiles] K/V tile range, or null
  int B, H, S;
  int n_qtiles, n_ktiles, nblk, n64p;
  int causal;
  int chunk_tiles;     // ring chunk in K/V tiles; 0 = natural order
  const int32_t* pos;  // [B,S] or null (pos = s), for the query rows' RoPE
  float q_scale;       // softmax scale * log2(e), folded into the query rows
  double turns[64];    // theta^(-2i/D) / (2 pi); all zero without RoPE
};

struct BwdArgs {
  const uint16_t* q;   // rotated queries times scale * log2(e), as in the forward
  const uint16_t* k;   // rotated keys
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;    // natural log
  float* ndelta;       // [B,H,S] workspace written by the dQ kernel: -<dO_i, O_i>
  float* nlse2;        // [B,H,S] workspace written by the dQ kernel: -LSE_i log2(e)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* seg;
  const int32_t* pos;  // [B,S] or null, for the RoPE backward
  const int2* blk;
  const int2* t64;      // segment ranges per 64-row tile, [B, n64p], or null
  const int2* qrange;   // per query tile (dQ kernel): K/V tile range
  const int2* krange;   // per key tile (dK/dV kernel): query tile range
  int B, H, S;
  int n_qtiles, n_ktiles, nblk, n64p;
  int n_bkv, n_bq;     // dK/dV kernel: key tiles of kBwdBlockK and query tiles of kBwdBlockQ
  float scale;         // softmax scale
  float dk_scale;      // scale / (scale log2 e): dK' from the scaled query rows
  int causal;
  int chunk_tiles;
  int rope;            // apply the RoPE backward
  double turns[64];
};

// Decode (split-K): one wave per chunk of `chunk` keys of one (b,h) keeps
// the online-softmax state of n_q <= 32 query rows; a second kernel merges
// the chunks.
constexpr int kDecodeTile = 32;     // keys per decode tile
constexpr int kDecodeMaxRows = 32;  // query rows per (b,h) in one decode call
constexpr int kDecodeMaxChunk = 1 << 20;  // keys per chunk at most

struct DecodeArgs {
  const uint16_t* q;  // rotated query rows times scale * log2(e) [B,H,n_q,D]
  const uint16_t* k;  // key cache [B,H,S,D] (rotated by the caller)
  const uint16_t* v;  // value cache [B,H,S,D]
  float* part_o;      // [B,H,n_chunks,n_q,D] unnormalised partial outputs
  float* part_ml;     // [B,H,n_chunks,n_q,2] (m in log2 units of the scaled scores, l)
  uint16_t* o;        // [B,H,n_q,D]
  float* lse;         // [B,H,n_q], natural log
  int B, H, S, n_q;
  int n_chunks, chunk;  // chunk: keys per chunk, a multiple of kDecodeTile
  int causal;
};

// fp32 variant: the same operation on fp32 tensors with fp32 MFMAs
// (v_mfma_f32_32x32x2_f32).  The forward keeps two waves per SIMD; the dQ and
// dK/dV kernels hold two stationary 32-row operands plus an accumulator per
// wave and run one wave per SIMD with the whole register file.
constexpr int kF32FwdBlockQ = 256;  // query rows per forward workgroup (8 waves x 32 rows)
constexpr int kF32DqBlockQ = 128;   // query rows per dQ workgroup (4 waves x 32 rows)
constexpr int kF32BwdBlockK = 128;  // keys per dK/dV workgroup (4 waves x 32 keys)
// streamed tiles: kFwdBlockK keys (forward, dQ) or kBwdBlockQ query rows (dK/dV)

struct F32Args {
  const float* q;      // rotated queries [B,H,S,D]
  const float* k;      // rotated keys
  const float* v;
  const float* o;      // backward: forward output
  const float* dout;   // backward: output gradient
  const float* lse;    // backward: natural-log LSE from the forward
  float* out_o;        // forward outputs
  float* out_lse;
  float* ndelta;       // [B,H,S] written by the dQ kernel: -<dO_i, O_i>
  float* nlse2;        // [B,H,S] written by the dQ kernel: -LSE_i log2(e)
  float* dq;
  float* dk;
  float* dv;
  const int32_t* seg;  // [B,S] or null
  const int32_t* pos;  // [B,S] or null, for the RoPE backward
  const int2* blk;     // segment ranges per 32 rows, or null
  const int2* range;   // per own tile of the launched kernel: [lo, hi) of streamed tiles, or null
  int B, H, S;
  int n_own, n_other, nblk;  // tiles of the launched kernel's own side and of the streamed side
  float scale, scale_log2;
  int causal;
  int chunk_tiles;     // ring chunk in streamed tiles; 0 = natural order
  int rope;            // apply the RoPE backward
  double turns[64];
};

// Re-weighted cross-entropy of packed token rows (loss side of masked
// sequence packing): token row t = b * S + s of bf16 logits [N, V].
struct CeArgs {
  const uint16_t* logits;  // bf16 [N, V]
  const int32_t* targets;  // [N]; outside [0, V): row without loss
  const int32_t* seg;      // [B, S] example ids, or null (one example per batch row)
  uint16_t* dlogits;       // bf16 [N, V] or null
  float* token_ce;         // [N] or null
  float* loss;             // one float
  int* counts;             // workspace [B * num_segments]: loss rows per example
  float* weights;          // workspace [B * num_segments]: 1 / (E n_e)
  float* wloss;            // workspace [N]: w_t ce_t
  int B, S, V, num_segments;
  float grad_scale;
};
constexpr int kCeThreads = 512;     // threads per row workgroup (8 waves)
constexpr int kCeMaxVocab = 65536;  // 512 threads x 16 chunks x 8 logits held in registers
// 16-byte chunks per thread of the row kernel (one of its compiled sizes),
// -1 if V is too large
inline int ce_chunks_per_thread(int V) {
  const int need = ((V >> 3) + kCeThreads - 1) / kCeThreads;
  const int opts[] = {2, 4, 6, 8, 10, 12, 16};
  for (int o : opts)
    if (need <= o) return o;
  return -1;
}

hipError_t launch_packed_ce_prologue(const CeArgs& a, hipStream_t st);
hipError_t launch_packed_ce_rows(const CeArgs& a, hipStream_t st);
hipError_t launch_packed_ce_sum(const CeArgs& a, hipStream_t st);
hipError_t launch_rope(const RopeArgs& a, hipStream_t st);
hipError_t launch_rope_f32(const RopeArgs& a, const float* x, float* y, hipStream_t st);
hipError_t launch_attn_fwd_f32(const F32Args& a, int D, hipStream_t st);
hipError_t launch_attn_bwd_dq_f32(const F32Args& a, int D, hipStream_t st);
hipError_t launch_attn_bwd_dkdv_f32(const F32Args& a, int D, hipStream_t st);
hipError_t launch_block_ranges(const int32_t* seg, int B, int S, int nblk, int2* out, hipStream_t st);
// Row pitch of the per-64-row tile range table: n64 = ceil(S / 64) entries
// and at least one more, an even count (16-byte aligned rows), the entries
// past the last tile repeating it, so a pair of entries can be read at once.
inline int tile64_pitch(int S) { return (((S + 63) / 64) + 2) & ~1; }
hipError_t launch_tile64_ranges(const int2* blk, int B, int S, int nblk, int n64p, int2* out, hipStream_t st);
hipError_t launch_tile_ranges(const TileRangeArgs& a, hipStream_t st);
hipError_t launch_attn_fwd(const FwdArgs& a, int D, hipStream_t st);
hipError_t launch_attn_bwd_dq(const BwdArgs& a, int D, hipStream_t st);
hipError_t launch_attn_bwd_dkdv(const BwdArgs& a, int D, hipStream_t st);
hipError_t launch_attn_decode_partial(const DecodeArgs& a, int D, hipStream_t st);
hipError_t launch_attn_decode_combine(const DecodeArgs& a, int D, hipStream_t st);

// Bytes of the file-scope device array that attn_decode_noalloc uses as its
// workspace (one copy per GPU, alive until the process ends).
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
// Device address of that array on the current device, looked up once per
// device (hipGetSymbolAddress) and cached.
hipError_t decode_scratch(void** ptr);

}  // namespace bwattn
