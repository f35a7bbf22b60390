// fp32 variant of blockwise exact attention: forward and backward on fp32
// tensors with fp32 MFMAs (gfx950 v_mfma_f32_32x32x2_f32, 32x32 output, k = 2).
//
// The paper trains and runs its million-token models in full precision
// (arXiv 2402.08268, training and inference setup); the method is the same
// exact blockwise attention with an online softmax as the bf16 kernels
// (zhao9797 page "LWM (Large World Model)", 模型架构), with the causal and the
// packing masks (训练方法, Masked Sequence Packing) and RoPE applied before.
//
// Operand layout.  A 32x32x2 MFMA takes one value of A and one of B per lane:
// lane l gives A[l % 32][k = l / 32] and B[k = l / 32][l % 32], and its result
// has lane l holding column l % 32, register r holding row
// kidx(r, l / 32) = 8 (r / 4) + 4 (l / 32) + r % 4.
//  - Row operands (K, V rows for S^T = K Q^T, dP^T = V dO^T; Q, dO rows for
//    S = Q K^T, dP = dO V^T): one 16-byte LDS read gives lane l the values
//    d = 8 c + 4 (l / 32) + e, e < 4, of row l % 32, which feed four MFMAs;
//    the stationary operand (Q, dO, K or V of the lane's own row) is held in
//    registers in the same d order.
//  - Column operands (V^T for O^T += V^T P^T, K^T for dQ^T, dO^T and Q^T for
//    dV^T, dK^T): for the k-step whose half-waves take rows kidx(kk, 0) and
//    kidx(kk, 1) of the streamed tile, lane l reads R = D/32 consecutive values
//    d = R (l % 32) + j of its half's row in one LDS read; they feed R MFMAs,
//    and block j of those accumulators holds row d = R i + j in its row i.
//    The other operand (P^T, dS^T, P or dS) is register kk of a score
//    result as it stands.  No transposed copy or transposing read is needed.
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace bwattn {

namespace {

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// row of a 32x32 result held in register r by half-wave h
__device__ __forceinline__ constexpr int kidx(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// LDS tile of R rows of D floats, one 16-byte chunk of padding per row (the
// row stride is 16 bytes off a multiple of 256, so 16-byte reads of 16
// consecutive rows at one column hit distinct bank groups).
template <int R, int D>
using FTile = PTile<R, D / 4, 1>;

// row operand: values d = 8 c + 4 (lane / 32) + [0, 4) of row r0 + lane % 32
template <class T>
__device__ __forceinline__ f32x4 row_op(const char* t, int r0, int c, int lane) {
  return __builtin_bit_cast(f32x4, T::read(t, r0, c, lane));
}

template <int R>
struct ColVec;
template <>
struct ColVec<4> {
  typedef f32x4 type;
};
template <>
struct ColVec<2> {
  typedef f32x2 type;
};

// column operand: values d = R (lane % 32) + [0, R) of tile row r
template <int D, class T>
__device__ __forceinline__ typename ColVec<D / 32>::type col_op(const char* t, int r, int lane) {
  typedef typename ColVec<D / 32>::type V;
  return *(const V*)(t + r * T::kStride + (lane & 31) * (D / 32) * 4);
}

// two operands read together (S and dP share the k-steps, and so do dV and dK)
template <class V>
struct OpPair {
  V x, y;
};
typedef OpPair<f32x4> F4Pair;

// Stationary operand of the lane's own row: d = 8 c + 4 hl + [0, 4).
template <int D>
__device__ __forceinline__ void load_own_row(const float* rowp, bool ok, int hl, f32x4 (&x)[D / 8]) {
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    f32x4 v = *(const f32x4*)(rowp + 8 * c + 4 * hl);
    x[c] = ok ? v : f32x4{};
  }
}

// Store an accumulator set in column layout (block j, register r holds
// d = R kidx(r, hl) + j of the lane's row) as fp32 times `mul`.
template <int D>
__device__ __forceinline__ void store_col_rows(float* dst_row, const f32x16 (&x)[D / 32], float mul, int hl) {
  constexpr int R = D / 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float* p = dst_row + R * kidx(r, hl);
    if constexpr (R == 4)
      *(f32x4*)p = f32x4{x[0][r] * mul, x[1][r] * mul, x[2][r] * mul, x[3][r] * mul};
    else
      *(f32x2*)p = f32x2{x[0][r] * mul, x[1][r] * mul};
  }
}

// RoPE backward (rotation by -pos w_p) of a row held in column layout: the
// pair (2p, 2p+1) is blocks (j, j+1), j even, of one register.
template <int D>
__device__ __forceinline__ void rope_backward_col(f32x16 (&x)[D / 32], double pos, const double* turns, int hl) {
  constexpr int R = D / 32;
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int j = 0; j < R; j += 2) {
      const int d = R * kidx(r, hl) + j;
      double rev = pos * turns[d >> 1];
      rev -= rint(rev);
      float f = (float)rev;
      float c = __builtin_amdgcn_cosf(f), s = __builtin_amdgcn_sinf(f);
      float x0 = x[j][r], x1 = x[j + 1][r];
      x[j][r] = x0 * c + x1 * s;
      x[j + 1][r] = x1 * c - x0 * s;
    }
}

// Walk over the K/V tiles of a query block (forward and dQ).
__device__ __forceinline__ TileWalk query_block_walk(const F32Args& a, int b, int qt, int Q0, int BQ, int BK,
                                                     const int2* blkb, bool use_seg) {
  TileWalk walk;
  const int S = a.S;
  if (a.range) {
    walk_range(walk, a.range[(int64_t)b * a.n_own + qt], blkb);
  } else {
    walk.lo = 0;
    walk.hi = a.causal ? min(a.n_other, (min(S, Q0 + BQ) - 1) / BK + 1) : a.n_other;
    walk.blk = nullptr;
  }
  walk.ct = a.chunk_tiles;
  walk.nc = a.chunk_tiles ? (a.n_other + a.chunk_tiles - 1) / a.chunk_tiles : 1;
  walk.r = a.chunk_tiles ? (Q0 / BK) / a.chunk_tiles : 0;
  walk.dir = -1;
  walk.desc = 0;
  walk.nblk = a.nblk;
  walk.rows = BK;
  walk.own = use_seg ? seg_range(blkb, a.nblk, Q0, min(BQ, S - Q0)) : make_int2(0, 0);
  walk.start();
  return walk;
}

}  // namespace

// ---------------------------------------------------------------------------
// Forward: NW waves x 32 query rows (two waves per SIMD); tiles of 64 keys of
// K and V rows in a two-slot LDS ring.  Per tile: S^T = K Q^T (lane = query
// row), mask, lazy online-softmax update, O^T += V^T P^T.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_f32_kernel(F32Args a) {
  constexpr int BQ = kF32FwdBlockQ, BK = kFwdBlockK;
  static_assert(BQ == NW * 32, "32 query rows per wave");
  static_assert(BK == 64, "two 32-key halves per tile");
  constexpr int NC = D / 8;   // row-operand reads over D (four k-steps each)
  constexpr int R = D / 32;   // accumulator blocks of O^T
  constexpr float kLazy = 8.f;
  using T = FTile<BK, D>;
  constexpr int SEG_OFF = 2 * T::kBytes;
  constexpr int BUF = SEG_OFF + 256;
  constexpr int NSTAGE = 2;
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * BUF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_own, bh, rank);
  const int qt = a.n_own - 1 - rank;  // causal work grows with the tile index
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int Q0 = qt * BQ;
  const int q0 = Q0 + w * 32;
  const int row = q0 + l32;
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;

  f32x4 qop[NC];
  load_own_row<D>(a.q + base + (int64_t)min(row, S - 1) * D, row < S, hl, qop);
  const int segq = (use_seg && row < S) ? segb[row] : 0;
  int2 wrange = make_int2(0, 0);
  if (use_seg && q0 < S) wrange = seg_range(blkb, a.nblk, q0, min(32, S - q0));
  TileWalk walk = query_block_walk(a, b, qt, Q0, BQ, BK, blkb, use_seg);

  float m = kNegInf, lsum = 0.f;
  f32x16 o[R];
#pragma unroll
  for (int j = 0; j < R; ++j) o[j] = f32x16{};
  const float sl2 = a.scale_log2;
  const float* kh = a.k + base;
  const float* vh = a.v + base;
  TileFill<BK, D / 4, NW> fill;
  fill.init(D * 4, tid);
  auto load = [&](int t, char* buf) {
    const uint32_t bytes = (uint32_t)min(S - t * BK, BK) * D * 4;  // rows past S read zero
    fill.fill(kh + (int64_t)t * BK * D, bytes, buf);
    fill.fill(vh + (int64_t)t * BK * D, bytes, buf + T::kBytes);
    if (use_seg && w == 0) row64_to_lds(segb, t * BK, S, buf + SEG_OFF, lane);
  };
  const int per_tile = 2 * fill.count() + (use_seg && w == 0 ? 1 : 0);

  auto compute = [&](int t, const char* buf) {
    const int k0 = t * BK;
    if (q0 >= S || (a.causal && k0 > q0 + 31)) return;  // nothing visible to this wave
    const char* ktl = buf;
    const char* vtl = buf + T::kBytes;
    // S^T: s[h] holds keys k0 + 32 h + kidx(r, hl) of this lane's row
    f32x16 s[2] = {f32x16{}, f32x16{}};
    lds_mfma_pipe<NC, 2>(
        [&](int c) { return F4Pair{row_op<T>(ktl, 0, c, lane), row_op<T>(ktl, 32, c, lane)}; },
        [&](int c, F4Pair x) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[0] = mfma_f32(x.x[e], qop[c][e], s[0]);
            s[1] = mfma_f32(x.y[e], qop[c][e], s[1]);
          }
        });
    bool seg_mask = false;
    if (use_seg) {
      int2 kr = seg_range(blkb, a.nblk, k0, BK);
      seg_mask = !(kr.x == kr.y && wrange.x == wrange.y && kr.x == wrange.x);
    }
    if (seg_mask || (k0 + BK > S) || (a.causal && k0 + BK - 1 > q0)) {
      const int* segk = (const int*)(buf + SEG_OFF);
      const int lim = a.causal ? min(S - 1, row) : S - 1;  // last visible key of this row
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = 32 * h + kidx(r, hl);
          const bool vis = (k0 + jj <= lim) && (!use_seg || segk[jj] == segq);
          s[h][r] = vis ? s[h][r] : kNegInf;
        }
    }
    // lazy online-softmax update: the running max m moves only when the
    // tile's max exceeds it by more than kLazy (log2 units); l and O share m,
    // so the normalised result is the same
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s[0][r]), s[1][r]);
    mx = pair_max(mx) * sl2;
    const bool grow = mx > m + kLazy;
    if (__ballot(grow)) {
      float mnew = grow ? fmaxf(m, mx) : m;
      float alpha = fast_exp2(m - (mnew == kNegInf ? 0.f : mnew));
      lsum *= alpha;
#pragma unroll
      for (int j = 0; j < R; ++j) o[j] *= alpha;
      m = mnew;
    }
    const float muse = m == kNegInf ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[h][r] = fast_exp2(__builtin_fmaf(s[h][r], sl2, -muse));
        rs += s[h][r];
      }
    lsum += rs;
    // O^T += V^T P^T: k-step kk of half h takes V rows 32 h + kidx(kk, .)
    lds_mfma_pipe<32, 3>([&](int i) { return col_op<D, T>(vtl, 32 * (i >> 4) + kidx(i & 15, hl), lane); },
                         [&](int i, auto x) {
#pragma unroll
                           for (int j = 0; j < R; ++j) o[j] = mfma_f32(x[j], s[i >> 4][i & 15], o[j]);
                         });
  };
  run_pipeline<NSTAGE, false>(walk, per_tile, smem, BUF, load, compute);

  // epilogue: O = O^T / l, LSE = ln 2 (m + log2 l)
  const float lt = pair_sum(lsum);
  if (row < S) {
    store_col_rows<D>(a.out_o + base + (int64_t)row * D, o, 1.f / lt, hl);
    if (hl == 0) a.out_lse[(int64_t)bh * S + row] = (m + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// dQ (and Delta): NW waves x 32 query rows, one wave per SIMD; tiles of 64
// keys of K and V.  Per 32-key half: S^T = K Q^T and dP^T = V dO^T, then
// dS^T = P^T (dP^T - Delta) and dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dq_f32_kernel(F32Args a) {
  constexpr int BQ = kF32DqBlockQ, BK = kFwdBlockK;
  static_assert(BQ == NW * 32, "32 query rows per wave");
  constexpr int NC = D / 8, R = D / 32;
  using T = FTile<BK, D>;
  constexpr int SEG_OFF = 2 * T::kBytes;
  constexpr int BUF = SEG_OFF + 256;
  constexpr int NSTAGE = 2;
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * BUF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_own, bh, rank);
  const int qt = a.n_own - 1 - rank;
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int Q0 = qt * BQ;
  const int q0 = Q0 + w * 32;
  const int row = q0 + l32;
  const bool ok = row < S;
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;

  f32x4 qop[NC], dop[NC];
  const int64_t ro = base + (int64_t)min(row, S - 1) * D;
  load_own_row<D>(a.q + ro, ok, hl, qop);
  load_own_row<D>(a.dout + ro, ok, hl, dop);
  float delta;
  {
    float dsum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      f32x4 ov = *(const f32x4*)(a.o + ro + 8 * c + 4 * hl);
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum = __builtin_fmaf(dop[c][e], ov[e], dsum);
    }
    dsum = pair_sum(dsum);
    delta = ok ? dsum : 0.f;
  }
  const float nlse2 = ok ? -a.lse[(int64_t)bh * S + row] * kLog2e : 0.f;
  if (ok && hl == 0) {  // row statistics for the dK/dV kernel
    a.ndelta[(int64_t)bh * S + row] = -delta;
    a.nlse2[(int64_t)bh * S + row] = nlse2;
  }
  const int segq = (use_seg && ok) ? segb[row] : 0;
  const int qlast = min(S - 1, q0 + 31);
  int2 wrange = make_int2(0, 0);
  if (use_seg && q0 < S) wrange = seg_range(blkb, a.nblk, q0, min(32, S - q0));
  TileWalk walk = query_block_walk(a, b, qt, Q0, BQ, BK, blkb, use_seg);

  f32x16 dq[R];
#pragma unroll
  for (int j = 0; j < R; ++j) dq[j] = f32x16{};
  const float sl2 = a.scale_log2;
  const float* kh = a.k + base;
  const float* vh = a.v + base;
  TileFill<BK, D / 4, NW> fill;
  fill.init(D * 4, tid);
  auto load = [&](int t, char* buf) {
    const uint32_t bytes = (uint32_t)min(S - t * BK, BK) * D * 4;  // rows past S read zero
    fill.fill(kh + (int64_t)t * BK * D, bytes, buf);
    fill.fill(vh + (int64_t)t * BK * D, bytes, buf + T::kBytes);
    if (use_seg && w == 0) row64_to_lds(segb, t * BK, S, buf + SEG_OFF, lane);
  };
  const int per_tile = 2 * fill.count() + (use_seg && w == 0 ? 1 : 0);

  auto compute = [&](int t, const char* buf) {
    const int k0 = t * BK;
    bool skip = q0 >= S || (a.causal && k0 > qlast);
    bool seg_mask = false;
    if (use_seg && !skip) {
      int2 kr = seg_range(blkb, a.nblk, k0, BK);
      if (!ranges_meet(kr, wrange))
        skip = true;
      else
        seg_mask = !(kr.x == kr.y && wrange.x == wrange.y && kr.x == wrange.x);
    }
    if (skip) return;
    const char* ktl = buf;
    const char* vtl = buf + T::kBytes;
    const int* segk = (const int*)(buf + SEG_OFF);
    const bool need_mask = seg_mask || (k0 + BK > S) || (a.causal && k0 + BK - 1 > q0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // dP^T starts from -Delta, so the MFMAs leave dP^T - Delta
      f32x16 s = f32x16{}, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = -delta;
      lds_mfma_pipe<NC, 2>(
          [&](int c) { return F4Pair{row_op<T>(ktl, 32 * h, c, lane), row_op<T>(vtl, 32 * h, c, lane)}; },
          [&](int c, F4Pair x) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s = mfma_f32(x.x[e], qop[c][e], s);
              dp = mfma_f32(x.y[e], dop[c][e], dp);
            }
          });
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = 32 * h + kidx(r, hl);
          const int j = k0 + jj;
          const bool vis = j < S && (!a.causal || j <= row) && (!use_seg || segk[jj] == segq);
          s[r] = vis ? s[r] : kNegInf;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(__builtin_fmaf(s[r], sl2, nlse2)) * dp[r];
      // dQ^T += K^T dS^T over the 32 keys of this half
      lds_mfma_pipe<16, 3>([&](int kk) { return col_op<D, T>(ktl, 32 * h + kidx(kk, hl), lane); },
                           [&](int kk, auto x) {
#pragma unroll
                             for (int j = 0; j < R; ++j) dq[j] = mfma_f32(x[j], s[kk], dq[j]);
                           });
    }
  };
  run_pipeline<NSTAGE, false>(walk, per_tile, smem, BUF, load, compute);

  if (ok) {
    if (a.rope) {
      double pos = a.pos ? (double)a.pos[(int64_t)b * S + row] : (double)row;
      rope_backward_col<D>(dq, pos, a.turns, hl);
    }
    store_col_rows<D>(a.dq + base + (int64_t)row * D, dq, a.scale, hl);
  }
}

// ---------------------------------------------------------------------------
// dK/dV: NW waves x 32 keys, one wave per SIMD; tiles of 64 query rows of Q
// and dO with their row statistics.  Scores with lane = key: S = Q K^T,
// dP = dO V^T (the lane's K and V rows in registers), then dV^T += dO^T P and
// dK^T += Q^T dS.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkdv_f32_kernel(F32Args a) {
  constexpr int BKV = kF32BwdBlockK, BQT = kF32BwdBlockQ;
  static_assert(BKV == NW * 32, "32 keys per wave");
  constexpr int NC = D / 8, R = D / 32;
  using T = FTile<BQT, D>;
  constexpr int SB = 2 * T::kBytes;  // -LSE log2e [64], -Delta [64], seg [64]
  constexpr int BUF = SB + 3 * 256;
  constexpr int NSTAGE = 2;
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * BUF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_own, bh, rank);
  const int kt_idx = rank;  // causal work shrinks with the key tile index: low tiles first
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int K0 = kt_idx * BKV;
  const int j0 = K0 + 32 * w;
  const int j = j0 + l32;  // this lane's key
  const bool jok = j < S;
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;

  f32x4 kop[NC], vop[NC];
  const int64_t ro = base + (int64_t)min(j, S - 1) * D;
  load_own_row<D>(a.k + ro, jok, hl, kop);
  load_own_row<D>(a.v + ro, jok, hl, vop);
  const int segk = (use_seg && jok) ? segb[j] : 0;
  int2 wrange = make_int2(0, 0);
  if (use_seg && j0 < S) wrange = seg_range(blkb, a.nblk, j0, min(32, S - j0));

  TileWalk walk;
  if (a.range) {
    walk_range(walk, a.range[(int64_t)b * a.n_own + kt_idx], blkb);
  } else {
    walk.lo = a.causal ? K0 / BQT : 0;
    walk.hi = a.n_other;
    walk.blk = nullptr;
  }
  walk.ct = a.chunk_tiles;
  walk.nc = a.chunk_tiles ? (a.n_other + a.chunk_tiles - 1) / a.chunk_tiles : 1;
  walk.r = a.chunk_tiles ? (K0 / BQT) / a.chunk_tiles : 0;
  walk.dir = +1;
  walk.desc = 1;  // natural order from the last query tile down (L2 reuse across workgroups)
  walk.nblk = a.nblk;
  walk.rows = BQT;
  walk.own = use_seg ? seg_range(blkb, a.nblk, K0, min(BKV, S - K0)) : make_int2(0, 0);
  walk.start();

  f32x16 dk[R], dv[R];
#pragma unroll
  for (int jb = 0; jb < R; ++jb) dk[jb] = dv[jb] = f32x16{};
  const float sl2 = a.scale_log2;
  const float* qh = a.q + base;
  const float* dh = a.dout + base;
  const float* nlse_h = a.nlse2 + (int64_t)bh * S;
  const float* ndel_h = a.ndelta + (int64_t)bh * S;
  TileFill<BQT, D / 4, NW> fill;
  fill.init(D * 4, tid);
  auto load = [&](int t, char* buf) {
    const uint32_t bytes = (uint32_t)min(S - t * BQT, BQT) * D * 4;  // rows past S read zero
    fill.fill(qh + (int64_t)t * BQT * D, bytes, buf);
    fill.fill(dh + (int64_t)t * BQT * D, bytes, buf + T::kBytes);
    if (w == 0) {
      row64_to_lds(nlse_h, t * BQT, S, buf + SB, lane);
      row64_to_lds(ndel_h, t * BQT, S, buf + SB + 256, lane);
      if (use_seg) row64_to_lds(segb, t * BQT, S, buf + SB + 512, lane);
    }
  };
  const int per_tile = 2 * fill.count() + (w == 0 ? (use_seg ? 3 : 2) : 0);

  auto compute = [&](int t, const char* buf) {
    const int i0 = t * BQT;
    const int ilast = min(S - 1, i0 + BQT - 1);
    bool skip = j0 >= S || (a.causal && ilast < j0);
    bool seg_mask = false;
    if (use_seg && !skip) {
      int2 qr = seg_range(blkb, a.nblk, i0, BQT);
      if (!ranges_meet(qr, wrange))
        skip = true;
      else
        seg_mask = !(qr.x == qr.y && wrange.x == wrange.y && qr.x == wrange.x);
    }
    if (skip) return;
    const char* qtl = buf;
    const char* dtl = buf + T::kBytes;
    const float* st = (const float*)(buf + SB);
    const bool need_mask = seg_mask || (i0 + BQT > S) || (a.causal && i0 < j0 + 31);
    // one 32-row half at a time (unrolled, the two halves' scores and
    // operands would not fit the register file next to K, V, dK and dV)
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      // S and dP for query rows i0 + 32 h + kidx(r, hl)
      f32x16 s = f32x16{}, dp = f32x16{};
      lds_mfma_pipe<NC, 2>(
          [&](int c) { return F4Pair{row_op<T>(qtl, 32 * h, c, lane), row_op<T>(dtl, 32 * h, c, lane)}; },
          [&](int c, F4Pair x) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s = mfma_f32(x.x[e], kop[c][e], s);
              dp = mfma_f32(x.y[e], vop[c][e], dp);
            }
          });
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ri = 32 * h + kidx(r, hl);
          const int i = i0 + ri;
          const int sq = ((const int*)st)[128 + ri];
          const bool vis = i < S && (!a.causal || j <= i) && (!use_seg || sq == segk);
          s[r] = vis ? s[r] : kNegInf;
        }
      }
      // P = exp(S scale - LSE) into s, dS = P (dP - Delta) into dp
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int ri = 32 * h + 8 * rq + 4 * hl;
        const f32x4 nl = *(const f32x4*)(st + ri);
        const f32x4 nd = *(const f32x4*)(st + 64 + ri);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[4 * rq + e], sl2, nl[e]));
          s[4 * rq + e] = p;
          dp[4 * rq + e] = p * (dp[4 * rq + e] + nd[e]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over these 32 rows
      lds_mfma_pipe<16, 3>(
          [&](int kk) {
            const int r = 32 * h + kidx(kk, hl);
            return OpPair<typename ColVec<R>::type>{col_op<D, T>(dtl, r, lane), col_op<D, T>(qtl, r, lane)};
          },
          [&](int kk, auto x) {
#pragma unroll
            for (int jb = 0; jb < R; ++jb) {
              dv[jb] = mfma_f32(x.x[jb], s[kk], dv[jb]);
              dk[jb] = mfma_f32(x.y[jb], dp[kk], dk[jb]);
            }
          });
    }
  };
  run_pipeline<NSTAGE, false>(walk, per_tile, smem, BUF, load, compute);

  if (jok) {
    if (a.rope) {
      double pos = a.pos ? (double)a.pos[(int64_t)b * S + j] : (double)j;
      rope_backward_col<D>(dk, pos, a.turns, hl);
    }
    store_col_rows<D>(a.dk + base + (int64_t)j * D, dk, a.scale, hl);
    store_col_rows<D>(a.dv + base + (int64_t)j * D, dv, 1.f, hl);
  }
}

hipError_t launch_attn_fwd_f32(const F32Args& a, int D, hipStream_t st) {
  constexpr int NW = kF32FwdBlockQ / 32;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_own)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<128, NW>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_f32_kernel<64, NW>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_f32(const F32Args& a, int D, hipStream_t st) {
  constexpr int NW = kF32DqBlockQ / 32;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_own)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_bwd_dq_f32_kernel<128, NW>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_f32_kernel<64, NW>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_f32(const F32Args& a, int D, hipStream_t st) {
  constexpr int NW = kF32BwdBlockK / 32;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_own)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_bwd_dkdv_f32_kernel<128, NW>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_f32_kernel<64, NW>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
