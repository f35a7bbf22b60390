// Forward of blockwise exact attention (gfx950, bf16 MFMA, fp32 accumulate).
//
// The paper trains with blockwise ring attention fused with FlashAttention:
// a block of queries streams K/V blocks and merges each block's partial
// result with an online softmax (running max m, running sum l), which gives
// exact attention (zhao9797 page "LWM (Large World Model)", 模型架构; elamur.ai
// summary page: no approximation).  Masks: causal (decoder-only model) and
// the packing mask (each packed example attends only to itself, 训练方法).
//
// Work decomposition: a workgroup of NW waves owns 256 query rows of one
// (batch, head); each wave owns 32 * QG rows.  Tiles of 64 keys of K and of
// the transposed V are double-buffered in LDS and filled by direct
// global-to-LDS loads.  Scores are computed transposed, S^T = K Q^T, so each
// lane holds one query row: the row max needs one exchange between lanes l
// and l^32, and the running rescale of O is a per-lane scalar.
// O^T = V^T P^T takes P^T straight from the score registers; the transposed V
// copy stores each 16 keys in the order those registers hold them, so both
// MFMA operands are plain 16-byte LDS reads.
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace bwattn {

template <int D, int NW, int QG, int NSTAGE>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdArgs a) {
  constexpr int BQ = kFwdBlockQ, BK = kFwdBlockK;
  static_assert(BQ == NW * 32 * QG, "query rows per workgroup");
  static_assert(BK == 64, "two 32-key halves per tile");
  constexpr int NDC = D / 16;             // 16-wide k steps over D for S^T
  constexpr int NDG = D / 32;             // 32-row groups of O^T over D
  constexpr float kLazy = 8.f;
  using KT = PTile<BK, D / 8>;            // K rows
  using VT = PTile<D, BK / 8>;            // V^T rows (d), 64 keys each
  constexpr int SEG_OFF = KT::kBytes + VT::kBytes;  // segment ids of the tile's keys
  constexpr int BUF = SEG_OFF + 256;
  // NSTAGE-deep ring of [K, V^T, seg] tiles: the loads for tile
  // t + NSTAGE - 1 are in flight while tile t is computed
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * BUF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_qtiles, bh, rank);
  const int qt = a.n_qtiles - 1 - rank;  // causal work grows with the tile index
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int Q0 = qt * BQ;
  constexpr int QW = 32 * QG;  // rows per wave
  const int q0 = Q0 + w * QW;
  const int qlast = min(S - 1, q0 + QW - 1);
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;

  // Q operand (B of S^T = K Q^T): lane holds row q0 + 32 qg + l32, d = 16 dc + 8 hl + [0,8)
  bf16x8 qop[QG][NDC];
  int segq[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    int row = q0 + 32 * qg + l32;
    bool ok = row < S;
    const uint16_t* src = a.q + base + (int64_t)min(row, S - 1) * D + 8 * hl;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      bf16x8 v = *(const bf16x8*)(src + 16 * dc);
      qop[qg][dc] = ok ? v : bf16x8{};
    }
    segq[qg] = (use_seg && ok) ? segb[row] : 0;
  }
  int2 wrange = make_int2(0, 0);
  if (use_seg && q0 < S) wrange = seg_range(blkb, a.nblk, q0, min(QW, S - q0));

  // K/V tile range and walk
  TileWalk walk;
  if (a.qrange) {
    int2 r = a.qrange[(int64_t)b * a.n_qtiles + qt];
    walk.lo = r.x;
    walk.hi = r.y;
  } else {
    walk.lo = 0;
    walk.hi = a.causal ? min(a.n_ktiles, (min(S, Q0 + BQ) - 1) / BK + 1) : a.n_ktiles;
  }
  walk.ct = a.chunk_tiles;
  walk.nc = a.chunk_tiles ? (a.n_ktiles + a.chunk_tiles - 1) / a.chunk_tiles : 1;
  walk.r = a.chunk_tiles ? (Q0 / BK) / a.chunk_tiles : 0;
  walk.dir = -1;
  walk.desc = false;
  walk.blk = blkb;
  walk.nblk = a.nblk;
  walk.rows = BK;
  walk.own = use_seg ? seg_range(blkb, a.nblk, Q0, min(BQ, S - Q0)) : make_int2(0, 0);
  walk.start();

  float m[QG], lsum[QG];
  f32x16 o[QG][NDG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    m[qg] = kNegInf;
    lsum[qg] = 0.f;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg) o[qg][dg] = f32x16{};
  }
  const float sl2 = a.scale_log2;
  const uint16_t* kh = a.k + base;
  const uint16_t* vth = a.vt + (int64_t)bh * D * a.sp;
  TileFill<BK, D / 8, NW> kfill;  // K rows
  TileFill<D, BK / 8, NW> vfill;  // V^T rows
  kfill.init(D * 2, tid);
  vfill.init(a.sp * 2, tid);
  auto load = [&](int t, char* buf) {
    kfill.fill(kh + (int64_t)t * BK * D, (uint32_t)(S - t * BK) * D * 2, buf);
    vfill.fill(vth + t * BK, (uint32_t)(D * a.sp - t * BK) * 2, buf + KT::kBytes);
    if (use_seg && w == 0) row64_to_lds(segb, t * BK, S, buf + SEG_OFF, lane);
  };
  // vector-memory instructions this wave issues per tile
  const int per_tile = kfill.count() + vfill.count() + (use_seg && w == 0 ? 1 : 0);
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
    if (!skip) {
      const char* kt = buf;
      const char* vt = buf + KT::kBytes;
      const int* segk_lds = (const int*)(buf + SEG_OFF);
      // S^T = K Q^T for both 32-key halves (independent accumulator chains):
      // s[qg][kg] holds keys k0 + 32 kg + 8 (r/4) + 4 hl + r%4 of row l32
      f32x16 s[QG][2];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) s[qg][0] = s[qg][1] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          bf16x8 ka = KT::read(kt, 32 * kg, dc, lane);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) s[qg][kg] = mfma32(ka, qop[qg][dc], s[qg][kg]);
        }
      }
      if (seg_mask || (k0 + BK > S) || (a.causal && k0 + BK - 1 > q0)) {
        // partial tile: causal, segment and sequence-end masks
        int jb = k0 + 4 * hl;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int j = jb + 32 * kg + 8 * (r >> 2) + (r & 3);
            int sk = 0;
            if (use_seg) sk = segk_lds[j - k0];
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
              int i = q0 + 32 * qg + l32;
              bool vis = j < S && (!a.causal || j <= i) && (!use_seg || sk == segq[qg]);
              s[qg][kg][r] = vis ? s[qg][kg][r] : kNegInf;
            }
          }
      }
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        // Online softmax merge.  A row's running max m is raised only when
        // its new max exceeds it by more than kLazy (log2 units); otherwise
        // the stale m stays, p <= 2^kLazy, and O is not touched.  l and O
        // share m, so the normalised result is unchanged.  The decision is
        // per row (the wave only branches when some row needs it), so a
        // row's result depends on its own visible keys alone.
        bf16x8 pk[QG][2];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          f32x16& sv = s[qg][kg];
          float mx = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
          for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, sv[r]), sv[r + 1]);
          mx = fmaxf(mx, sv[15]);
          mx = pair_max(mx) * sl2;
          const bool grow = mx > m[qg] + kLazy;
          if (__ballot(grow)) {
            float mnew = grow ? fmaxf(m[qg], mx) : m[qg];
            float alpha = fast_exp2(m[qg] - (mnew == kNegInf ? 0.f : mnew));  // 1 when m stays
            lsum[qg] *= alpha;
#pragma unroll
            for (int dg = 0; dg < NDG; ++dg) o[qg][dg] *= alpha;
            m[qg] = mnew;
          }
          const float muse = (m[qg] == kNegInf) ? 0.f : m[qg];
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = fast_exp2(__builtin_fmaf(sv[r], sl2, -muse));
          // P in bf16 feeds the MFMA; the row sum adds the same bf16 values
          float rs = lsum[qg];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            int r0 = 8 * c;
            u32x4 pw = {pack_bf16x2(sv[r0], sv[r0 + 1]), pack_bf16x2(sv[r0 + 2], sv[r0 + 3]),
                        pack_bf16x2(sv[r0 + 4], sv[r0 + 5]), pack_bf16x2(sv[r0 + 6], sv[r0 + 7])};
#pragma unroll
            for (int e = 0; e < 4; ++e) rs = dot2_bf16(pw[e], kBf16OnePair, rs);
            pk[qg][c] = __builtin_bit_cast(bf16x8, pw);
          }
          lsum[qg] = rs;
        }
        // O^T += V^T P^T over the 32 keys of this half
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg) {
            bf16x8 va = VT::read(vt, 32 * dg, 2 * kg + c, lane);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) o[qg][dg] = mfma32(va, pk[qg][c], o[qg][dg]);
          }
        }
      }
    }
  };
  run_pipeline<NSTAGE>(walk, per_tile, smem, BUF, load, compute);

  // epilogue: O = O^T / l, LSE = ln2 (m + log2 l)
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    int row = q0 + 32 * qg + l32;
    float lt = pair_sum(lsum[qg]);
    float inv = 1.f / lt;
    if (row < S) {
      uint16_t* dst = a.o + base + (int64_t)row * D + 4 * hl;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16& ov = o[qg][dg];
          uint32_t w0 = pack_bf16x2(ov[4 * rq] * inv, ov[4 * rq + 1] * inv);
          uint32_t w1 = pack_bf16x2(ov[4 * rq + 2] * inv, ov[4 * rq + 3] * inv);
          *(u32x2*)(dst + 32 * dg + 8 * rq) = u32x2{w0, w1};
        }
      if (hl == 0) a.lse[(int64_t)bh * S + row] = (m[qg] + __log2f(lt)) * kLn2;
    }
  }
}

hipError_t launch_attn_fwd(const FwdArgs& a, int D, hipStream_t st) {
  constexpr int NW = 8, QG = 1, NSTAGE = 3;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_qtiles)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, NW, QG, NSTAGE>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, NW, QG, NSTAGE>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
