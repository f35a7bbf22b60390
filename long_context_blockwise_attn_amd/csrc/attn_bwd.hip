// Backward of blockwise exact attention (gfx950, bf16 MFMA, fp32 accumulate).
//
// Training takes gradient steps through the attention (zhao9797 page
// "LWM (Large World Model)", 训练方法).  Memory stays linear in S as in the
// blockwise method: the probabilities are recomputed from the saved
// log-sum-exp,  P_ij = exp(scale <q'_i, k'_j> - LSE_i), and with
// Delta_i = <dO_i, O_i>:
//   dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - Delta_i),
//   dv_j = sum_i P_ij dO_i,  dk'_j = scale sum_i dS_ij q'_i,
//   dq'_i = scale sum_j dS_ij k'_j,
// then the RoPE backward dq = R(-a) dq', dk = R(-a) dk'.
//
// Two kernels, no atomics (the result is bitwise reproducible):
//  - dQ kernel: a workgroup owns 256 query rows (like the forward) and
//    streams K/V tiles of 128 keys (two-slot ring); it also forms Delta for
//    its rows.  3 contractions per tile pair (S, dP, dQ).
//  - dK/dV kernel: a workgroup owns kBwdBlockK keys and streams Q/dO tiles of
//    kBwdBlockQ rows (two-slot ring).  4 contractions per tile pair (S, dP,
//    dV, dK).
// Each wave issues its share of the next tile's loads between the 32-row (or
// 32-key) halves of the tile it computes, where its issue stall overlaps
// the MFMAs of the other wave of its SIMD.
// Operands with k along the sequence (K^T for dQ, Q^T and dO^T for dK/dV)
// are read from the same row tiles with transposing LDS reads
// (PTile::read_tr), so each tile is loaded once and no transposed copy is
// made.
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace bwattn {

// Rotate pairs (x[2p], x[2p+1]) of one row at position `pos` by -pos*w_p in
// registers; x holds d = 32 dg + 8 (r/4) + 4 hl + r%4, so pairs are the
// register pairs (r, r+1) with r even.
template <int NDG>
__device__ __forceinline__ void rope_backward_row(f32x16 (&x)[NDG], double pos, const double* turns, int hl) {
#pragma unroll
  for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      int d = 32 * dg + 8 * (r >> 2) + 4 * hl + (r & 3);
      double rev = pos * turns[d >> 1];
      rev -= rint(rev);
      float f = (float)rev;
      float c = __builtin_amdgcn_cosf(f), s = __builtin_amdgcn_sinf(f);
      float x0 = x[dg][r], x1 = x[dg][r + 1];
      x[dg][r] = x0 * c + x1 * s;
      x[dg][r + 1] = x1 * c - x0 * s;
    }
}

// Store rows held transposed (lane = row, registers = d) as bf16, times `mul`.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* dst_row, const f32x16 (&x)[D / 32], float mul, int hl) {
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      uint32_t w0 = pack_bf16x2(x[dg][4 * rq] * mul, x[dg][4 * rq + 1] * mul);
      uint32_t w1 = pack_bf16x2(x[dg][4 * rq + 2] * mul, x[dg][4 * rq + 3] * mul);
      *(u32x2*)(dst_row + 32 * dg + 8 * rq + 4 * hl) = u32x2{w0, w1};
    }
}

// ---------------------------------------------------------------------------
// dQ (and Delta): NW waves x 32 query rows; tiles of 64 keys of K and V in
// LDS.  Per 32-key half: S^T = K Q^T and dP^T = V dO^T
// (lane = query row), then dS^T = P^T (dP^T - Delta) and dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
template <int D, int NW, int NSTAGE>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int BQ = kFwdBlockQ, BK = 2 * kFwdBlockK;  // two tiles of the K/V range table per tile
  static_assert(BQ == NW * 32, "one 32-row group per wave");
  constexpr int NDC = D / 16, NDG = D / 32;
  using KT = PTile<BK, D / 8, 3>;  // K and V rows (K^T read transposed)
  constexpr int SEG_OFF = 2 * KT::kBytes;  // segment ids of the tile's keys
  constexpr int BUF = SEG_OFF + 4 * BK;
  // ring of [K, V, seg] stages (see run_pipeline)
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * BUF];

  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_qtiles, bh, rank);
  const int qt = a.n_qtiles - 1 - rank;
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int Q0 = qt * BQ;
  const int q0 = Q0 + w * 32;
  const int row = q0 + l32;  // this lane's query row
  const bool ok = row < S;
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;
  const int2* t64b = use_seg ? a.t64 + (int64_t)b * a.n64p : nullptr;

  bf16x8 qop[NDC], dop[NDC];
  float delta;
  {
    int64_t ro = base + (int64_t)min(row, S - 1) * D + 8 * hl;
    float dsum = 0.f;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      bf16x8 qv = *(const bf16x8*)(a.q + ro + 16 * dc);
      u32x4 dv = *(const u32x4*)(a.dout + ro + 16 * dc);
      u32x4 ov = *(const u32x4*)(a.o + ro + 16 * dc);
      qop[dc] = ok ? qv : bf16x8{};
      dop[dc] = ok ? __builtin_bit_cast(bf16x8, dv) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum += bf16_lo(dv[e]) * bf16_lo(ov[e]) + bf16_hi(dv[e]) * bf16_hi(ov[e]);
    }
    dsum = pair_sum(dsum);
    delta = ok ? dsum : 0.f;
  }
  const float nlse2 = ok ? -a.lse[(int64_t)bh * S + row] * kLog2e : 0.f;
  if (ok && hl == 0) {  // row statistics for the dK/dV kernel
    a.ndelta[(int64_t)bh * S + row] = -delta;
    a.nlse2[(int64_t)bh * S + row] = nlse2;
  }
  // start values of the S^T and dP^T MFMAs: the query operand carries
  // scale * log2(e), so S^T starts from -LSE log2(e) and leaves the exponent
  // of exp2; dP^T starts from -Delta and leaves dP^T - Delta
  f32x16 s_init, dp_init;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s_init[r] = nlse2;
    dp_init[r] = -delta;
  }
  const int segq = (use_seg && ok) ? segb[row] : 0;
  const int qlast = min(S - 1, q0 + 31);
  int2 wrange = make_int2(0, 0);
  if (use_seg && q0 < S) wrange = seg_range(blkb, a.nblk, q0, min(32, S - q0));

  TileWalk walk;
  const int nk = (S + BK - 1) / BK;  // K/V tiles of BK keys
  if (a.qrange) {
    // the range table counts tiles of kFwdBlockK keys; a tile of BK keys that
    // holds a useful one is useful, so a dense range stays dense
    walk_range(walk, a.qrange[(int64_t)b * a.n_qtiles + qt], blkb);
    walk.lo = walk.lo * kFwdBlockK / BK;
    walk.hi = min(nk, (walk.hi * kFwdBlockK + BK - 1) / BK);
  } else {
    walk.lo = 0;
    walk.hi = a.causal ? min(nk, (min(S, Q0 + BQ) - 1) / BK + 1) : nk;
    walk.blk = nullptr;
  }
  // ring order over chunks of kv_chunk keys, counted in whole tiles of BK
  // keys (rounded down; every tile is visited once either way)
  const int ctk = a.chunk_tiles * kFwdBlockK / BK;
  walk.ct = ctk;
  walk.nc = ctk ? (nk + ctk - 1) / ctk : 1;
  walk.r = ctk ? (Q0 / BK) / ctk : 0;
  walk.dir = -1;
  walk.desc = false;
  walk.nblk = a.nblk;
  walk.rows = BK;
  walk.own = use_seg ? seg_range(blkb, a.nblk, Q0, min(BQ, S - Q0)) : make_int2(0, 0);
  walk.start();

  f32x16 dq[NDG];
#pragma unroll
  for (int dg = 0; dg < NDG; ++dg) dq[dg] = f32x16{};
  const uint16_t* kh = a.k + base;
  const uint16_t* vh = a.v + base;
  TileFill<BK, D / 8, NW, 3> rfill;  // K and V rows
  rfill.init(D * 2, tid);
  auto load = [&](int t, char* buf, int part) {
    if (part != 0) return;  // this kernel issues a tile's loads in one go
    const uint32_t rbytes = (uint32_t)min(S - t * BK, BK) * D * 2;  // rows past S read zero
    rfill.fill(kh + (int64_t)t * BK * D, rbytes, buf);
    rfill.fill(vh + (int64_t)t * BK * D, rbytes, buf + KT::kBytes);
    if (use_seg && w == 0) {
      row64_to_lds(segb, t * BK, S, buf + SEG_OFF, lane);
      row64_to_lds(segb, min(t * BK + 64, S), S, buf + SEG_OFF + 256, lane);
    }
  };
  const int per_tile = 2 * rfill.count() + (use_seg && w == 0 ? 2 : 0);
  auto compute = [&](int t, const char* buf, auto&& issue) {
    const int k0 = t * BK;
    bool skip = q0 >= S || (a.causal && k0 > qlast);
    bool seg_mask = false;
    if (use_seg && !skip) {
      int2 kr = tile128_range(t64b, t);
      if (!ranges_meet(kr, wrange))
        skip = true;
      else
        seg_mask = !(kr.x == kr.y && wrange.x == wrange.y && kr.x == wrange.x);
    }
    if (uniform(skip)) { issue(0); issue(1); }  // a skipped tile still issues this wave's loads
    if (!skip) {
      const char* ktl = buf;
      const char* vtl = buf + KT::kBytes;
      const int* segk_lds = (const int*)(buf + SEG_OFF);
      const bool lim_mask = (k0 + BK > S) || (a.causal && k0 + BK - 1 > q0);
      const bool need_mask = seg_mask || lim_mask;
      const int lim = (a.causal ? min(S - 1, row) : S - 1) - k0 - 4 * hl;  // last visible key, tile-relative
#pragma unroll
      for (int kg = 0; kg < BK / 32; ++kg) {
        f32x16 s = s_init, dp = dp_init;
        lds_mfma_pipe<2 * NDC, 6>(
            [&](int i) { return KT::read((i & 1) ? vtl : ktl, 32 * kg, i >> 1, lane); },
            [&](int i, bf16x8 x) {
              if (i & 1)
                dp = mfma32(x, dop[i >> 1], dp);
              else
                s = mfma32(x, qop[i >> 1], s);
            });
        if (uniform(need_mask)) {
          // key k0 + 32 kg + 8 (r/4) + 4 hl + r%4 in register r; test only
          // what the tile needs
          if (!uniform(seg_mask)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = (32 * kg + 8 * (r >> 2) + (r & 3) <= lim) ? s[r] : kNegInf;
          } else {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int4 sk = *(const int4*)(segk_lds + 32 * kg + 8 * rq + 4 * hl);
              const int sk_[4] = {sk.x, sk.y, sk.z, sk.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool vis = (uniform(lim_mask) ? (32 * kg + 8 * rq + e <= lim) : true) & (sk_[e] == segq);
                s[4 * rq + e] = vis ? s[4 * rq + e] : kNegInf;
              }
            }
          }
        }
        bf16x8 dsk[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r]) * dp[r];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          int r0 = 8 * c;
          dsk[c] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(s[r0], s[r0 + 1]), pack_bf16x2(s[r0 + 2], s[r0 + 3]),
                                                    pack_bf16x2(s[r0 + 4], s[r0 + 5]), pack_bf16x2(s[r0 + 6], s[r0 + 7])});
        }
        // dQ^T += K^T dS^T over the 32 keys of this half
        // K^T operands straight from the K rows: keys 32 kg + 16 c .. in the
        // order dsk[c] holds them
        lds_mfma_pipe<2 * NDG, 6>(
            [&](int i) { return KT::read_tr(ktl, 32 * kg + 16 * (i / NDG), 32 * (i % NDG), lane); },
            [&](int i, bf16x8 x) { dq[i % NDG] = mfma32(x, dsk[i / NDG], dq[i % NDG]); });
        if (kg == BK / 64 - 1) {  // the loads of tile t + 1, in the middle of the tile
          issue(0);
          issue(1);
        }
      }
    }
  };
  run_pipeline_mid<NSTAGE>(walk, per_tile, smem, BUF, load, compute);

  if (ok) {
    if (a.rope) {
      double pos = a.pos ? (double)a.pos[(int64_t)b * S + row] : (double)row;
      rope_backward_row<NDG>(dq, pos, a.turns, hl);
    }
    store_rows<D>(a.dq + base + (int64_t)row * D, dq, a.scale, hl);
  }
}

// ---------------------------------------------------------------------------
// dK/dV: NW waves x 32 keys; tiles of 64 query rows of Q and dO in LDS.  Scores are kept with lane = key: S = Q K^T and
// dP = dO V^T (K and V rows of the lane's key stay in registers), then
// dV^T += dO^T P and dK^T += Q^T dS.
// ---------------------------------------------------------------------------
template <int D, int NW, int NSTAGE>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BKV = kBwdBlockK, BQT = kBwdBlockQ;
  static_assert(BKV == NW * 32, "one 32-key group per wave");
  constexpr int NDC = D / 16, NDG = D / 32;
  using QT = PTile<BQT, D / 8, 3>;  // Q and dO rows (Q^T, dO^T read transposed)
  constexpr int SB = 2 * QT::kBytes;  // row statistics: -LSE log2e [BQT], -Delta [BQT], seg [BQT]
  constexpr int BUF = SB + 3 * 4 * BQT;
  static_assert(BQT == 128, "statistics fetched as two 64-row runs");
  // ring of [Q, dO, statistics] stages (see run_pipeline)
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * BUF];

  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_bkv, bh, rank);
  const int kt_idx = rank;  // causal work shrinks with the key tile index: low tiles first
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int K0 = kt_idx * BKV;
  const int j0 = K0 + 32 * w;  // this wave's first key
  const int j = j0 + l32;      // this lane's key
  const bool jok = j < S;
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;
  const int2* t64b = use_seg ? a.t64 + (int64_t)b * a.n64p : nullptr;

  bf16x8 kop[NDC], vop[NDC];
  {
    int64_t ro = base + (int64_t)min(j, S - 1) * D + 8 * hl;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      bf16x8 kv = *(const bf16x8*)(a.k + ro + 16 * dc);
      bf16x8 vv = *(const bf16x8*)(a.v + ro + 16 * dc);
      kop[dc] = jok ? kv : bf16x8{};
      vop[dc] = jok ? vv : bf16x8{};
    }
  }
  const int segk = (use_seg && jok) ? segb[j] : 0;
  int2 wrange = make_int2(0, 0);
  if (use_seg && j0 < S) wrange = seg_range(blkb, a.nblk, j0, min(32, S - j0));
  wrange = make_int2(uniform(wrange.x), uniform(wrange.y));

  TileWalk walk;
  if (a.krange) {
    walk_range(walk, a.krange[(int64_t)b * a.n_bkv + kt_idx], blkb);
  } else {
    walk.lo = a.causal ? K0 / BQT : 0;
    walk.hi = a.n_bq;
    walk.blk = nullptr;
  }
  // ring order over chunks of kv_chunk rows, counted in whole tiles of BQT
  // rows (rounded down: a kv_chunk of 64 rows walks in natural order, an odd
  // multiple of 64 in chunks one half tile short; every tile is visited once)
  const int ctq = a.chunk_tiles * kFwdBlockK / BQT;
  walk.ct = ctq;  // a chunk of kv_chunk rows is kv_chunk / 64 tiles on both sides
  walk.nc = ctq ? (a.n_bq + ctq - 1) / ctq : 1;
  walk.r = ctq ? (K0 / BQT) / ctq : 0;
  walk.dir = +1;
  // natural order: from the last query tile down, so that workgroups of one
  // head stream the same Q/dO tiles at the same time (L2 reuse)
  walk.desc = true;
  walk.nblk = a.nblk;
  walk.rows = BQT;
  walk.own = use_seg ? seg_range(blkb, a.nblk, K0, min(BKV, S - K0)) : make_int2(0, 0);
  walk.start();

  f32x16 dk[NDG], dv[NDG];
#pragma unroll
  for (int dg = 0; dg < NDG; ++dg) dk[dg] = dv[dg] = f32x16{};
  const uint16_t* qh = a.q + base;
  const uint16_t* dh = a.dout + base;
  const float* nlse_h = a.nlse2 + (int64_t)bh * S;
  const float* ndel_h = a.ndelta + (int64_t)bh * S;

  // tiles of a Q block and its row statistics (-LSE log2(e), -Delta,
  // segment id), the statistics fetched by wave 0
  TileFill<BQT, D / 8, NW, 3> rfill;  // Q and dO rows
  rfill.init(D * 2, tid);
  auto load = [&](int t, char* buf, int part) {
    const uint32_t rbytes = (uint32_t)min(S - t * BQT, BQT) * D * 2;  // rows past S read zero
    if (part == 0) {
      rfill.fill(qh + (int64_t)t * BQT * D, rbytes, buf);
      return;
    }
    rfill.fill(dh + (int64_t)t * BQT * D, rbytes, buf + QT::kBytes);
    // statistics: wave 0 -LSE log2e, wave 1 -Delta, wave 2 the segment ids
    if (w == 0) {
      row64_to_lds(nlse_h, t * BQT, S, buf + SB, lane);
      row64_to_lds(nlse_h, min(t * BQT + 64, S), S, buf + SB + 256, lane);
    } else if (w == 1) {
      row64_to_lds(ndel_h, t * BQT, S, buf + SB + 4 * BQT, lane);
      row64_to_lds(ndel_h, min(t * BQT + 64, S), S, buf + SB + 4 * BQT + 256, lane);
    } else if (w == 2 && use_seg) {
      row64_to_lds(segb, t * BQT, S, buf + SB + 8 * BQT, lane);
      row64_to_lds(segb, min(t * BQT + 64, S), S, buf + SB + 8 * BQT + 256, lane);
    }
  };
  const int per_tile = 2 * rfill.count() + ((w == 0 || w == 1 || (w == 2 && use_seg)) ? 2 : 0);
  auto compute = [&](int t, const char* buf, auto&& issue) {
    const int i0 = t * BQT;
    const int ilast = min(S - 1, i0 + BQT - 1);
    bool skip = j0 >= S || (a.causal && ilast < j0);
    bool seg_mask = false;
    if (use_seg && !skip) {
      int2 qr = tile128_range(t64b, t);
      if (!ranges_meet(qr, wrange))
        skip = true;
      else
        seg_mask = !(qr.x == qr.y && wrange.x == wrange.y && qr.x == wrange.x);
    }
    if (uniform(skip)) { issue(0); issue(1); }  // a skipped tile still issues this wave's loads
    if (!skip) {
      const char* qtl = buf;
      const char* dtl = buf + QT::kBytes;
      const float* st = (const float*)(buf + SB);
      // the per-lane LDS offsets are re-formed per tile: kept live across the
      // loop they would be spilled, and their reload's vmcnt wait would also
      // wait for the next tile's loads
      const int ln = opaque(lane);
      const bool need_mask = seg_mask || (i0 + BQT > S) || (a.causal && i0 < j0 + 31);
#pragma unroll
      for (int qg = 0; qg < BQT / 32; ++qg) {
        // S[i][j] and dP[i][j] for rows i = i0 + 32 qg + 8 (r/4) + 4 hl + r%4.
        // The MFMAs start from the rows' statistics: S (whose query operand
        // carries scale * log2(e)) from -LSE log2(e), dP from -Delta, so they
        // leave the exponent of exp2 and dP - Delta
        f32x16 s, dp;
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int ri = 32 * qg + 8 * rq + 4 * hl;
          const f32x4 nl = *(const f32x4*)(st + ri);
          const f32x4 nd = *(const f32x4*)(st + BQT + ri);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[4 * rq + e] = nl[e];
            dp[4 * rq + e] = nd[e];
          }
        }
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          bf16x8 qa = QT::read(qtl, 32 * qg, dc, ln);
          bf16x8 da = QT::read(dtl, 32 * qg, dc, ln);
          s = mfma32(qa, kop[dc], s);
          dp = mfma32(da, vop[dc], dp);
        }
        if (need_mask) {
          // rows i0 + 32 qg + 8 rq + 4 hl + e in registers s[4 rq + e]; their
          // segment ids, when the tile needs them, read four at a time
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int ri = 32 * qg + 8 * rq + 4 * hl;
            int4 sq = make_int4(segk, segk, segk, segk);
            if (uniform(seg_mask)) sq = *(const int4*)((const int*)st + 2 * BQT + ri);
            const int sq_[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = i0 + ri + e;
              const bool vis = i < S && (!a.causal || j <= i) && sq_[e] == segk;
              s[4 * rq + e] = vis ? s[4 * rq + e] : kNegInf;
            }
          }
        }
        // P = exp(S scale - LSE) and dS = P (dP - Delta)
        bf16x8 pk[2], dsk[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          uint32_t pw[4], dw[4];
#pragma unroll
          for (int hq = 0; hq < 2; ++hq) {
            const int rq = 2 * c + hq;
            float pv[4], dsv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pv[e] = fast_exp2(s[4 * rq + e]);
              dsv[e] = pv[e] * dp[4 * rq + e];
            }
            pw[2 * hq] = pack_bf16x2(pv[0], pv[1]);
            pw[2 * hq + 1] = pack_bf16x2(pv[2], pv[3]);
            dw[2 * hq] = pack_bf16x2(dsv[0], dsv[1]);
            dw[2 * hq + 1] = pack_bf16x2(dsv[2], dsv[3]);
          }
          pk[c] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
          dsk[c] = __builtin_bit_cast(bf16x8, u32x4{dw[0], dw[1], dw[2], dw[3]});
        }
        // dV^T += dO^T P, dK^T += Q^T dS over these 32 rows
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg) {
            // dO^T and Q^T from the row tiles: rows 32 qg + 16 c .. in the
            // order pk[c] and dsk[c] hold them
            bf16x8 dta = QT::read_tr(dtl, 32 * qg + 16 * c, 32 * dg, ln);
            bf16x8 qta = QT::read_tr(qtl, 32 * qg + 16 * c, 32 * dg, ln);
            dv[dg] = mfma32(dta, pk[c], dv[dg]);
            dk[dg] = mfma32(qta, dsk[c], dk[dg]);
          }
        }
        // the loads of tile t + 1 in two parts, Q after the first 32 rows and
        // dO with the statistics after the second: one burst of every wave's
        // loads stalled each wave longer (dK/dV -1% split)
        if (qg == 0) issue(0);
        if (qg == 1) issue(1);
      }
    }
  };
  run_pipeline_mid<NSTAGE>(walk, per_tile, smem, BUF, load, compute);

  if (jok) {
    if (a.rope) {
      double pos = a.pos ? (double)a.pos[(int64_t)b * S + j] : (double)j;
      rope_backward_row<NDG>(dk, pos, a.turns, hl);
    }
    store_rows<D>(a.dk + base + (int64_t)j * D, dk, a.dk_scale, hl);  // Q^T dS used the scaled query rows
    store_rows<D>(a.dv + base + (int64_t)j * D, dv, 1.f, hl);
  }
}

hipError_t launch_attn_bwd_dq(const BwdArgs& a, int D, hipStream_t st) {
  constexpr int NW = 8, NSTAGE = 2;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_qtiles)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<128, NW, NSTAGE>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<64, NW, NSTAGE>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const BwdArgs& a, int D, hipStream_t st) {
  constexpr int NW = 8, NSTAGE = 2;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_bkv)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<128, NW, NSTAGE>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<64, NW, NSTAGE>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
