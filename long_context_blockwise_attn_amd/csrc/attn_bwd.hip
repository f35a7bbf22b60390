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
//    streams K/V tiles; it also forms Delta for its rows.  3 contractions per
//    tile pair (S, dP, dQ).
//  - dK/dV kernel: a workgroup owns kBwdBlockK keys and streams Q/dO tiles of
//    64 rows.  4 contractions per tile pair (S, dP, dV, dK).
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
// dQ (and Delta): 4 waves x 64 query rows; K/V tiles of 64 keys in LDS.
// Per 32-key half: S^T = K Q^T and dP^T = V dO^T (lane = query row), then
// dS^T = P^T (dP^T - Delta) and dQ^T += K^T dS^T with K^T from the
// transposing LDS read.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int BQ = kFwdBlockQ, BK = kFwdBlockK, QG = 2;
  constexpr int NDC = D / 16, NDG = D / 32;
  constexpr int TB = BK * D * 2;
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[4 * TB];  // [buffer][K, V]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_qtiles, bh, rank);
  const int qt = a.n_qtiles - 1 - rank;
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int Q0 = qt * BQ;
  const int q0 = Q0 + w * 64;
  const int qlast = min(S - 1, q0 + 63);
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;

  bf16x8 qop[QG][NDC], dop[QG][NDC];
  int segq[QG];
  float nlse2[QG], delta[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    int row = q0 + 32 * qg + l32;
    bool ok = row < S;
    int64_t ro = base + (int64_t)min(row, S - 1) * D + 8 * hl;
    float dsum = 0.f;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      bf16x8 qv = *(const bf16x8*)(a.q + ro + 16 * dc);
      u32x4 dv = *(const u32x4*)(a.dout + ro + 16 * dc);
      u32x4 ov = *(const u32x4*)(a.o + ro + 16 * dc);
      qop[qg][dc] = ok ? qv : bf16x8{};
      dop[qg][dc] = ok ? __builtin_bit_cast(bf16x8, dv) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dsum += bf16_lo(dv[e]) * bf16_lo(ov[e]) + bf16_hi(dv[e]) * bf16_hi(ov[e]);
    }
    dsum = pair_sum(dsum);
    delta[qg] = ok ? dsum : 0.f;
    if (ok && hl == 0) a.delta[(int64_t)bh * S + row] = dsum;
    nlse2[qg] = ok ? -a.lse[(int64_t)bh * S + row] * kLog2e : 0.f;
    segq[qg] = (use_seg && ok) ? segb[row] : 0;
  }
  int2 wrange = make_int2(0, 0);
  if (use_seg && q0 < S) wrange = seg_range(blkb, a.nblk, q0, min(64, S - q0));

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
  walk.blk = blkb;
  walk.nblk = a.nblk;
  walk.rows = BK;
  walk.own = use_seg ? seg_range(blkb, a.nblk, Q0, min(BQ, S - Q0)) : make_int2(0, 0);
  walk.start();

  f32x16 dq[QG][NDG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg) dq[qg][dg] = f32x16{};
  const float sl2 = a.scale_log2;
  const uint16_t* kh = a.k + base;
  const uint16_t* vh = a.v + base;

  if (walk.t >= 0) {
    tile_to_lds<D, 256>(kh, walk.t * BK, S, smem, tid);
    tile_to_lds<D, 256>(vh, walk.t * BK, S, smem + TB, tid);
  }
  wait_loads();
  __syncthreads();
  int buf = 0;
  while (walk.t >= 0) {
    TileWalk nx = walk;
    nx.next();
    if (nx.t >= 0) {
      char* nb = smem + (buf ^ 1) * 2 * TB;
      tile_to_lds<D, 256>(kh, nx.t * BK, S, nb, tid);
      tile_to_lds<D, 256>(vh, nx.t * BK, S, nb + TB, tid);
    }
    const int k0 = walk.t * BK;
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
      const char* kt = smem + buf * 2 * TB;
      const char* vt = kt + TB;
      const bool need_mask = seg_mask || (k0 + BK > S) || (a.causal && k0 + BK - 1 > q0);
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        f32x16 s[QG], dp[QG];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) s[qg] = dp[qg] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          bf16x8 ka = T::read_rows(kt, 32 * kg, dc, lane);
          bf16x8 va = T::read_rows(vt, 32 * kg, dc, lane);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            s[qg] = mfma32(ka, qop[qg][dc], s[qg]);
            dp[qg] = mfma32(va, dop[qg][dc], dp[qg]);
          }
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int j = k0 + 32 * kg + 8 * (r >> 2) + 4 * hl + (r & 3);
            int sk = (seg_mask && j < S) ? segb[j] : 0;
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
              int i = q0 + 32 * qg + l32;
              bool vis = j < S && (!a.causal || j <= i) && (!seg_mask || sk == segq[qg]);
              s[qg][r] = vis ? s[qg][r] : kNegInf;
            }
          }
        }
        bf16x8 dsk[QG][2];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(__builtin_fmaf(s[qg][r], sl2, nlse2[qg]));
            s[qg][r] = p * (dp[qg][r] - delta[qg]);
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            int r0 = 8 * c;
            uint32_t w0 = pack_bf16x2(s[qg][r0 + 0], s[qg][r0 + 1]);
            uint32_t w1 = pack_bf16x2(s[qg][r0 + 2], s[qg][r0 + 3]);
            uint32_t w2 = pack_bf16x2(s[qg][r0 + 4], s[qg][r0 + 5]);
            uint32_t w3 = pack_bf16x2(s[qg][r0 + 6], s[qg][r0 + 7]);
            dsk[qg][c] = __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
          }
        }
        // dQ^T += K^T dS^T over the 32 keys of this half
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg) {
            bf16x8 kta = T::read_cols(kt, 32 * kg + 16 * c, 32 * dg, lane);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) dq[qg][dg] = mfma32(kta, dsk[qg][c], dq[qg][dg]);
          }
        }
      }
    }
    wait_loads();
    __syncthreads();
    buf ^= 1;
    walk = nx;
  }

#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    int row = q0 + 32 * qg + l32;
    if (row < S) {
      if (a.rope) {
        double pos = a.pos ? (double)a.pos[(int64_t)b * S + row] : (double)row;
        rope_backward_row<NDG>(dq[qg], pos, a.turns, hl);
      }
      store_rows<D>(a.dq + base + (int64_t)row * D, dq[qg], a.scale, hl);
    }
  }
}

// ---------------------------------------------------------------------------
// dK/dV: NW waves x 32 keys; Q/dO tiles of 64 rows in LDS.  Scores are kept
// with lane = key: S = Q K^T and dP = dO V^T (K and V rows of the wave stay
// in registers), then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T
// from the transposing LDS read.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 4, BKV = kBwdBlockK, BQT = kBwdBlockQ;
  static_assert(BKV == NW * 32, "one 32-key group per wave");
  constexpr int NDC = D / 16, NDG = D / 32;
  constexpr int TB = BQT * D * 2;
  constexpr int SB = 4 * TB;         // row statistics after the four tiles
  using T = Tile<D>;
  // [buffer][Q, dO] tiles, then per buffer: LSE[64], Delta[64], seg[64]
  __shared__ __attribute__((aligned(16))) char smem[4 * TB + 2 * 3 * 256];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  int bh, rank;
  xcd_tile_order(blockIdx.x, a.B * a.H, a.n_bkv, bh, rank);
  // causal work shrinks with the key tile index: low tiles first
  const int kt_idx = rank;
  const int b = bh / a.H;
  const int S = a.S;
  const int64_t base = (int64_t)bh * S * D;
  const int K0 = kt_idx * BKV;
  const int j0 = K0 + 32 * w;         // this wave's first key
  const int j = j0 + l32;             // this lane's key
  const bool jok = j < S;
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;

  // K and V rows of this lane's key as B operands (k along d)
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

  TileWalk walk;
  if (a.krange) {
    int2 r = a.krange[(int64_t)b * a.n_bkv + kt_idx];
    walk.lo = r.x;
    walk.hi = r.y;
  } else {
    walk.lo = a.causal ? K0 / BQT : 0;
    walk.hi = a.n_bq;
  }
  walk.ct = a.chunk_tiles;  // a chunk of kv_chunk rows is kv_chunk / 64 tiles on both sides
  walk.nc = a.chunk_tiles ? (a.n_bq + a.chunk_tiles - 1) / a.chunk_tiles : 1;
  walk.r = a.chunk_tiles ? (K0 / BQT) / a.chunk_tiles : 0;
  walk.dir = +1;
  walk.blk = blkb;
  walk.nblk = a.nblk;
  walk.rows = BQT;
  walk.own = use_seg ? seg_range(blkb, a.nblk, K0, min(BKV, S - K0)) : make_int2(0, 0);
  walk.start();

  f32x16 dk[NDG], dv[NDG];
#pragma unroll
  for (int dg = 0; dg < NDG; ++dg) dk[dg] = dv[dg] = f32x16{};
  const float sl2 = a.scale_log2;
  const uint16_t* qh = a.q + base;
  const uint16_t* dh = a.dout + base;
  const float* lse_h = a.lse + (int64_t)bh * S;
  const float* del_h = a.delta + (int64_t)bh * S;

  // row statistics of a Q tile (LSE, Delta, segment id of its 64 rows),
  // fetched by wave 0 straight into LDS
  auto load_stats = [&](int t, int bsel) {
    if (w == 0) {
      int i = min(t * BQT + lane, S - 1);
      char* st = smem + SB + bsel * 768;
      __builtin_amdgcn_global_load_lds((const void*)(lse_h + i), (__attribute__((address_space(3))) void*)(st), 4, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(del_h + i), (__attribute__((address_space(3))) void*)(st + 256), 4, 0, 0);
      if (use_seg)
        __builtin_amdgcn_global_load_lds((const void*)(segb + i), (__attribute__((address_space(3))) void*)(st + 512), 4, 0, 0);
    }
  };

  if (walk.t >= 0) {
    tile_to_lds<D, 256>(qh, walk.t * BQT, S, smem, tid);
    tile_to_lds<D, 256>(dh, walk.t * BQT, S, smem + TB, tid);
    load_stats(walk.t, 0);
  }
  wait_loads();
  __syncthreads();
  int buf = 0;
  while (walk.t >= 0) {
    TileWalk nx = walk;
    nx.next();
    if (nx.t >= 0) {
      char* nb = smem + (buf ^ 1) * 2 * TB;
      tile_to_lds<D, 256>(qh, nx.t * BQT, S, nb, tid);
      tile_to_lds<D, 256>(dh, nx.t * BQT, S, nb + TB, tid);
      load_stats(nx.t, buf ^ 1);
    }
    const int i0 = walk.t * BQT;
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
    if (!skip) {
      const char* qtl = smem + buf * 2 * TB;
      const char* dtl = qtl + TB;
      const float* st = (const float*)(smem + SB + buf * 768);
      const bool need_mask = seg_mask || (i0 + BQT > S) || (a.causal && i0 < j0 + 31);
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        // S[i][j] and dP[i][j] for 32 rows i = i0 + 32 qg + 8 (r/4) + 4 hl + r%4
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          bf16x8 qa = T::read_rows(qtl, 32 * qg, dc, lane);
          bf16x8 da = T::read_rows(dtl, 32 * qg, dc, lane);
          s = mfma32(qa, kop[dc], s);
          dp = mfma32(da, vop[dc], dp);
        }
        f32x4 nl[4], de[4];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          int ri = 32 * qg + 8 * rq + 4 * hl;
          nl[rq] = *(const f32x4*)(st + ri) * -kLog2e;
          de[rq] = *(const f32x4*)(st + 64 + ri);
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int ri = 32 * qg + 8 * (r >> 2) + 4 * hl + (r & 3);
            int i = i0 + ri;
            int sq = ((const int*)st)[128 + ri];
            bool vis = i < S && (!a.causal || j <= i) && (!seg_mask || sq == segk);
            s[r] = vis ? s[r] : kNegInf;
          }
        }
        bf16x8 pk[2], dsk[2];
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], sl2, nl[r >> 2][r & 3]));
          pv[r] = p;
          s[r] = p * (dp[r] - de[r >> 2][r & 3]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          int r0 = 8 * c;
          pk[c] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(pv[r0], pv[r0 + 1]), pack_bf16x2(pv[r0 + 2], pv[r0 + 3]),
                                                   pack_bf16x2(pv[r0 + 4], pv[r0 + 5]), pack_bf16x2(pv[r0 + 6], pv[r0 + 7])});
          dsk[c] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(s[r0], s[r0 + 1]), pack_bf16x2(s[r0 + 2], s[r0 + 3]),
                                                    pack_bf16x2(s[r0 + 4], s[r0 + 5]), pack_bf16x2(s[r0 + 6], s[r0 + 7])});
        }
        // dV^T += dO^T P, dK^T += Q^T dS over these 32 rows
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg) {
            bf16x8 dta = T::read_cols(dtl, 32 * qg + 16 * c, 32 * dg, lane);
            bf16x8 qta = T::read_cols(qtl, 32 * qg + 16 * c, 32 * dg, lane);
            dv[dg] = mfma32(dta, pk[c], dv[dg]);
            dk[dg] = mfma32(qta, dsk[c], dk[dg]);
          }
        }
      }
    }
    wait_loads();
    __syncthreads();
    buf ^= 1;
    walk = nx;
  }

  if (jok) {
    if (a.rope) {
      double pos = a.pos ? (double)a.pos[(int64_t)b * S + j] : (double)j;
      rope_backward_row<NDG>(dk, pos, a.turns, hl);
    }
    store_rows<D>(a.dk + base + (int64_t)j * D, dk, a.scale, hl);
    store_rows<D>(a.dv + base + (int64_t)j * D, dv, 1.f, hl);
  }
}

hipError_t launch_attn_bwd_dq(const BwdArgs& a, int D, hipStream_t st) {
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_qtiles)), block(256);
  if (D == 128)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const BwdArgs& a, int D, hipStream_t st) {
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_bkv)), block(256);
  if (D == 128)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
