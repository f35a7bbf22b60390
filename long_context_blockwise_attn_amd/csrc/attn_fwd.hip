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
// (batch, head); each wave owns 32 rows.  Each lane rotates its query row
// (RoPE) and multiplies it by scale * log2(e) as it loads it, and the score
// MFMAs start from -m, the row's running max, so they leave
// scale * log2(e) * <q', k'> - m, the exponent of exp2 itself.  Tiles of 64 keys of K and V rows sit
// in an NSTAGE-deep LDS ring filled by buffer-to-LDS loads.  Scores are
// computed transposed, S^T = K Q^T, so each lane holds one query row: the row
// max needs one exchange between lanes l and l^32, and the running rescale of
// O is a per-lane scalar.  O^T = V^T P^T takes P^T straight from the score
// registers; its V^T operand is read from the V rows with transposing LDS
// reads (PTile::read_tr), which deliver the keys in the order the score
// registers hold them, so no transposed copy of V is made.
//
// Two wave groups run one phase apart (ping-pong, below): on every SIMD one
// wave issues the matrix phase (S^T of the next tile, O^T += V^T P^T) while
// the other runs the vector phase (mask, max, lazy rescale, softmax).
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace bwattn {

template <int D, int NW, int NSTAGE>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdArgs a) {
  constexpr int BQ = kFwdBlockQ, BK = kFwdBlockK;
  static_assert(BQ == NW * 32, "32 query rows per wave");
  static_assert(BK == 64, "two 32-key halves per tile");
  static_assert(NSTAGE >= 3, "K of tile t+1 and V of tile t are read in the same step");
  constexpr int NDC = D / 16;  // 16-wide k steps over D for S^T
  constexpr int NDG = D / 32;  // 32-row groups of O^T over D
  constexpr float kLazy = 8.f;
  using KT = PTile<BK, D / 8>;  // K rows
  // V rows (V^T read transposed).  P = 4 would make these reads conflict-free
  // but measured no faster: its two extra pad chunks per row lengthen the loads.
  using VR = PTile<BK, D / 8, 2>;
  constexpr int SEG_OFF = KT::kBytes + VR::kBytes;  // segment ids of the tile's keys
  constexpr int BUF = SEG_OFF + 256;
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
  const int q0 = Q0 + w * 32;
  const int row = q0 + l32;  // this lane's query row
  const bool use_seg = a.seg != nullptr;
  const int32_t* segb = use_seg ? a.seg + (int64_t)b * S : nullptr;
  const int2* blkb = use_seg ? a.blk + (int64_t)b * a.nblk : nullptr;
  const int2* t64b = use_seg ? a.t64 + (int64_t)b * a.n64p : nullptr;

  // Q operand (B of S^T = K Q^T): lane holds row `row`, d = 16 dc + 8 hl + [0,8),
  // that is the pairs 8 dc + 4 hl + [0,4), rotated to the row's position and
  // times scale * log2(e) (the same bits the RoPE pre-pass writes)
  bf16x8 qop[NDC];
  {
    const int r = min(row, S - 1);
    const uint16_t* src = a.q + base + (int64_t)r * D + 8 * hl;
    const double pos = a.pos ? (double)a.pos[(int64_t)b * S + r] : (double)r;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const u32x4 x = *(const u32x4*)(src + 16 * dc);
      u32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float c, s;
        rope_cos_sin(pos, a.turns[8 * dc + 4 * hl + e], c, s);
        y[e] = rope_pair(x[e], c, s, a.q_scale);
      }
      qop[dc] = row < S ? __builtin_bit_cast(bf16x8, y) : bf16x8{};
    }
  }
  const int segq = (use_seg && row < S) ? segb[row] : 0;
  const int segsel = use_seg ? -1 : 0;  // the LDS segment ids are ignored without packing
  int2 wrange = make_int2(0, 0);
  if (use_seg && q0 < S) wrange = seg_range(blkb, a.nblk, q0, min(32, S - q0));

  // K/V tile range and walk
  TileWalk walk;
  if (a.qrange) {
    walk_range(walk, a.qrange[(int64_t)b * a.n_qtiles + qt], blkb);
  } else {
    walk.lo = 0;
    walk.hi = a.causal ? min(a.n_ktiles, (min(S, Q0 + BQ) - 1) / BK + 1) : a.n_ktiles;
    walk.blk = nullptr;
  }
  walk.ct = a.chunk_tiles;
  walk.nc = a.chunk_tiles ? (a.n_ktiles + a.chunk_tiles - 1) / a.chunk_tiles : 1;
  walk.r = a.chunk_tiles ? (Q0 / BK) / a.chunk_tiles : 0;
  walk.dir = -1;
  walk.desc = false;
  walk.nblk = a.nblk;
  walk.rows = BK;
  walk.own = use_seg ? seg_range(blkb, a.nblk, Q0, min(BQ, S - Q0)) : make_int2(0, 0);
  walk.start();

  float m = kNegInf, lsum = 0.f;  // running max (log2 units) and sum
  f32x16 negm = f32x16{};          // -m in every register (0 while m = -inf)
  f32x16 o[NDG];
#pragma unroll
  for (int dg = 0; dg < NDG; ++dg) o[dg] = f32x16{};

  const uint16_t* kh = a.k + base;
  const uint16_t* vh = a.v + base;
  TileFill<BK, D / 8, NW> kfill;     // K rows
  TileFill<BK, D / 8, NW, 2> vfill;  // V rows
  kfill.init(D * 2, tid);
  vfill.init(D * 2, tid);
  auto load = [&](int t, char* buf) {
    const uint32_t rbytes = (uint32_t)min(S - t * BK, BK) * D * 2;  // rows past S read zero
    kfill.fill(kh + (int64_t)t * BK * D, rbytes, buf);
    vfill.fill(vh + (int64_t)t * BK * D, rbytes, buf + KT::kBytes);
    if (use_seg && w == 0) row64_to_lds(segb, t * BK, S, buf + SEG_OFF, lane);
  };
  // vector-memory instructions this wave issues per tile
  const int per_tile = kfill.count() + vfill.count() + (use_seg && w == 0 ? 1 : 0);
  // the fewest any wave issues: a compile-time wait count.  Waiting until
  // that many are in flight completes the wave's loads of the older of two
  // positions (a wave with more loads also waits for a few of the newer
  // position, issued a step earlier); a wait on the exact count would need a
  // branch table, whose scalar code cost ~3% of the forward's time.
  constexpr int kLeastPerTile = KT::kBlocks / NW + VR::kBlocks / NW;

  // --- per-tile pieces -----------------------------------------------------
  // S^T - m of the tile in `buf` (log2 units): s[kg] holds keys
  // k0 + 32 kg + 8 (r/4) + 4 hl + r%4
  auto scores = [&](const char* buf, f32x16 (&s)[2]) {
    s[0] = s[1] = negm;
    lds_mfma_pipe<2 * NDC, 3>([&](int i) { return KT::read(buf, 32 * (i & 1), i >> 1, lane); },
                              [&](int i, bf16x8 x) { s[i & 1] = mfma32(x, qop[i >> 1], s[i & 1]); });
  };
  // causal / segment / sequence-end mask of tile t.  The decisions are
  // wave-uniform, and a tile tests only what it needs: the position limit
  // (diagonal, sequence end), the segment ids (document edge), or both.
  auto mask = [&](int t, const char* buf, f32x16 (&s)[2]) {
    const int k0 = t * BK;
    bool seg_mask = false;
    if (use_seg) {
      int2 kr = tile64_range(t64b, t);
      seg_mask = !(kr.x == kr.y && wrange.x == wrange.y && kr.x == wrange.x);
    }
    const bool lim_mask = (k0 + BK > S) || (a.causal && k0 + BK - 1 > q0);
    if (uniform(seg_mask || lim_mask)) {
      const int* segk = (const int*)(buf + SEG_OFF);
      const int lim = (a.causal ? min(S - 1, row) : S - 1) - k0 - 4 * hl;  // last visible key, tile-relative
      // keys k0 + 32 kg + 8 rq + 4 hl + e in registers s[kg][4 rq + e]
      if (!uniform(seg_mask)) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kg][r] = (32 * kg + 8 * (r >> 2) + (r & 3) <= lim) ? s[kg][r] : kNegInf;
      } else {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int jj = 32 * kg + 8 * rq + 4 * hl;
            const int4 sk = *(const int4*)(segk + jj);
            const int sk_[4] = {sk.x, sk.y, sk.z, sk.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool vis = (uniform(lim_mask) ? (32 * kg + 8 * rq + e <= lim) : true) & (sk_[e] == segq);
              s[kg][4 * rq + e] = vis ? s[kg][4 * rq + e] : kNegInf;
            }
          }
      }
    }
  };
  // Row max of a tile's scores, relative to m (to 0 while m = -inf), in four
  // independent chains: with the other wave of the SIMD issuing MFMAs, one
  // dependent chain of 16 steps left this wave idle between them.
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) mc[c] = fmaxf(s[c >> 1][8 * (c & 1)], s[c >> 1][8 * (c & 1) + 1]);
#pragma unroll
    for (int e = 2; e < 8; e += 2)
#pragma unroll
      for (int c = 0; c < 4; ++c) mc[c] = fmaxf(fmaxf(mc[c], s[c >> 1][8 * (c & 1) + e]), s[c >> 1][8 * (c & 1) + e + 1]);
    return pair_max(fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3])));
  };
  // Lazy online-softmax max update.  A row's running max m is raised only
  // when its new max exceeds it by more than kLazy (log2 units); otherwise
  // the stale m stays, p <= 2^kLazy, and O is not touched.  l and O share m,
  // so the normalised result is unchanged.  The decision is per row (the
  // wave only branches when some row needs it), so a row's result depends on
  // its own visible keys alone.  A raised m moves the tile's scores by the
  // rise and the start value of later tiles' score MFMAs with it.
  auto rescale = [&](float mx, f32x16 (&s)[2]) {
    const bool grow = mx > (m == kNegInf ? kNegInf : kLazy);
    if (__ballot(grow)) {
      const float rise = grow ? mx : 0.f;
      const float mnew = grow ? (m == kNegInf ? mx : m + mx) : m;
      const float alpha = fast_exp2(grow ? m - mnew : 0.f);  // 0 from m = -inf, where l and O are 0
      lsum *= alpha;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) o[dg] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[0][r] -= rise;
        s[1][r] -= rise;
      }
      m = mnew;
      const float nm = (m == kNegInf) ? 0.f : -m;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = nm;
    }
  };
  // P = 2^(S*scale*log2e - m) as bf16 MFMA operands pk[kc] (keys 16 kc ..),
  // and the row sum over the same bf16 values (one chain per kc)
  auto softmax = [&](const f32x16 (&s)[2], bf16x8 (&pk)[4]) {
    float rsc[4] = {lsum, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      float rs = rsc[kc];
      const int r0 = 8 * (kc & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(s[kc >> 1][r0 + e]);
      u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                  pack_bf16x2(p[6], p[7])};
#pragma unroll
      for (int e = 0; e < 4; ++e) rs = dot2_bf16(pw[e], kBf16OnePair, rs);
      rsc[kc] = rs;
      pk[kc] = __builtin_bit_cast(bf16x8, pw);
    }
    lsum = (rsc[0] + rsc[1]) + (rsc[2] + rsc[3]);
  };
  auto pv = [&](const char* buf, const bf16x8 (&pk)[4]) {
    // V^T operand for keys 16 kc .. 16 kc + 15 (the keys of pk[kc]) and d 32 dg ..
    const char* vr = buf + KT::kBytes;
    lds_mfma_pipe<4 * NDG, 3>([&](int i) { return VR::read_tr(vr, 16 * (i / NDG), 32 * (i % NDG), lane); },
                              [&](int i, bf16x8 x) { o[i % NDG] = mfma32(x, pk[i / NDG], o[i % NDG]); });
  };

  // --- ping-pong pipeline -------------------------------------------------
  // Waves 0-3 and 4-7 form two groups with one wave of each on every SIMD.
  // Each step has a matrix phase (S^T of tile k+1, O^T += V^T P^T of tile k)
  // and a vector phase (mask, max, rescale and softmax of tile k+1).  Group 1
  // runs one barrier behind group 0, so on every SIMD one wave issues MFMAs
  // while the other runs the softmax, and they swap at each barrier.
  // Barrier G_j: group 0 runs the matrix phase of step k between G_2k and
  // G_2k+1, group 1 between G_2k+1 and G_2k+2.  Tile position p lives in ring
  // slot p % 4; it is read from G_2p-2 (K of p in the matrix phase of step
  // p-1) until G_2p+2 (V of p in group 1's matrix phase of step p).  So each
  // wave issues position k+4 right after G_2k+2 and, before G_2k+2, waits for
  // its loads of position k+2 (only k+3 may still be in flight).
  static_assert(NW == 8 && NSTAGE == 4, "two groups of four waves, four-slot ring");
  const int grp = uniform(w >> 2);
  auto slot = [&](int p) { return smem + (p & (NSTAGE - 1)) * BUF; };
  if (walk.t >= 0) {
    TileWalk w1 = walk;  // position k + 1
    w1.next();
    TileWalk ahead = w1;  // newest position issued
    load(uniform(walk.t), slot(0));
    int pend = 0;
    if (w1.t >= 0) {
      load(uniform(w1.t), slot(1));
#pragma unroll
      for (int p = 2; p < NSTAGE; ++p) {
        if (ahead.t >= 0) ahead.next();
        if (ahead.t >= 0) {
          load(uniform(ahead.t), slot(p));
          ++pend;
        }
      }
    }
    int ahead_pos = 1 + pend;  // position of `ahead` when it is valid
    wait_vmem_le(pend * per_tile);
    __syncthreads();  // G_0

    bf16x8 pk[4];
    {
      f32x16 s0[2];
      scores(slot(0), s0);
      mask(uniform(walk.t), slot(0), s0);
      rescale(tile_max(s0), s0);
      softmax(s0, pk);
    }
    if (grp == 1) __syncthreads();  // G_1: group 1 starts one phase later

    // wait for position k+2 (k+3 may be in flight), barrier, issue k+4
    auto refill = [&](int k) {
      if (ahead.t >= 0 && ahead_pos >= k + 3)
        wait_vmem_le<kLeastPerTile>();
      else
        wait_vmem_le<0>();
      __syncthreads();
      if (ahead.t >= 0) ahead.next();
      if (ahead.t >= 0) {
        ++ahead_pos;
        load(uniform(ahead.t), slot(ahead_pos));
      }
    };

    int k = 0;
    while (walk.t >= 0) {
      const bool more = w1.t >= 0;
      f32x16 s_next[2];
      __builtin_amdgcn_s_setprio(1);
      if (more) scores(slot(k + 1), s_next);
      pv(slot(k), pk);
      __builtin_amdgcn_s_setprio(0);
      if (grp == 0)
        __syncthreads();
      else
        refill(k);
      if (more) {
        mask(uniform(w1.t), slot(k + 1), s_next);
        rescale(tile_max(s_next), s_next);
        softmax(s_next, pk);
      }
      if (grp == 0)
        refill(k);
      else
        __syncthreads();
      walk = w1;
      if (w1.t >= 0) w1.next();
      ++k;
    }
    if (grp == 0) __syncthreads();  // matches group 1's extra barrier
  }

  // epilogue: O = O^T / l, LSE = ln2 (m + log2 l)
  const float lt = pair_sum(lsum);
  const float inv = 1.f / lt;
  if (row < S) {
    uint16_t* dst = a.o + base + (int64_t)row * D + 4 * hl;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& ov = o[dg];
        uint32_t w0 = pack_bf16x2(ov[4 * rq] * inv, ov[4 * rq + 1] * inv);
        uint32_t w1 = pack_bf16x2(ov[4 * rq + 2] * inv, ov[4 * rq + 3] * inv);
        *(u32x2*)(dst + 32 * dg + 8 * rq) = u32x2{w0, w1};
      }
    if (hl == 0) a.lse[(int64_t)bh * S + row] = (m + __log2f(lt)) * kLn2;
  }
}

hipError_t launch_attn_fwd(const FwdArgs& a, int D, hipStream_t st) {
  constexpr int NW = 8, NSTAGE = 4;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_qtiles)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, NW, NSTAGE>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, NW, NSTAGE>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
