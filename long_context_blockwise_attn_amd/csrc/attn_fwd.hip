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
// scale * log2(e) * <q', k'> - m, the exponent of exp2 itself (or -inf where
// a mask hides the key).  Tiles of 64 keys of K and V rows sit in LDS rings
// filled by buffer-to-LDS loads and are taken in halves of 32 keys.  Scores are
// computed transposed, S^T = K Q^T, so each lane holds one query row: the row
// max needs one exchange between lanes l and l^32, and the running rescale of
// O is a per-lane scalar.  O^T = V^T P^T takes P^T straight from the score
// registers; its V^T operand is read from the V rows with transposing LDS
// reads (PTile::read_tr), which deliver the keys in the order the score
// registers hold them, so no transposed copy of V is made.
//
// Each wave interleaves its own matrix and vector work (the software
// pipeline below): a wave's vector instructions placed between its own
// MFMAs issue while those run, whereas one wave issuing only MFMAs beside
// another issuing only vector work on the same SIMD overlaps poorly (a
// measured property of this hardware, not a documented one).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace bwattn {

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdArgs a) {
  constexpr int BQ = kFwdBlockQ, BK = kFwdBlockK;
  static_assert(BQ == NW * 32, "32 query rows per wave");
  static_assert(BK == 64, "two 32-key halves per tile");
  constexpr int NDC = D / 16;  // 16-wide k steps over D for S^T
  constexpr int NDG = D / 32;  // 32-row groups of O^T over D
  constexpr float kLazy = 8.f;
  using KT = PTile<BK, D / 8>;  // K rows
  // V rows (V^T read transposed).  P = 4 would make these reads conflict-free
  // but measured no faster: its two extra pad chunks per row lengthen the loads.
  using VR = PTile<BK, D / 8, 2>;
  constexpr int NKS = 4, NVS = 4, NSS = 4;  // K, V and segment-id slots
  constexpr int SEG_OFF = NKS * KT::kBytes + NVS * VR::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[SEG_OFF + NSS * 256];

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
  // -m in every register (0 while m = -inf): the score MFMAs start from it.
  // Hidden from the optimizer (an empty asm statement) wherever it is set:
  // knowing the 16 values equal, it kept one register and rebuilt the tile
  // with 16 moves before every score chain.
  f32x16 negm = f32x16{};
  asm volatile("" : "+v"(negm));
  f32x16 o[NDG];
#pragma unroll
  for (int dg = 0; dg < NDG; ++dg) o[dg] = f32x16{};

  const uint16_t* kh = a.k + base;
  const uint16_t* vh = a.v + base;
  TileFill<BK, D / 8, NW> kfill;     // K rows
  TileFill<BK, D / 8, NW, 2> vfill;  // V rows
  kfill.init(D * 2, tid);
  vfill.init(D * 2, tid);
  // --- per-tile pieces -----------------------------------------------------
  // Start values of the score MFMAs of the half (32 keys) j of tile t: key
  // k0 + 32 j + 8 (r/4) + 4 hl + r%4 in register r starts from -m, or from
  // -inf where the causal, segment or sequence-end mask hides the key, so
  // that masked scores leave the MFMAs as -inf and no vector code touches
  // them.  The decisions are wave-uniform, and a tile tests only what it
  // needs: the position limit (diagonal, sequence end), the segment ids
  // (document edge), or both.
  struct MaskPlan {
    int k0;
    bool lim_mask, seg_mask;
  };
  auto mask_plan = [&](int t) {
    MaskPlan p;
    p.k0 = t * BK;
    p.seg_mask = false;
    if (use_seg) {
      int2 kr = tile64_range(t64b, t);
      p.seg_mask = !(kr.x == kr.y && wrange.x == wrange.y && kr.x == wrange.x);
    }
    p.lim_mask = (p.k0 + BK > S) || (a.causal && p.k0 + BK - 1 > q0);
    return p;
  };
  auto score_init = [&](const MaskPlan& p, const char* segbuf, int j) -> f32x16 {
    if (!uniform(p.seg_mask || p.lim_mask)) return negm;
    const float nm = negm[0];
    const int lim = (a.causal ? min(S - 1, row) : S - 1) - p.k0 - 4 * hl;  // last visible key, tile-relative
    f32x16 c;
    if (!uniform(p.seg_mask)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = (32 * j + 8 * (r >> 2) + (r & 3) <= lim) ? nm : kNegInf;
    } else {
      const int* segk = (const int*)segbuf;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int4 sk = *(const int4*)(segk + 32 * j + 8 * rq + 4 * hl);
        const int sk_[4] = {sk.x, sk.y, sk.z, sk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = (uniform(p.lim_mask) ? (32 * j + 8 * rq + e <= lim) : true) & (sk_[e] == segq);
          c[4 * rq + e] = vis ? nm : kNegInf;
        }
      }
    }
    return c;
  };
  // Row max of a half tile's scores, relative to m (to 0 while m = -inf), in
  // 8 pieces over four independent chains: chain c covers registers 4c..4c+3.
  // (IEEE maximum: the same value as fmaxf for the scores, which are never
  // NaN, without the canonicalising max fmaxf adds for each MFMA result.)
  auto vmax = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  auto max_piece = [&](int j, const f32x16& s, float (&mc)[4]) {
    const int c = j & 3;
    if (j < 4)
      mc[c] = vmax(s[4 * c], s[4 * c + 1]);
    else
      mc[c] = vmax(vmax(mc[c], s[4 * c + 2]), s[4 * c + 3]);
  };
  auto max_done = [&](const float (&mc)[4]) {
    const float x = vmax(vmax(mc[0], mc[1]), vmax(mc[2], mc[3]));
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  // Lazy online-softmax max update.  A row's running max m is raised only
  // when its new max exceeds it by more than kLazy (log2 units); otherwise
  // the stale m stays, p <= 2^kLazy, and O is not touched.  l and O share m,
  // so the normalised result is unchanged.  The decision is per row (the
  // wave only branches when some row needs it), so a row's result depends on
  // its own visible keys alone.  A raised m moves the half tile's scores by
  // the rise and the start value of later score MFMAs with it.
  auto grows = [&](float mx) { return mx > (m == kNegInf ? kNegInf : kLazy); };
  // (grows: the row's vote; rescale: what the wave does when any row votes)
  auto rescale = [&](float mx, bool grow, f32x16& s) {
    const float rise = grow ? mx : 0.f;
    const float mnew = grow ? (m == kNegInf ? mx : m + mx) : m;
    const float alpha = fast_exp2(grow ? m - mnew : 0.f);  // 0 from m = -inf, where l and O are 0
    lsum *= alpha;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg) o[dg] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] -= rise;
    m = mnew;
    const float nm = (m == kNegInf) ? 0.f : -m;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = nm;
    asm volatile("" : "+v"(negm));
  };
  // P = 2^(S*scale*log2e - m) of a half tile as bf16 MFMA operands pk[kc]
  // (its keys 16 kc ..) and the row sum over the same bf16 values (one chain
  // per kc), in 8 pieces: piece j makes the pair 2 (j % 4) of pk[j / 4]
  auto softmax_piece = [&](int j, const f32x16& s, u32x4 (&pw)[2], float (&rs)[2]) {
    const int kc = j >> 2, e = j & 3, r = 8 * kc + 2 * e;
    pw[kc][e] = pack_bf16x2(fast_exp2(s[r]), fast_exp2(s[r + 1]));
    rs[kc] = dot2_bf16(pw[kc][e], kBf16OnePair, rs[kc]);
  };

  // --- software pipeline --------------------------------------------------
  // The keys of a 64-key tile are taken in two halves of 32 (half-steps).
  // Half-step h runs O^T += V^T P^T of half h, the softmax of half h+1 and
  // the scores of half h+2, so the matrix work of a half-step never waits on
  // its vector work: each wave issues its own MFMAs with its vector
  // instructions between them (two waves per SIMD run the same program).
  // The first part pairs the PV MFMAs with the row max of half h+1; after the
  // max update, the second pairs the score MFMAs of half h+2 (which start from
  // the updated -m) with the exponentials of half h+1.
  //
  // Step k is half-steps 2k and 2k+1: it reads V of tile position k and K
  // and the segment ids of position k+1.  LDS: K, V and segment ids of
  // position p in slot p % 4 of their rings.  Step k issues K and the
  // segment ids of position k+3 and V of position k+2, one load between two
  // MFMAs of its first half-step (issued in a burst after a barrier, they
  // stalled every wave at once).  Only even steps open with a barrier, after
  // each wave has waited for all its loads: those of step k-1 are read from
  // step k+1 on, and no wave can still be in step k-1 when one issues into
  // the slots that steps k-2 and earlier read.  With four slots per ring a
  // load never lands in a slot some wave may still read, and half of the
  // barriers go.
  auto kslot = [&](int p) { return smem + (p % NKS) * KT::kBytes; };
  auto vslot = [&](int p) { return smem + NKS * KT::kBytes + (p % NVS) * VR::kBytes; };
  auto sslot = [&](int p) { return smem + SEG_OFF + (p & (NSS - 1)) * 256; };
  // Buffer resources of tile t's K (V) rows; a position past the end of the
  // walk (t < 0) gets an empty resource, so its loads only write zeros into
  // a free slot and every step issues the same loads.
  auto rows_rsrc = [&](const uint16_t* h, int t) {
    const int tt = max(t, 0);
    const uint32_t rbytes = t < 0 ? 0u : (uint32_t)min(S - tt * BK, BK) * D * 2;  // rows past S read zero
    return make_rsrc(h + (int64_t)tt * BK * D, rbytes);
  };
  auto seg_rsrc = [&](int t) {
    const int tt = max(t, 0);
    return make_rsrc(segb + tt * BK, t < 0 ? 0u : (uint32_t)(S - tt * BK) * 4);
  };
  auto load_k = [&](int t, int p) {
    const i32x4 rk = rows_rsrc(kh, t);
#pragma unroll
    for (int i = 0; i < decltype(kfill)::kPer; ++i) kfill.fill_part(i, rk, kslot(p));
    if (use_seg && w == 0) dma_b32(seg_rsrc(t), sslot(p), lane * 4);
  };
  auto load_v = [&](int t, int p) {
    const i32x4 rv = rows_rsrc(vh, t);
#pragma unroll
    for (int i = 0; i < decltype(vfill)::kPer; ++i) vfill.fill_part(i, rv, vslot(p));
  };
  // the fewest K (V) loads any wave issues per tile: compile-time wait counts
  // (a wave with more also waits for a few of the newer tile)
  constexpr int kLeastK = KT::kBlocks / NW, kLeastV = VR::kBlocks / NW;
  static_assert(decltype(kfill)::kPer <= 3 && decltype(vfill)::kPer <= 3, "three load slots per part");

  // One half-step.  J: the half of the tile whose V rows PV reads (the
  // scores it makes are of the same half of the next tile).  PV: o += V^T pk
  // from V slot vb.  SM: softmax of s1 into pk.  SC: scores from the K rows
  // in kb into s2, started by score_init.  The vector work of each part is
  // cut into 16 slots spread evenly over its MFMAs: the row max takes the
  // first half of the PV part's slots, its reduction and the wave's rescale
  // vote two more, so the vote is in by the end of the PV MFMAs; exA(slot)
  // and exB(slot) may fill the free slots of the two parts (the loads of
  // later tiles).
  auto half = [&](auto j_, auto pv_, auto sm_, auto sc_, const char* vb, const char* kb, const char* sb,
                  const MaskPlan& plan, f32x16& s1, f32x16& s2, bf16x8 (&pk)[2], auto&& exA, auto&& exB) {
    constexpr int J = decltype(j_)::value;
    constexpr bool PV = decltype(pv_)::value, SM = decltype(sm_)::value, SC = decltype(sc_)::value;
    float mc[4], mx = 0.f;
    bool grow = false;
    uint64_t vote = 0;
    auto slotA = [&](int j) {
      if constexpr (SM) {
        if (j < 8) max_piece(j, s1, mc);
        if (j == 8) mx = max_done(mc);
        if (j == 10) {
          grow = grows(mx);
          vote = __ballot(grow);
        }
      }
      exA(j);
    };
    if constexpr (PV) {
      lds_mfma_pipe_mixed<2 * NDG, 2, 16>(
          [&](int i) { return VR::read_tr(vb, 32 * J + 16 * (i / NDG), 32 * (i % NDG), lane); },
          [&](int i, bf16x8 x) { o[i % NDG] = mfma32(x, pk[i / NDG], o[i % NDG]); }, slotA);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) slotA(j);
    }
    if constexpr (SM) {
      if (vote) rescale(mx, grow, s1);
    }
    u32x4 pw[2];
    float rs[2] = {lsum, 0.f};
    auto slotB = [&](int j) {
      if constexpr (SM) {
        if ((j & 1) == 0) softmax_piece(j >> 1, s1, pw, rs);
      }
      exB(j);
    };
    if constexpr (SC) {
      s2 = score_init(plan, sb, J);
      lds_mfma_pipe_mixed<NDC, 3, 16>([&](int i) { return KT::read(kb, 32 * J, i, lane); },
                                      [&](int i, bf16x8 x) { s2 = mfma32(x, qop[i], s2); }, slotB);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) slotB(j);
    }
    if constexpr (SM) {
      lsum = rs[0] + rs[1];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) pk[kc] = __builtin_bit_cast(bf16x8, pw[kc]);
    }
  };
  auto nop = [](int) {};
  using T_ = BoolC<true>;
  using F_ = BoolC<false>;
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;

  if (walk.t >= 0) {
    // tile indices of positions k+1, k+2 (-1 past the end) as step k starts;
    // `lw` walks the newest K position issued
    TileWalk lw = walk;
    const int t0 = walk.t;
    int t1, t2;
    load_k(t0, 0);
    lw.next();
    t1 = lw.t;
    load_k(t1, 1);
    load_v(t0, 0);
    wait_vmem_le<kLeastK + kLeastV>();
    __syncthreads();  // step -1: K of position 0 is in
    if (lw.t >= 0) lw.next();
    t2 = lw.t;
    load_k(t2, 2);
    load_v(t1, 1);
    bf16x8 pk[2];
    f32x16 sA, sB;
    {
      const MaskPlan p0 = mask_plan(t0);
      half(J0{}, F_{}, F_{}, T_{}, nullptr, kslot(0), sslot(0), p0, sB, sA, pk, nop, nop);  // scores of (0, 0)
      half(J1{}, F_{}, T_{}, T_{}, nullptr, kslot(0), sslot(0), p0, sA, sB, pk, nop,
           nop);  // softmax (0, 0), scores (0, 1)
    }
    // step k: s of (k, 1) in sB.  Every step issued the same loads (empty
    // ones past the end of the walk), so a constant wait count holds.
    int k = 0;
    auto sync = [&]() {
      if ((k & 1) == 0) {
        wait_vmem_le<0>();
        __syncthreads();
      }
      if (lw.t >= 0) lw.next();
      return (int)lw.t;
    };
    while (t1 >= 0) {
      const int t3 = sync();
      const MaskPlan p1 = mask_plan(t1);
      const char* vb = vslot(k);
      const char* kb = kslot(k + 1);
      const char* sb = sslot(k + 1);
      // loads of K of position k+3 (and its segment ids) and V of k+2, one
      // between MFMAs, into slots that step k-1 was the last to read
      const i32x4 rk = rows_rsrc(kh, t3), rv = rows_rsrc(vh, t2), rsg = seg_rsrc(t3);
      char* kd = kslot(k + 3);
      char* vd = vslot(k + 2);
      char* sd = sslot(k + 3);
      auto exA = [&](int j) {
        if (j == 11) kfill.fill_part(0, rk, kd);
        if constexpr (decltype(kfill)::kPer > 1)
          if (j == 13) kfill.fill_part(1, rk, kd);
        if constexpr (decltype(kfill)::kPer > 2)
          if (j == 15) kfill.fill_part(2, rk, kd);
      };
      auto exB = [&](int j) {
        if (j == 1) vfill.fill_part(0, rv, vd);
        if constexpr (decltype(vfill)::kPer > 1)
          if (j == 3) vfill.fill_part(1, rv, vd);
        if constexpr (decltype(vfill)::kPer > 2)
          if (j == 5) vfill.fill_part(2, rv, vd);
        if (j == 7 && use_seg && w == 0) dma_b32(rsg, sd, lane * 4);
      };
      half(J0{}, T_{}, T_{}, T_{}, vb, kb, sb, p1, sB, sA, pk, exA, exB);  // PV (k, 0), softmax (k, 1), scores (k+1, 0)
      half(J1{}, T_{}, T_{}, T_{}, vb, kb, sb, p1, sA, sB, pk, nop, nop);  // PV (k, 1), softmax (k+1, 0), scores (k+1, 1)
      t1 = t2;
      t2 = t3;
      ++k;
    }
    wait_vmem_le<0>();
    __syncthreads();
    const MaskPlan none{};
    const char* vb = vslot(k);
    half(J0{}, T_{}, T_{}, F_{}, vb, nullptr, nullptr, none, sB, sA, pk, nop, nop);  // PV (k, 0), softmax (k, 1)
    half(J1{}, T_{}, F_{}, F_{}, vb, nullptr, nullptr, none, sA, sB, pk, nop, nop);  // PV (k, 1)
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
  constexpr int NW = 8;
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_qtiles)), block(NW * 64);
  if (D == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, NW>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, NW>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
