// Decode attention against a long key/value cache (gfx950, bf16 MFMA, fp32
// accumulate): n_q <= 32 new query rows of each (b, h) against S cached
// keys.  The pages run 1M-token inference with the same blockwise attention;
// here the keys are split into chunks (split-K), one wave per chunk streams
// its K/V tiles once from HBM and keeps the online-softmax state (running max
// m, running sum l, unnormalised O) of every query row, and a second kernel
// merges the chunks with the same rule: M = max_c m_c,
// l = sum_c l_c 2^(m_c - M), O = sum_c O_c 2^(m_c - M) / l (zhao9797 page
// "LWM (Large World Model)", 模型架构: blockwise attention, exact).
//
// The work is HBM-bound: each cache element is read once, and the MFMAs for
// up to 32 rows cost far less than the bytes.  Per 32-key tile a wave
//  - reads K rows straight into registers as the A operand of S^T = K Q^T
//    (lane = key row, 16 bytes of d per MFMA), the next tile's K and V
//    already in flight;
//  - writes the V rows (read as contiguous 1 KB lines) to its own LDS tile
//    and takes the V^T operand of O^T += V^T P^T with transposing LDS reads
//    (ds_read_b64_tr_b16), so the cache needs no transposed copy.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace bwattn {

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Cache policy of a buffer load: default, or non-temporal (streamed once).
constexpr int kCpolDefault = 0, kCpolStream = 2;

// 16 bytes at byte offset `off` of a buffer resource (zero past its end).
template <int CPOL>
__device__ __forceinline__ bf16x8 buffer_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL));
}

template <int D>
__global__ __launch_bounds__(64) void attn_decode_partial_kernel(DecodeArgs a) {
  constexpr int TK = kDecodeTile;  // keys per tile
  constexpr int NDC = D / 16, NDG = D / 32;
  constexpr int NV = TK * D / 8 / 64;  // 16-byte V chunks per lane per tile
  static_assert(TK == 32, "one 32x32 score tile per step");
  __shared__ __attribute__((aligned(16))) uint16_t vtile[TK * D];

  const int lane = threadIdx.x, hl = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x / a.n_chunks, c = blockIdx.x - bh * a.n_chunks;
  const int S = a.S, nq = a.n_q;
  const int k0 = c * a.chunk, k1 = min(S, k0 + a.chunk);

  // Q operand (B of S^T = K Q^T): lane holds query row l32, d = 16 dc + 8 hl + [0, 8)
  bf16x8 qop[NDC];
  {
    const uint16_t* qrow = a.q + ((int64_t)bh * nq + min(l32, nq - 1)) * D + 8 * hl;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      bf16x8 x = *(const bf16x8*)(qrow + 16 * dc);
      qop[dc] = l32 < nq ? x : bf16x8{};
    }
  }
  // query row r sits at sequence index S - nq + r
  const int lim = a.causal ? S - nq + l32 : S - 1;  // last key this row sees
  const int first_limited = a.causal ? S - nq : S - 1;  // keys above this are masked for some row

  // buffers over this chunk's keys (a chunk holds at most kDecodeMaxChunk
  // keys, so byte offsets stay far below 2^31)
  const int64_t base = ((int64_t)bh * S + k0) * D;
  const int nbytes = max(k1 - k0, 0) * D * 2;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + base), (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + base), (short)0, nbytes, 0x00020000);
  // Each K load takes 32 bytes of each of 32 rows, so the rest of those
  // cache lines is read by the next loads: K keeps the default policy (as
  // streamed loads, the lines were re-fetched: +3% bytes, -12% rate).  Each
  // V load reads 1 KB in one run and nothing reads it again: streamed, which
  // took the kernel from ~5.9 to ~6.4 TB/s.
  auto load_k = [&](int t0, bf16x8 (&kk)[NDC]) {
    const uint32_t off = ((uint32_t)(t0 - k0 + l32) * D + 8 * hl) * 2;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) kk[dc] = buffer_b128<kCpolDefault>(kr, off + 32 * dc);
  };
  auto load_v = [&](int t0, bf16x8 (&vv)[NV]) {
    const uint32_t off = (uint32_t)(t0 - k0) * D * 2 + lane * 16;
#pragma unroll
    for (int i = 0; i < NV; ++i) vv[i] = buffer_b128<kCpolStream>(vr, off + i * 1024);
  };

  // transposing-read address of lane L = 16 g + s: the A operand of
  // O^T += V^T P^T for keys 16 kc .. and d 32 dg .. puts V[key][d] with
  // d = 32 dg + L % 32 and key = 16 kc + 8 h + 4 (L / 32) + r in element
  // 4 h + r (the key order in which the score registers hold P), h = 0, 1
  const int g = lane >> 4, s16 = lane & 15;
  const int tr_key = 4 * (g >> 1) + (s16 >> 2);
  const int tr_d = (16 * g + 4 * (s16 & 3)) & 31;
  auto vt_operand = [&](int kc, int dg) {
    const uint16_t* p0 = vtile + (16 * kc + tr_key) * D + 32 * dg + tr_d;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0 + 8 * D));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, x);
  };

  float m = kNegInf, lsum = 0.f;
  f32x16 o[NDG];
#pragma unroll
  for (int dg = 0; dg < NDG; ++dg) o[dg] = f32x16{};
  constexpr float kLazy = 8.f;

  bf16x8 kc_[NDC], vc_[NV];
  if (k0 < k1) {
    load_k(k0, kc_);
    load_v(k0, vc_);
  }
  for (int t0 = k0; t0 < k1; t0 += TK) {
    bf16x8 kn[NDC], vn[NV];
    const bool more = t0 + TK < k1;
    if (more) {
      load_k(t0 + TK, kn);
      load_v(t0 + TK, vn);
    }
    // S^T in log2 units (the query rows carry scale * log2(e)): s[i] holds
    // key t0 + 8 (i/4) + 4 hl + i%4 of this lane's row
    f32x16 s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) s = mfma32(kc_[dc], qop[dc], s);
    if (t0 + TK > k1 || t0 + TK - 1 > first_limited) {
      const int klim = min(lim, k1 - 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = t0 + 8 * (i >> 2) + 4 * hl + (i & 3);
        s[i] = j <= klim ? s[i] : kNegInf;
      }
    }
    // online softmax, the running max raised lazily per row (as in the forward)
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = pair_max(mx);
    const bool grow = mx > m + kLazy;
    if (__ballot(grow)) {
      const float mnew = grow ? fmaxf(m, mx) : m;
      const float alpha = fast_exp2(m - (mnew == kNegInf ? 0.f : mnew));
      lsum *= alpha;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) o[dg] *= alpha;
      m = mnew;
    }
    const float muse = (m == kNegInf) ? 0.f : m;
    bf16x8 pk[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(s[8 * kc + e] - muse);
      u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                  pack_bf16x2(p[6], p[7])};
#pragma unroll
      for (int e = 0; e < 4; ++e) lsum = dot2_bf16(pw[e], kBf16OnePair, lsum);
      pk[kc] = __builtin_bit_cast(bf16x8, pw);
    }
    // V rows to LDS (the tile's 16-byte chunks in order), then O^T += V^T P^T
#pragma unroll
    for (int i = 0; i < NV; ++i) *(bf16x8*)(vtile + (i * 64 + lane) * 8) = vc_[i];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) o[dg] = mfma32(vt_operand(kc, dg), pk[kc], o[dg]);
    if (more) {
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) kc_[dc] = kn[dc];
#pragma unroll
      for (int i = 0; i < NV; ++i) vc_[i] = vn[i];
    }
  }

  // partial state of the rows < nq: O unnormalised [d], (m, l)
  const float lt = pair_sum(lsum);
  if (l32 < nq) {
    const int64_t prow = ((int64_t)blockIdx.x * nq + l32);
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& ov = o[dg];
        *(f32x4*)(po + 32 * dg + 8 * rq + 4 * hl) = f32x4{ov[4 * rq], ov[4 * rq + 1], ov[4 * rq + 2], ov[4 * rq + 3]};
      }
    if (hl == 0) *(f32x2*)(a.part_ml + prow * 2) = f32x2{m, lt};
  }
}

// Merge of the chunk states of one (b, h, query row) per workgroup; thread t
// holds d = t + 64 i.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(DecodeArgs a) {
  constexpr int ND = D / 64;
  const int t = threadIdx.x;
  const int row = blockIdx.x % a.n_q;
  const int64_t bh = blockIdx.x / a.n_q;
  const int nc = a.n_chunks;
  auto prow = [&](int c) { return (bh * nc + c) * a.n_q + row; };
  float M = kNegInf;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, a.part_ml[prow(c) * 2]);
  const float mref = M == kNegInf ? 0.f : M;
  float l = 0.f, acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = 0.f;
  for (int c = 0; c < nc; ++c) {
    const f32x2 ml = *(const f32x2*)(a.part_ml + prow(c) * 2);
    const float w = fast_exp2(ml[0] - mref);  // 0 for a chunk that saw no key of this row
    l += w * ml[1];
    const float* po = a.part_o + prow(c) * D;
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] += w * po[t + 64 * i];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* dst = a.o + (bh * a.n_q + row) * D;
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    f32x2 f = {acc[i] * inv, 0.f};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    dst[t + 64 * i] = __builtin_bit_cast(uint32_t, h) & 0xffffu;
  }
  if (t == 0) a.lse[bh * a.n_q + row] = l > 0.f ? (M + __log2f(l)) * kLn2 : kNegInf;
}

// Workspace of attn_decode_noalloc: a file-scope array in device memory, so
// that entry point allocates nothing.  Host code never uses the array's name
// as an address (on the host it only names the symbol): decode_scratch looks
// up its device address once per device with that device current, and the
// kernels receive that address.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attn_decode_partial(const DecodeArgs& a, int D, hipStream_t st) {
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_chunks)), block(64);
  if (D == 128)
    hipLaunchKernelGGL(attn_decode_partial_kernel<128>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(attn_decode_partial_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_decode_combine(const DecodeArgs& a, int D, hipStream_t st) {
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_q)), block(64);
  if (D == 128)
    hipLaunchKernelGGL(attn_decode_combine_kernel<128>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(attn_decode_combine_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
