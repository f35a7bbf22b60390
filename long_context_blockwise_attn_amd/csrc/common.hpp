// Device-side helpers shared by the HIP kernels of the library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bwattn {

typedef uint16_t bf16_t;  // raw bf16 bits in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// a.x * b.x + a.y * b.y + c for packed bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
constexpr uint32_t kBf16OnePair = 0x3f803f80u;  // (1.0, 1.0) in bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// RoPE of one pair (RoFormer's rotation of adjacent pairs, base theta scaled
// with the context: zhao9797 page "LWM (Large World Model)", 模型架构).  The
// angle pos * turns (in turns) is reduced to [-1/2, 1/2] turn in fp64 before
// the fp32 cosine and sine: positions reach 2^20 and theta 5e7.  The RoPE
// pre-pass and the forward's query load both go through these two functions,
// so the forward's rotated query rows are bitwise those the backward reads.
__device__ __forceinline__ void rope_cos_sin(double pos, double turns, float& c, float& s) {
  double rev = pos * turns;
  rev -= rint(rev);
  const float f = (float)rev;
  c = __builtin_amdgcn_cosf(f);  // cos(2 pi f)
  s = __builtin_amdgcn_sinf(f);
}
// bf16 pair (x0, x1) -> bf16 pair of (R x) * scale, R the rotation by (c, s)
__device__ __forceinline__ uint32_t rope_pair(uint32_t x, float c, float s, float scale) {
  const float x0 = bf16_lo(x), x1 = bf16_hi(x);
  const float y0 = x0 * c - x1 * s;
  const float y1 = x0 * s + x1 * c;
  return pack_bf16x2(y0 * scale, y1 * scale);
}

// Workgroup order for long-to-short scheduling with heads grouped per XCD.
// Workgroups are handed to the 8 XCDs round robin; when the number of (b,h)
// slices is a multiple of 8, all tiles of one slice go to one XCD so that its
// concurrent workgroups share K/V in that XCD's L2.  Tiles are issued in the
// order given by `rank` (0 = first).  The map is a bijection in every case.
__device__ __forceinline__ void xcd_tile_order(int bid, int n_bh, int n_tiles, int& bh, int& rank) {
  if ((n_bh & 7) == 0) {
    int xcd = bid & 7, j = bid >> 3;
    int per = n_bh >> 3;
    rank = j / per;
    bh = xcd + 8 * (j - rank * per);
  } else {
    rank = bid / n_bh;
    bh = bid - rank * n_bh;
  }
}

}  // namespace bwattn
