// LDS tile layout, MFMA operand reads and the K/V (or Q/dO) tile walk shared
// by the attention kernels.
#pragma once
#include "common.hpp"

namespace bwattn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// A tile of `rows` x D bf16 in LDS, row-major.  Each row's 16-byte chunks are
// XOR-swizzled by swz(row) so that both operand reads below hit 32 distinct
// banks per group of lanes: the 16-byte read (8 consecutive rows, one chunk)
// and the transposing 8-byte read (4 consecutive rows, two adjacent chunks).
template <int D>
struct Tile {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;
  __device__ static __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
  __device__ static __forceinline__ uint32_t off(int row, int chunk) {
    return (uint32_t)(row * kRowBytes + ((chunk ^ swz(row)) << 4));
  }
  // MFMA operand whose lane l holds row r0 + (l % 32), columns
  // 16 c + 8 (l / 32) + [0, 8): a 32x32x16 operand with k along the row.
  __device__ static __forceinline__ bf16x8 read_rows(const char* t, int r0, int c, int lane) {
    return *(const bf16x8*)(t + off(r0 + (lane & 31), 2 * c + (lane >> 5)));
  }
  // MFMA operand with k along the column: lane l holds column col0 + (l % 32)
  // at rows r0 + 4h + {0..3} and r0 + 8 + 4h + {0..3} (h = l / 32), built
  // from two transposing 8-byte reads (ds_read_b64_tr_b16: within a group of
  // 16 lanes, output lane i element r comes from source lane 4r + i/4,
  // element i % 4).
  __device__ static __forceinline__ bf16x8 read_cols(const char* t, int r0, int col0, int lane) {
    int j = lane & 15;
    int col = col0 + ((lane >> 4) & 1) * 16 + 4 * (j & 3);
    int row = r0 + 4 * (lane >> 5) + (j >> 2);
    uint32_t sub = ((col >> 2) & 1) * 8;
    const char* p1 = t + off(row, col >> 3) + sub;
    const char* p2 = t + off(row + 8, col >> 3) + sub;
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p2));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, r);
  }
};

// Copy rows [r0, r0 + 64) of a [S, D] bf16 matrix into an LDS tile with the
// swizzled layout, by direct global-to-LDS loads (no registers).  NT threads
// share the copy; each 64-lane load fills 1 KiB of consecutive LDS, so lane
// i of a load fetches the global chunk that belongs at its LDS position.
// Rows at or past S read row S-1 instead (finite data that the kernels mask).
template <int D, int NT>
__device__ __forceinline__ void tile_to_lds(const uint16_t* src, int r0, int S, char* tile, int tid) {
  constexpr int NCH = D / 8;
  constexpr int PER = 64 * NCH / NT;  // loads per wave
  const int w = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int blk = w * PER + i;
    int p = blk * 64 + lane;
    int row = p / NCH, phys = p % NCH;
    int logical = phys ^ Tile<D>::swz(row);
    int key = min(r0 + row, S - 1);
    __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)key * D + logical * 8),
                                     (__attribute__((address_space(3))) void*)(tile + blk * 1024), 16, 0, 0);
  }
}

// Copy columns [c0, c0 + 64) of a transposed [D, sp] bf16 matrix (rows d,
// sp a multiple of 64) into an LDS tile of D rows x 64 elements (Tile<64>
// layout), by direct global-to-LDS loads.
template <int D, int NT>
__device__ __forceinline__ void tile_t_to_lds(const uint16_t* src, int sp, int c0, char* tile, int tid) {
  constexpr int PER = D * 8 / NT;  // loads per wave (8 chunks per row of 64)
  const int w = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int blk = w * PER + i;
    int p = blk * 64 + lane;
    int row = p >> 3, phys = p & 7;
    int logical = phys ^ Tile<64>::swz(row);
    __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)row * sp + c0 + logical * 8),
                                     (__attribute__((address_space(3))) void*)(tile + blk * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Max and sum over the two lanes l and l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int2 range_union(int2 a, int2 b) { return make_int2(min(a.x, b.x), max(a.y, b.y)); }
__device__ __forceinline__ bool ranges_meet(int2 a, int2 b) { return !(a.y < b.x || a.x > b.y); }

// Segment-id range of rows [r0, r0 + rows) from the 32-row block ranges.
__device__ __forceinline__ int2 seg_range(const int2* blk, int nblk, int r0, int rows) {
  int b0 = r0 >> 5, b1 = min(nblk, (r0 + rows + 31) >> 5);
  int2 acc = blk[b0];
  for (int k = b0 + 1; k < b1; ++k) acc = range_union(acc, blk[k]);
  return acc;
}

// Walk over tiles [lo, hi) of the streamed side.  ct > 0 selects ring order:
// tiles are grouped in chunks of ct; the walk visits the own chunk r first,
// then r + dir, r + 2 dir, ... (mod nc), tiles ascending inside each chunk.
// dir = -1 is the order in which a query block on one device of a ring sees
// its predecessors' K/V blocks arrive; dir = +1 the order in which a K/V
// block travelling the ring meets the following devices' query blocks.
// Tiles whose segment range misses `own` are passed over.  All state is
// uniform across the workgroup.
struct TileWalk {
  int lo, hi, ct, nc, r, dir;
  int step, t;
  const int2* blk;
  int nblk, rows;
  int2 own;
  __device__ bool useful(int tile) const {
    return blk == nullptr || ranges_meet(seg_range(blk, nblk, tile * rows, rows), own);
  }
  __device__ void seek(int after) {
    if (ct == 0) {
      for (int c = after + 1; c < hi; ++c)
        if (useful(c)) { t = c; return; }
      t = -1;
      return;
    }
    while (step < nc) {
      int c = r + dir * step;
      if (c < 0) c += nc;
      if (c >= nc) c -= nc;
      int c1 = min(hi, (c + 1) * ct);
      for (int x = max(max(lo, c * ct), after + 1); x < c1; ++x)
        if (useful(x)) { t = x; return; }
      ++step;
      after = -1;
    }
    t = -1;
  }
  __device__ void start() {
    step = 0;
    seek(lo - 1);
  }
  __device__ void next() { seek(t); }
};

}  // namespace bwattn
