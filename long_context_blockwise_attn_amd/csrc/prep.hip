// RoPE and tile-schedule kernels.
//
// RoPE ("standard RoPE" with a context-scaled base theta: zhao9797 page
// "LWM (Large World Model)", 模型架构 and the Stage I table of 训练方法; read as
// RoFormer's rotation of adjacent pairs): pair i of a row at position pos turns
// by pos * theta^(-2i/D).  Positions reach 2^20 and theta 5e7, so the angle is
// formed and reduced to one turn in fp64 before the fp32 sine and cosine.
//
// Tile schedule (masked sequence packing: each packed example attends only to
// itself, 训练方法): per 32-row block the min and max segment id, and per tile
// the range of tiles on the other side that can hold a visible pair.  A pair
// of tiles whose segment-id ranges do not intersect has no visible pair, which
// holds for any int32 ids; the range is tight when documents are contiguous.
#include "common.hpp"
#include "kernels.hpp"

namespace bwattn {

// One thread per (b, s, group of 4 pairs); it forms the 4 angles once and
// rotates that group in every head, so the fp64 work is shared by H rows.
// rope_group gives the thread's cosines and sines and the element offset of
// its group in head 0 (-1: no work).
__device__ __forceinline__ int64_t rope_group(const RopeArgs& a, float (&c)[4], float (&sn)[4]) {
  const int groups = a.D / 8;
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)a.B * a.S * groups;
  if (tid >= total) return -1;
  int g = (int)(tid % groups);
  int64_t bs = tid / groups;
  int s = (int)(bs % a.S);
  int b = (int)(bs / a.S);
  double pos = a.pos ? (double)a.pos[bs] : (double)(a.pos_base + s);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rope_cos_sin(pos, a.turns[4 * g + i], c[i], sn[i]);
    if (a.inverse) sn[i] = -sn[i];
  }
  return ((int64_t)b * a.H * a.S + s) * a.D + 8 * g;
}

// bf16 rows: y = bf16((R x) * out_scale).  The attention kernels take the
// query rows with out_scale = softmax scale * log2(e), so their score MFMAs
// leave scores in log2 units (the forward forms them itself, with the same
// functions, as it loads its query rows); keys and rope_apply use 1.
__global__ void rope_kernel(RopeArgs a) {
  float c[4], sn[4];
  int64_t off = rope_group(a, c, sn);
  if (off < 0) return;
  const int64_t head_stride = (int64_t)a.S * a.D;
  if (!a.stream) {
    for (int h = 0; h < a.H; ++h, off += head_stride) {
      u32x4 x = *(const u32x4*)(a.x + off);
      u32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = rope_pair(x[i], c[i], sn[i], a.out_scale);
      *(u32x4*)(a.y + off) = y;
    }
    return;
  }
  // large tensors: four heads' loads in flight per thread, and non-temporal
  // accesses (every byte is read and written once)
  int h = 0;
  for (; h + 4 <= a.H; h += 4, off += 4 * head_stride) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load((const u32x4*)(a.x + off + u * head_stride));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = rope_pair(x[u][i], c[i], sn[i], a.out_scale);
      __builtin_nontemporal_store(y, (u32x4*)(a.y + off + u * head_stride));
    }
  }
  for (; h < a.H; ++h, off += head_stride) {
    u32x4 x = __builtin_nontemporal_load((const u32x4*)(a.x + off));
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = rope_pair(x[i], c[i], sn[i], a.out_scale);
    __builtin_nontemporal_store(y, (u32x4*)(a.y + off));
  }
}

// fp32 rows: the same rotation, fp32 in and out.
__global__ void rope_f32_kernel(RopeArgs a, const float* x, float* y) {
  float c[4], sn[4];
  int64_t off = rope_group(a, c, sn);
  if (off < 0) return;
  const int64_t head_stride = (int64_t)a.S * a.D;
  for (int h = 0; h < a.H; ++h, off += head_stride) {
    f32x4 u = *(const f32x4*)(x + off), w = *(const f32x4*)(x + off + 4);
    float v[8] = {u[0], u[1], u[2], u[3], w[0], w[1], w[2], w[3]};
    float r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = v[2 * i] * c[i] - v[2 * i + 1] * sn[i];
      r[2 * i + 1] = v[2 * i] * sn[i] + v[2 * i + 1] * c[i];
    }
    *(f32x4*)(y + off) = f32x4{r[0], r[1], r[2], r[3]};
    *(f32x4*)(y + off + 4) = f32x4{r[4], r[5], r[6], r[7]};
  }
}

// Min and max segment id of every 32-row block of every batch row.
__global__ void block_range_kernel(const int32_t* seg, int B, int S, int nblk, int2* out) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= (int64_t)B * nblk) return;
  int blk = (int)(tid % nblk);
  int b = (int)(tid / nblk);
  int r0 = blk * 32, r1 = min(S, r0 + 32);
  const int32_t* sb = seg + (int64_t)b * S;
  int mn = sb[r0], mx = sb[r0];
  for (int r = r0 + 1; r < r1; ++r) {
    mn = min(mn, sb[r]);
    mx = max(mx, sb[r]);
  }
  out[tid] = make_int2(mn, mx);
}

// Min and max segment id of every 64-row tile (from the 32-row blocks), in
// rows of n64p entries; entries past the last tile repeat it.
__global__ void tile64_range_kernel(const int2* blk, int B, int S, int nblk, int n64p, int2* out) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= (int64_t)B * n64p) return;
  const int b = (int)(tid / n64p);
  const int n64 = (S + 63) / 64;
  const int t = min((int)(tid % n64p), n64 - 1);
  const int2* br = blk + (int64_t)b * nblk;
  int2 r = br[2 * t];
  if (2 * t + 1 < nblk) {
    const int2 u = br[2 * t + 1];
    r = make_int2(min(r.x, u.x), max(r.y, u.y));
  }
  out[tid] = r;
}

__device__ __forceinline__ int2 rows_range(const int2* br, int nblk, int r0, int rows) {
  int b0 = r0 >> 5, b1 = min(nblk, (r0 + rows + 31) >> 5);
  int2 acc = br[b0];
  for (int k = b0 + 1; k < b1; ++k) {
    int2 v = br[k];
    acc.x = min(acc.x, v.x);
    acc.y = max(acc.y, v.y);
  }
  return acc;
}

// One wave per (b, own tile).  Writes [lo, hi) over the other side's tiles:
// the first and one past the last tile whose segment range meets the own
// tile's, within the causal candidates.  own_is_query selects which side of
// the causal condition the own tile is on.
__global__ void tile_range_kernel(TileRangeArgs a) {
  int wid = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6);
  int lane = threadIdx.x & 63;
  if (wid >= a.B * a.n_own) return;
  int t = wid % a.n_own;
  int b = wid / a.n_own;
  int own0 = t * a.own_rows;
  int own1 = min(a.S, own0 + a.own_rows);  // exclusive
  int c_lo = 0, c_hi = a.n_other;
  if (a.causal) {
    if (a.own_is_query)
      c_hi = min(a.n_other, (own1 - 1) / a.other_rows + 1);
    else
      c_lo = own0 / a.other_rows;
  }
  int lo = c_lo, hi = c_hi;
  if (a.blk != nullptr && c_lo < c_hi) {
    const int2* br = a.blk + (int64_t)b * a.nblk;
    int2 own = rows_range(br, a.nblk, own0, own1 - own0);
    lo = c_hi;
    for (int base = c_lo; base < c_hi; base += 64) {
      int c = base + lane;
      bool hit = false;
      if (c < c_hi) {
        int2 o = rows_range(br, a.nblk, c * a.other_rows, a.other_rows);
        hit = !(o.y < own.x || o.x > own.y);
      }
      unsigned long long m = __ballot(hit);
      if (m) {
        lo = base + __ffsll((long long)m) - 1;
        break;
      }
    }
    hi = lo;
    for (int top = c_hi; top > lo; top -= 64) {
      int c = top - 1 - lane;
      bool hit = false;
      if (c >= lo) {
        int2 o = rows_range(br, a.nblk, c * a.other_rows, a.other_rows);
        hit = !(o.y < own.x || o.x > own.y);
      }
      unsigned long long m = __ballot(hit);
      if (m) {
        hi = top - (__ffsll((long long)m) - 1);
        break;
      }
    }
  }
  // does every tile in [lo, hi) meet the own tile's segment range?
  bool sparse = false;
  if (a.blk != nullptr && lo < hi) {
    const int2* br = a.blk + (int64_t)b * a.nblk;
    int2 own = rows_range(br, a.nblk, own0, own1 - own0);
    for (int base = lo; base < hi; base += 64) {
      int c = base + lane;
      bool miss = false;
      if (c < hi) {
        int2 o = rows_range(br, a.nblk, c * a.other_rows, a.other_rows);
        miss = o.y < own.x || o.x > own.y;
      }
      if (__ballot(miss)) {
        sparse = true;
        break;
      }
    }
  }
  if (lane == 0) a.out[wid] = make_int2(lo | (sparse ? kRangeSparse : 0), hi);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_rope(const RopeArgs& a, hipStream_t st) {
  int64_t total = (int64_t)a.B * a.S * (a.D / 8);
  int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  // Streaming accesses pay off only for tensors well beyond the 256 MB
  // last-level cache: measured -6% at 1 GiB, +25% at 256 MiB.
  RopeArgs b = a;
  b.stream = (int64_t)a.B * a.H * a.S * a.D * 2 >= (int64_t(512) << 20) ? 1 : 0;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_rope_f32(const RopeArgs& a, const float* x, float* y, hipStream_t st) {
  int64_t total = (int64_t)a.B * a.S * (a.D / 8);
  int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_f32_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, a, x, y);
  return hipGetLastError();
}

hipError_t launch_block_ranges(const int32_t* seg, int B, int S, int nblk, int2* out, hipStream_t st) {
  int64_t total = (int64_t)B * nblk;
  int threads = 256;
  hipLaunchKernelGGL(block_range_kernel, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, st,
                     seg, B, S, nblk, out);
  return hipGetLastError();
}

hipError_t launch_tile64_ranges(const int2* blk, int B, int S, int nblk, int n64p, int2* out, hipStream_t st) {
  int64_t total = (int64_t)B * n64p;
  int threads = 256;
  hipLaunchKernelGGL(tile64_range_kernel, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, st,
                     blk, B, S, nblk, n64p, out);
  return hipGetLastError();
}

hipError_t launch_tile_ranges(const TileRangeArgs& a, hipStream_t st) {
  int64_t waves = (int64_t)a.B * a.n_own;
  int threads = 256;
  int64_t blocks = (waves * 64 + threads - 1) / threads;
  hipLaunchKernelGGL(tile_range_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
