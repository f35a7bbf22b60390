// LDS tile layout, MFMA operand reads and the K/V (or Q/dO) tile walk shared
// by the attention kernels.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace bwattn {

// An LDS tile of R rows x C 16-byte chunks (8 bf16 each), row-major with P
// chunks of padding per row (row stride (C+P)*16 bytes); a lane's reads at
// different chunks differ by immediate offsets.  The LDS serves a 16-byte
// read 16 lanes at a time over 256 bytes of banks, and a ds_read_b64_tr_b16
// 32 lanes at a time, which here means 4 rows x 64 bytes.  So read (below)
// is conflict-free when C + P is odd (16 consecutive rows fall on 16
// distinct 16-byte bank groups), and read_tr when the stride is 64 modulo
// 128 bytes (the 4 rows fall on distinct quarters of the banks); no padding
// gives both.  Measured on gfx950 at C = 16: P = 1 or 3 run the 16-byte
// reads at full rate and P = 2 or 4 at half rate; P = 4 runs the
// transposing reads at full rate, P = 2 or 3 at half and P = 1 at a quarter.
// The backward's tiles, read both ways, take P = 3.
template <int R, int C, int P = 1>
struct PTile {
  static constexpr int kChunks = C;
  static constexpr int kPad = P;
  static constexpr int kStride = (C + P) * 16;
  static constexpr int kBytes = R * kStride;
  static constexpr int kBlocks = R * (C + P) / 64;  // 1 KiB direct-load blocks
  static_assert((R * (C + P)) % 64 == 0, "tile must be whole 1 KiB blocks");
  // MFMA operand whose lane l holds row r0 + (l % 32) at chunk
  // 2 c + (l / 32): a 32x32x16 operand with k along the row.
  __device__ static __forceinline__ bf16x8 read(const char* t, int r0, int c, int lane) {
    return *(const bf16x8*)(t + (r0 + (lane & 31)) * kStride + (2 * c + (lane >> 5)) * 16);
  }
  // The transposed operand (k along the rows): lane l holds column
  // d = d0 + l % 32 of rows r0 + 8 h + 4 (l / 32) + r in element 4 h + r
  // (h, r < 2, 4) -- the row order in which a 32x32x16 MFMA result holds its
  // rows, so a score tile packed to bf16 is the other operand as it stands.
  // Two ds_read_b64_tr_b16: within each 16-lane group g the instruction
  // hands lane i element r of the 4 elements that lane 4 r + i / 4 addressed,
  // element i % 4; lane 16 g + s therefore addresses row 4 (g / 2) + s / 4,
  // column (16 g + 4 (s % 4)) % 32.
  __device__ static __forceinline__ bf16x8 read_tr(const char* t, int r0, int d0, int lane) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const int g = lane >> 4, s = lane & 15;
    const char* p = t + (r0 + 4 * (g >> 1) + (s >> 2)) * kStride + (d0 + ((16 * g + 4 * (s & 3)) & 31)) * 2;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 8 * kStride));
    i16x8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, x);
  }
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// x, hidden from the optimizer (an empty asm statement that emits no
// instruction): addresses derived from it inside a loop body are formed again
// in each iteration instead of being kept live, and spilled, across the loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A value the caller knows to be the same in every lane, held in a scalar
// register so that branches on it are wave-level jumps.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Raw buffer resource over `bytes` bytes from `base` (stride 0): loads at
// offsets past the end return zero.  Word 3 is the raw-buffer format word of
// gfx9.  The value is uniform across the wave.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Direct buffer-to-LDS loads: lane i writes its 16 (or 4) bytes at LDS byte
// address lds + 16 i (4 i); lds is uniform across the wave.  Issued through
// inline assembly so that the compiler does not treat the in-flight LDS write
// as aliasing the LDS reads that follow: the kernels wait for these loads
// themselves (wait_vmem_le + barrier) before reading the destination.  The
// instructions have no register results.
__device__ __forceinline__ void dma_b128(i32x4 rsrc, const char* lds, uint32_t voffset) {
  uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(i32x4 rsrc, const char* lds, uint32_t voffset) {
  uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// Direct buffer-to-LDS fill of a PTile<R, C, P>.  Each 64-lane load fills
// 1 KiB of consecutive LDS, so lane i fetches the global chunk that belongs at
// its LDS position (pad slots fetch a repeat of the row's last chunk).  The NW
// waves share the kBlocks blocks; a wave's per-lane byte offsets depend only
// on the lane and the row pitch, so they are formed once (init) and each tile
// only moves the buffer base.
template <int R, int C, int NW, int P = 1>
struct TileFill {
  static constexpr int kBlocks = PTile<R, C, P>::kBlocks;
  static constexpr int kPer = (kBlocks + NW - 1) / NW;
  uint32_t voff[kPer];
  int w;
  static_assert((NW & (NW - 1)) == 0, "power-of-two wave count");
  __device__ void init(uint32_t row_bytes, int tid) {
    // tid < NW * 64: the mask changes nothing but tells the compiler that
    // w < NW, so the per-block bounds tests of fill() that always pass fold
    w = uniform(tid >> 6) & (NW - 1);
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int p = (w + NW * i) * 64 + lane;
      int row = p / (C + P), c = min(p % (C + P), C - 1);
      voff[i] = row * row_bytes + c * 16;
    }
  }
  // number of load instructions this wave issues per fill
  __device__ int count() const { return kBlocks / NW + (w < kBlocks % NW ? 1 : 0); }
  // rows of the tile start at src; reads at or past `bytes` return zero
  __device__ void fill(const void* src, uint32_t bytes, char* tile) const {
    const i32x4 rs = make_rsrc(src, bytes);
#pragma unroll
    for (int i = 0; i < kPer; ++i) fill_part(i, rs, tile);
  }
  // the i-th of this wave's loads of a fill (i < kPer) from resource rs
  __device__ void fill_part(int i, i32x4 rs, char* tile) const {
    const int blk = w + NW * i;
    if (kBlocks % NW == 0 || blk < kBlocks) dma_b128(rs, tile + blk * 1024, voff[i]);
  }
};

// 64 consecutive 4-byte values from src[i0 ..] into LDS (one wave; values
// past `n` read as zero).
__device__ __forceinline__ void row64_to_lds(const void* src, int i0, int n, char* dst, int lane) {
  const i32x4 rs = make_rsrc((const char*)src + (int64_t)i0 * 4, (uint32_t)(n - i0) * 4);
  dma_b32(rs, dst, lane * 4);
}

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt holds six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most n vector-memory operations of this wave are in flight
// (n uniform across the wave, 0 <= n < 64).  s_waitcnt takes an immediate,
// hence the table; expcnt and lgkmcnt are left at their maxima.
__device__ __forceinline__ void wait_vmem_le(int n) {
#define BWATTN_VMCNT(k) \
  case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | 0x0F70); break;
  switch (uniform(n)) {
    BWATTN_VMCNT(0) BWATTN_VMCNT(1) BWATTN_VMCNT(2) BWATTN_VMCNT(3) BWATTN_VMCNT(4) BWATTN_VMCNT(5)
    BWATTN_VMCNT(6) BWATTN_VMCNT(7) BWATTN_VMCNT(8) BWATTN_VMCNT(9) BWATTN_VMCNT(10) BWATTN_VMCNT(11)
    BWATTN_VMCNT(12) BWATTN_VMCNT(13) BWATTN_VMCNT(14) BWATTN_VMCNT(15) BWATTN_VMCNT(16) BWATTN_VMCNT(17)
    BWATTN_VMCNT(18) BWATTN_VMCNT(19) BWATTN_VMCNT(20) BWATTN_VMCNT(21) BWATTN_VMCNT(22) BWATTN_VMCNT(23)
    BWATTN_VMCNT(24) BWATTN_VMCNT(25) BWATTN_VMCNT(26) BWATTN_VMCNT(27) BWATTN_VMCNT(28) BWATTN_VMCNT(29)
    BWATTN_VMCNT(30) BWATTN_VMCNT(31)
    default: __builtin_amdgcn_s_waitcnt(0); break;
  }
#undef BWATTN_VMCNT
}


__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// N (LDS read, MFMA) pairs with the read of pair i issued LA pairs ahead of
// the MFMA that consumes it: rd(i) returns operand i, mm(i, x) issues MFMA i.
// Scheduling fences hold that order; left alone, the compiler tends to reuse
// one register and wait on every read, which leaves the matrix core waiting
// on LDS latency.
template <int N, int LA, class Rd, class Mm>
__device__ __forceinline__ void lds_mfma_pipe(Rd&& rd, Mm&& mm) {
  decltype(rd(0)) r[N];
#pragma unroll
  for (int i = 0; i < LA && i < N; ++i) r[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i + LA < N) r[i + LA] = rd(i + LA);
    mm(i, r[i]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// lds_mfma_pipe with M vector-ALU pieces vc(0..M-1) spread evenly between
// the N MFMAs: the pieces of a step issue while its MFMA runs.
template <int N, int LA, int M, class Rd, class Mm, class Vc>
__device__ __forceinline__ void lds_mfma_pipe_mixed(Rd&& rd, Mm&& mm, Vc&& vc) {
  decltype(rd(0)) r[N];
#pragma unroll
  for (int i = 0; i < LA && i < N; ++i) r[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i + LA < N) r[i + LA] = rd(i + LA);
    mm(i, r[i]);
#pragma unroll
    for (int j = i * M / N; j < (i + 1) * M / N; ++j) vc(j);
  }
  __builtin_amdgcn_sched_barrier(0);
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

// Loads from a table this kernel only reads, at a wave-uniform address,
// through the scalar cache, waiting for the result in the same asm block.
// The compiler makes plain loads from these tables vector loads (the
// buffer-to-LDS asm may write memory, as far as it knows), and the zero
// vector-memory count it then waits for would also wait for every
// buffer-to-LDS load in flight.  Call them where no LDS read is in flight
// that the wait would stall on.
__device__ __forceinline__ int2 scalar_load(const int2* p) {
  const uint64_t a = ((uint64_t)(uint32_t)uniform((int)(uint32_t)(uintptr_t)p)) |
                     ((uint64_t)(uint32_t)uniform((int)(uint32_t)((uintptr_t)p >> 32)) << 32);
  uint64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(a));
  return make_int2((int)(uint32_t)v, (int)(uint32_t)(v >> 32));
}
__device__ __forceinline__ int4 scalar_load(const int4* p) {
  const uint64_t a = ((uint64_t)(uint32_t)uniform((int)(uint32_t)(uintptr_t)p)) |
                     ((uint64_t)(uint32_t)uniform((int)(uint32_t)((uintptr_t)p >> 32)) << 32);
  i32x4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(a));
  return make_int4(v[0], v[1], v[2], v[3]);
}

// Segment-id range of rows [r0, r0 + rows) from the 32-row block ranges.
// (r0 and rows are uniform across the wave; the loads are scalar.)
__device__ __forceinline__ int2 seg_range(const int2* blk, int nblk, int r0, int rows) {
  r0 = uniform(r0);
  rows = uniform(rows);
  int b0 = r0 >> 5, b1 = min(nblk, (r0 + rows + 31) >> 5);
  int2 acc = scalar_load(blk + b0);
  for (int k = b0 + 1; k < b1; ++k) acc = range_union(acc, scalar_load(blk + k));
  return acc;
}

// Segment range of 64-row tile t, and of 128-row tile t (64-row tiles 2t and
// 2t + 1, one 16-byte scalar load), from a row of the per-64-row table (its
// padding entries make the pair read safe at the last tile).
__device__ __forceinline__ int2 tile64_range(const int2* t64b, int t) { return scalar_load(t64b + uniform(t)); }
__device__ __forceinline__ int2 tile128_range(const int2* t64b, int t) {
  const int4 v = scalar_load((const int4*)(t64b + 2 * uniform(t)));
  return make_int2(min(v.x, v.z), max(v.y, v.w));
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
  int desc;  // natural order (ct == 0) only, nonzero: visit hi-1 down to lo
  int step, t;
  int run_hi;  // ascending walks: the tiles t+1 .. run_hi-1 that are useful follow t in order (0 once ended)
  const int2* blk;
  int nblk, rows;
  int2 own;
  __device__ bool useful(int tile) const {
    return blk == nullptr || ranges_meet(seg_range(blk, nblk, tile * rows, rows), own);
  }
  __device__ void seek(int after) {
    run_hi = desc ? 0 : hi;
    if (ct == 0 && blk == nullptr) {  // natural order, every tile useful
      int c = desc ? after - 1 : after + 1;
      t = (c >= lo && c < hi) ? c : -1;
      if (t < 0) run_hi = 0;
      return;
    }
    if (ct == 0) {
      if (desc) {
        for (int c = after - 1; c >= lo; --c)
          if (useful(c)) { t = c; return; }
      } else {
        for (int c = after + 1; c < hi; ++c)
          if (useful(c)) { t = c; return; }
      }
      t = -1;
      run_hi = 0;
      return;
    }
    while (step < nc) {
      int c = r + dir * step;
      if (c < 0) c += nc;
      if (c >= nc) c -= nc;
      int c1 = min(hi, (c + 1) * ct);
      run_hi = c1;
      for (int x = max(max(lo, c * ct), after + 1); x < c1; ++x)
        if (useful(x)) { t = x; return; }
      ++step;
      after = -1;
    }
    t = -1;
    run_hi = 0;
  }
  __device__ void start() {
    step = 0;
    seek(ct == 0 && desc ? hi : lo - 1);
  }
  // the common case (the next tile of the same run) without the search
  __device__ void next() {
    if (t + 1 < run_hi && useful(t + 1)) {
      ++t;
      return;
    }
    seek(t);
  }
};

// Set a walk's range from a range-table entry: the per-tile segment test
// (blk) is kept only for ranges marked sparse.
__device__ __forceinline__ void walk_range(TileWalk& w, int2 r, const int2* blk) {
  w.lo = r.x & (kRangeSparse - 1);
  w.hi = r.y;
  w.blk = (r.x & kRangeSparse) ? blk : nullptr;
}

// Software pipeline over the tile walk with an NSTAGE ring of LDS buffers
// (ring[i] = base + i * stride), in one of two orders:
//  - LATE = false: a wave issues its loads of tile t + NSTAGE - 1 (into the
//    slot of tile t - 1, free since the last barrier) before computing tile t;
//  - LATE = true (NSTAGE >= 3): it issues them after computing tile t.  This
//    lets the waves that finish first feed the load path while the others
//    still compute, instead of every wave stalling at the top of the step
//    until the path has taken the burst.
// Then it waits for its loads of tile t + 1 and meets the others at the
// barrier.  Waits are explicit: `per_tile` is the number of vector-memory
// instructions this wave issues per load(t, buf) call.
//   load(t, buf):    issue the loads of tile t into buf
//   compute(t, buf): use tile t in buf
template <int NSTAGE, bool LATE, class Load, class Compute>
__device__ __forceinline__ void run_pipeline(TileWalk walk, int per_tile, char* base, int stride, Load&& load,
                                             Compute&& compute) {
  static_assert(NSTAGE >= 2 && (!LATE || NSTAGE >= 3), "the slot of tile t - 1 takes tile t + NSTAGE - 1");
  TileWalk ahead = walk;  // walk position of the newest tile issued
  int issued = 0;         // tiles issued beyond the one being computed
  if (walk.t >= 0) load(uniform(walk.t), base);
  for (int st = 1; st < NSTAGE - 1; ++st) {
    if (ahead.t >= 0) ahead.next();
    if (ahead.t >= 0) {
      load(uniform(ahead.t), base + st * stride);
      ++issued;
    }
  }
  wait_vmem_le(issued * per_tile);
  __syncthreads();
  int cur = 0;
  auto issue_next = [&]() {
    if (ahead.t >= 0) ahead.next();
    if (ahead.t >= 0) {
      const int fill = cur == 0 ? NSTAGE - 1 : cur - 1;
      load(uniform(ahead.t), base + fill * stride);
      ++issued;
    }
  };
  while (walk.t >= 0) {
    TileWalk nx = walk;
    nx.next();
    if (!LATE) issue_next();
    compute(uniform(walk.t), (const char*)(base + cur * stride));
    if (LATE) issue_next();
    if (nx.t >= 0) --issued;
    wait_vmem_le(issued * per_tile);
    __syncthreads();
    cur = cur + 1 == NSTAGE ? 0 : cur + 1;
    walk = nx;
  }
}

// As run_pipeline<NSTAGE, true>, but the loads of tile t + NSTAGE - 1 (into
// the slot of tile t - 1, free since the last barrier) go out from inside
// compute(t, buf, issue), which calls issue(0) and then issue(1) exactly once
// each per tile, at points of its choosing; issue(p) calls load(t', buf', p)
// for the next tile.  A wave that issues between its own MFMA phases takes
// the load path's stall while the other wave of its SIMD keeps the matrix
// unit busy, and two parts spread the stall.
template <int NSTAGE, class Load, class Compute>
__device__ __forceinline__ void run_pipeline_mid(TileWalk walk, int per_tile, char* base, int stride, Load&& load,
                                                 Compute&& compute) {
  static_assert(NSTAGE >= 2, "the slot of tile t - 1 takes tile t + NSTAGE - 1");
  TileWalk ahead = walk;
  int issued = 0;
  if (walk.t >= 0) { load(uniform(walk.t), base, 0); load(uniform(walk.t), base, 1); }
  for (int st = 1; st < NSTAGE - 1; ++st) {
    if (ahead.t >= 0) ahead.next();
    if (ahead.t >= 0) {
      load(uniform(ahead.t), base + st * stride, 0);
      load(uniform(ahead.t), base + st * stride, 1);
      ++issued;
    }
  }
  wait_vmem_le(issued * per_tile);
  __syncthreads();
  int cur = 0;
  auto issue_next = [&](int part) {
    if (part == 0) {
      if (ahead.t >= 0) ahead.next();
      if (ahead.t >= 0) ++issued;
    }
    if (ahead.t >= 0) {
      const int fill = cur == 0 ? NSTAGE - 1 : cur - 1;
      load(uniform(ahead.t), base + fill * stride, part);
    }
  };
  while (walk.t >= 0) {
    TileWalk nx = walk;
    nx.next();
    compute(uniform(walk.t), (const char*)(base + cur * stride), issue_next);
    if (nx.t >= 0) --issued;
    if constexpr (NSTAGE == 2)
      wait_vmem_le<0>();  // only tile t + 1's loads can be in flight
    else
      wait_vmem_le(issued * per_tile);
    __syncthreads();
    cur = cur + 1 == NSTAGE ? 0 : cur + 1;
    walk = nx;
  }
}

}  // namespace bwattn
