// Loss side of masked sequence packing: cross-entropy of every packed token
// row, re-weighted so that each packed example counts as it would unpacked.
//
// Short examples are packed into one training row with the attention masked
// to each example, and the loss is re-weighted so that packed training
// computes what unpacked training with padding computes; naive packing
// would weigh short answers down (zhao9797 page "LWM (Large World Model)",
// 数据 and 训练方法 with its ablation table).  With E examples that have loss
// rows and n_e loss rows in example e, the unpacked objective (each example's
// mean cross-entropy, averaged over examples) is
//   loss = sum_t w_t ce_t,  w_t = 1 / (E n_e(t)),
//   ce_t = logsumexp(x_t) - x_t[y_t],
//   dloss/dx_t = w_t (softmax(x_t) - onehot(y_t)).
//
// Kernels: zero the per-example counters; count loss rows per example
// (integer atomics: exact, so the result does not depend on their order);
// one workgroup forms E and the weights; one workgroup per token row reads
// the row once into registers, reduces max and sum over the workgroup, and
// writes the weighted gradient once (HBM-bound: V bf16 read, V bf16 written
// per row); one workgroup sums the weighted row losses in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace bwattn {

namespace {

__device__ __forceinline__ bool ce_loss_row(const CeArgs& a, int64_t t, int& key) {
  const int y = a.targets[t];
  const int b = (int)(t / a.S);
  const int id = a.seg ? a.seg[t] : 0;
  key = b * a.num_segments + id;
  return y >= 0 && y < a.V && id >= 0 && id < a.num_segments;
}

// sum over the 64 lanes of a wave (xor butterfly)
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

}  // namespace

__global__ void ce_zero_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Loss rows per example.  Packed examples are contiguous, so a wave's loss
// rows mostly share one key: the first lane of each run of equal keys adds
// the run's loss rows with one atomic (runs are cut by rows without loss).
__global__ void ce_count_kernel(CeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lane = threadIdx.x & 63;
  int key = -1;
  bool lr = false;
  if (t < (int64_t)a.B * a.S) lr = ce_loss_row(a, t, key);
  if (!lr) key = -1;
  const int prev = __shfl_up(key, 1, 64);
  const bool start = lr && (lane == 0 || prev != key);
  const uint64_t starts = __ballot(start);
  const uint64_t loss = __ballot(lr);
  if (start) {
    const uint64_t later = lane == 63 ? 0ull : starts & (~0ull << (lane + 1));
    const int end = later ? __ffsll((long long)later) - 1 : 64;  // next run start (exclusive end)
    const uint64_t upto = end == 64 ? ~0ull : ((1ull << end) - 1);
    atomicAdd(a.counts + key, __popcll(loss & upto & (~0ull << lane)));
  }
}

// E = number of examples with a loss row; w_e = 1 / (E n_e) (0 if n_e = 0).
__global__ __launch_bounds__(1024) void ce_weight_kernel(CeArgs a) {
  __shared__ int part[16];
  const int n = a.B * a.num_segments;
  int c = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) c += a.counts[i] > 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  int E = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) E += part[i];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int k = a.counts[i];
    a.weights[i] = k > 0 ? (float)(1.0 / ((double)E * (double)k)) : 0.f;
  }
}

// One workgroup per token row; NCH 16-byte chunks (8 bf16) of the row per
// thread, held in registers as fp32.
template <int NCH>
__global__ __launch_bounds__(kCeThreads) void ce_row_kernel(CeArgs a) {
  __shared__ float red[2][kCeThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t t = blockIdx.x;
  const int nchunks = a.V >> 3;
  int key;
  const bool loss_row = ce_loss_row(a, t, key);
  u32x4* drow = a.dlogits ? (u32x4*)(a.dlogits + t * a.V) : nullptr;
  if (!loss_row) {  // no loss: zero gradient row
    if (drow)
      for (int c = tid; c < nchunks; c += kCeThreads) __builtin_nontemporal_store(u32x4{0, 0, 0, 0}, drow + c);
    if (tid == 0) {
      a.wloss[t] = 0.f;
      if (a.token_ce) a.token_ce[t] = 0.f;
    }
    return;
  }
  const u32x4* row = (const u32x4*)(a.logits + t * a.V);
  float x[NCH][8];
  float m = kNegInf;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + kCeThreads * i;
    const u32x4 v = c < nchunks ? __builtin_nontemporal_load(row + c) : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[i][2 * e] = bf16_lo(v[e]);
      x[i][2 * e + 1] = bf16_hi(v[e]);
      m = fmaxf(m, fmaxf(x[i][2 * e], x[i][2 * e + 1]));
    }
  }
  // row max
  m = wave_max(m);
  if (lane == 0) red[0][wv] = m;
  __syncthreads();
  m = red[0][0];
#pragma unroll
  for (int i = 1; i < kCeThreads / 64; ++i) m = fmaxf(m, red[0][i]);
  // sum of exp(x - m), in base 2
  const float ml2 = m * kLog2e;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += fast_exp2(__builtin_fmaf(x[i][e], kLog2e, -ml2));
  s = wave_sum(s);
  if (lane == 0) red[1][wv] = s;
  __syncthreads();
  s = 0.f;
#pragma unroll
  for (int i = 0; i < kCeThreads / 64; ++i) s += red[1][i];
  const float lse = m + __logf(s);
  const int y = a.targets[t];
  const float xy = bf16_lo((uint32_t)((const uint16_t*)(a.logits + t * a.V))[y]);
  const float w = a.weights[key];
  if (tid == 0) {
    const float ce = lse - xy;
    a.wloss[t] = w * ce;
    if (a.token_ce) a.token_ce[t] = ce;
  }
  if (drow) {
    // g_j = sw softmax(x)_j - sw [j == y], sw = grad_scale w; for sw > 0 the
    // factor folds into the exponent: sw 2^((x - lse) log2e) = 2^(x log2e - c)
    const float sw = a.grad_scale * w;
    const int cy = y >> 3, ey = y & 7;
    auto write = [&](auto&& gfun) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + kCeThreads * i;
        if (c >= nchunks) continue;
        float g[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) g[e] = gfun(x[i][e]);
        if (c == cy) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e == ey) g[e] -= sw;
        }
        const u32x4 o = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                         pack_bf16x2(g[6], g[7])};
        __builtin_nontemporal_store(o, drow + c);
      }
    };
    if (sw > 0.f) {
      const float cc = lse * kLog2e - __log2f(sw);
      write([&](float v) { return fast_exp2(__builtin_fmaf(v, kLog2e, -cc)); });
    } else {
      const float c0 = lse * kLog2e;
      write([&](float v) { return sw * fast_exp2(__builtin_fmaf(v, kLog2e, -c0)); });
    }
  }
}

// loss = sum_t wloss[t], summed in a fixed order in fp64.
__global__ __launch_bounds__(1024) void ce_sum_kernel(CeArgs a) {
  __shared__ double part[16];
  const int64_t n = (int64_t)a.B * a.S;
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += (double)a.wloss[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += part[i];
    *a.loss = (float)tot;
  }
}

hipError_t launch_packed_ce_prologue(const CeArgs& a, hipStream_t st) {
  const int n = a.B * a.num_segments;
  hipLaunchKernelGGL(ce_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.counts, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t N = (int64_t)a.B * a.S;
  hipLaunchKernelGGL(ce_count_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ce_weight_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_packed_ce_rows(const CeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.B * a.S)), block(kCeThreads);
  switch (ce_chunks_per_thread(a.V)) {
    case 2: hipLaunchKernelGGL(ce_row_kernel<2>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(ce_row_kernel<4>, grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL(ce_row_kernel<6>, grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL(ce_row_kernel<8>, grid, block, 0, st, a); break;
    case 10: hipLaunchKernelGGL(ce_row_kernel<10>, grid, block, 0, st, a); break;
    case 12: hipLaunchKernelGGL(ce_row_kernel<12>, grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL(ce_row_kernel<16>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_packed_ce_sum(const CeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(ce_sum_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace bwattn
