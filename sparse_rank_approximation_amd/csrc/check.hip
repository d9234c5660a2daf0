// check.hip -- debug check of the selection orders that the sparse kernels use to
// gather rows (elsaa_check_orders, and elsaa_fwd / elsaa_bwd when the environment
// variable ELSAA_CHECK_ORDERS is 1): every entry must be a token of the range its
// position stands for, and each range must hold each of its tokens exactly once.
//
// For one order at a time (round r, level l; q_perm, then k_perm):
//   order_fill_kernel    zeroes the per-token counters (a kernel, not a memset);
//   order_mark_kernel    per entry: a token outside [0, N), or outside its
//                        segment's half (causal: queries the future half
//                        [a + n/2, a + n), keys the past half [a, a + n/2) of the
//                        segment of n = N >> l tokens at a), counts as bad;
//                        otherwise its counter is incremented;
//   order_verify_kernel  per token: its counter must be 1 if the order covers it
//                        (causal: the half it lies in at level l; otherwise
//                        always), else 0; each mismatch counts as bad.
// Counts are integer atomics, so the result does not depend on their order.
//
// finite_count_kernel counts the NaN and infinite entries of a tensor (the
// ELSAA_CHECK_FINITE debug mode of elsaa_fwd / elsaa_bwd). Without it such values
// simply propagate: a non-finite key or value reaches every query whose support
// or low-rank sums include it, a non-finite query only its own row.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

__global__ void __launch_bounds__(256) order_fill_kernel(int32_t* __restrict__ m, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    m[i] = 0;
}

__global__ void __launch_bounds__(256)
    order_mark_kernel(const int32_t* __restrict__ perm, size_t P, size_t off, int len, int N,
                      int lev, int causal, int query, int32_t* __restrict__ mark,
                      int32_t* __restrict__ bad) {
  const int bh = blockIdx.y;
  for (int t = blockIdx.x * 256 + threadIdx.x; t < len; t += gridDim.x * 256) {
    const int v = perm[(size_t)bh * P + off + t];
    int lo = 0, hi = N;
    if (causal) {
      const int n = N >> lev, half = n / 2, a = (t / half) * n;
      lo = query ? a + half : a;
      hi = lo + half;
    }
    if (v < lo || v >= hi) atomicAdd(&bad[bh], 1);
    else atomicAdd(&mark[(size_t)bh * N + v], 1);
  }
}

__global__ void __launch_bounds__(256)
    order_verify_kernel(const int32_t* __restrict__ mark, int N, int lev, int causal, int query,
                        int32_t* __restrict__ bad) {
  const int bh = blockIdx.y;
  const int logN = causal ? 31 - __clz(N) : 0;
  for (int v = blockIdx.x * 256 + threadIdx.x; v < N; v += gridDim.x * 256) {
    const bool future = causal && ((v >> (logN - 1 - lev)) & 1);
    const int want = !causal || future == (query != 0) ? 1 : 0;
    if (mark[(size_t)bh * N + v] != want) atomicAdd(&bad[bh], 1);
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
    finite_count_kernel(const T* __restrict__ x, size_t n, int32_t* __restrict__ count) {
  int c = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    c += isfinite((float)x[i]) ? 0 : 1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(count, c);
}

}  // namespace

void launch_finite_count(const Problem& pb, const void* const* xs, int nx, int32_t* counts,
                         hipStream_t st) {
  const size_t n = (size_t)pb.B * pb.H * pb.N * pb.d;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 2048);
  ELSAA_LAUNCH("check_fill", order_fill_kernel, dim3(1), dim3(256), 0, st, counts, (size_t)nx);
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    for (int i = 0; i < nx; ++i)
      ELSAA_LAUNCH("check_finite", finite_count_kernel<T>, dim3(grid), dim3(256), 0, st,
                   (const T*)xs[i], n, counts + i);
  });
}

size_t check_ws_bytes(const Problem& pb) {
  return ((size_t)pb.B * pb.H * pb.N * sizeof(int32_t) + 255) & ~(size_t)255;
}

void launch_check_orders(const Problem& pb, const int32_t* qperm, const int32_t* kperm,
                         int32_t* bad, int32_t* mark, hipStream_t st) {
  const int BH = pb.B * pb.H;
  const size_t P = perm_stride(pb.N, pb.levels, pb.causal, pb.rounds);
  const int len = pb.causal ? pb.N / 2 : pb.N;
  const int nord = pb.causal ? pb.rounds * pb.levels : pb.rounds;
  const int gx = std::min((pb.N + 255) / 256, 256);
  ELSAA_LAUNCH("check_fill", order_fill_kernel, dim3(1), dim3(256), 0, st, bad, (size_t)BH);
  for (int c = 0; c < nord; ++c) {
    const int lev = pb.causal ? c % pb.levels : 0;
    for (int query = 1; query >= 0; --query) {
      ELSAA_LAUNCH("check_fill", order_fill_kernel, dim3(std::min(BH * gx, 4096)), dim3(256), 0,
                   st, mark, (size_t)BH * pb.N);
      ELSAA_LAUNCH("check_mark", order_mark_kernel, dim3(gx, BH), dim3(256), 0, st,
                   query ? qperm : kperm, P, (size_t)c * len, len, pb.N, lev, (int)pb.causal,
                   query, mark, bad);
      ELSAA_LAUNCH("check_verify", order_verify_kernel, dim3(gx, BH), dim3(256), 0, st, mark,
                   pb.N, lev, (int)pb.causal, query, bad);
    }
  }
}

}  // namespace elsaa
