// select.hip -- sortLSH selection: hash codes and sorted orders (ELSAA paper,
// Section 3.2: queries and keys are hashed, sorted by hash and cut into
// equal-size blocks; causally, per level of the past/future divide-and-conquer).
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

// One thread per (token, tensor): bit b of the code is the sign of the fp64
// fused-multiply-add chain over the row against hyperplane b, in index order
// from +0.0. Correctly rounded FMA in a fixed order makes every bit
// reproducible by any other correctly rounded implementation.
template <typename T>
__global__ void __launch_bounds__(256) hash_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const float* __restrict__ planes,
                                                   uint16_t* __restrict__ qc,
                                                   uint16_t* __restrict__ kc, int H, int N, int d,
                                                   int bits) {
  __shared__ double pl[kMaxHashBits * kMaxDh];
  const int bh = blockIdx.y, h = bh % H;
  for (int i = threadIdx.x; i < bits * d; i += blockDim.x)
    pl[i] = (double)planes[(size_t)h * bits * d + i];
  __syncthreads();
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const T* x = (blockIdx.z ? K : Q) + ((size_t)bh * N + t) * d;
  double acc[kMaxHashBits];
#pragma unroll
  for (int b = 0; b < kMaxHashBits; ++b) acc[b] = 0.0;
  for (int j0 = 0; j0 < d; j0 += 8) {
    float xv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = to_f(x[j0 + e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double xd = (double)xv[e];
#pragma unroll
      for (int b = 0; b < kMaxHashBits; ++b)
        if (b < bits) acc[b] = __builtin_fma(xd, pl[b * d + j0 + e], acc[b]);
    }
  }
  unsigned code = 0;
#pragma unroll
  for (int b = 0; b < kMaxHashBits; ++b)
    if (b < bits && acc[b] > 0.0) code |= 1u << b;
  (blockIdx.z ? kc : qc)[(size_t)bh * N + t] = (uint16_t)code;
}

// Stable counting sort of one segment half by Gray rank (ties by token index).
// Grid: x = segment over all levels (causal: level l has 2^l segments, id =
// 2^l - 1 + g), y = batch*head, z = 0 (queries, future half) / 1 (keys, past
// half). Four waves each take a contiguous quarter of the tokens; counts are
// kept per (wave, bin) so offsets are bin-major, wave-minor, and inside a wave
// 64 tokens at a time are placed with ballots (lanes with equal rank are
// ordered by lane), which keeps the order stable without atomics on positions.
constexpr int kSortWaves = 4;

__global__ void __launch_bounds__(256) sort_kernel(const uint16_t* __restrict__ qc,
                                                   const uint16_t* __restrict__ kc,
                                                   int32_t* __restrict__ qperm,
                                                   int32_t* __restrict__ kperm, int N, int causal,
                                                   int levels, int bits) {
  extern __shared__ int smem[];
  const int nbins = 1 << bits;
  int* cnt = smem;                               // [kSortWaves][nbins]
  int* part = smem + kSortWaves * nbins;         // [256]
  const int bh = blockIdx.y, isk = blockIdx.z;
  int base, count;
  size_t out_off;
  if (causal) {
    const int id = blockIdx.x;
    const int l = 31 - __clz(id + 1);
    const int g = id + 1 - (1 << l);
    const int n = N >> l, half = n >> 1;
    base = g * n + (isk ? 0 : half);
    count = half;
    out_off = (size_t)l * (N / 2) + (size_t)g * half;
  } else {
    base = 0;
    count = N;
    out_off = 0;
  }
  const uint16_t* code = (isk ? kc : qc) + (size_t)bh * N;
  int32_t* out = (isk ? kperm : qperm) + (size_t)bh * perm_stride(N, levels, causal) + out_off;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kSortWaves * nbins; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int per = (count + kSortWaves - 1) / kSortWaves;
  const int beg = min(count, w * per), end = min(count, beg + per);
  for (int t = beg + lane; t < end; t += 64) atomicAdd(&cnt[w * nbins + gray_rank(code[base + t])], 1);
  __syncthreads();

  // Exclusive scan of cnt in (bin, wave) order, written back as start offsets.
  const int E = kSortWaves * nbins;
  const int chunk = (E + blockDim.x - 1) / blockDim.x;
  auto at = [&](int e) -> int& { return cnt[(e % kSortWaves) * nbins + e / kSortWaves]; };
  int s = 0;
  for (int e = tid * chunk; e < min(E, (tid + 1) * chunk); ++e) s += at(e);
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < (int)blockDim.x; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  s = part[tid];
  for (int e = tid * chunk; e < min(E, (tid + 1) * chunk); ++e) {
    const int v = at(e);
    at(e) = s;
    s += v;
  }
  __syncthreads();

  int* off = cnt + w * nbins;
  for (int t0 = beg; t0 < end; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < end;
    const unsigned key = valid ? gray_rank(code[base + t]) : 0u;
    unsigned long long eq = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const unsigned long long m = __ballot(valid && ((key >> b) & 1u));
      eq &= ((key >> b) & 1u) ? m : ~m;
    }
    if (valid) {
      const unsigned long long below = (lane == 0) ? 0ull : (eq & ((1ull << lane) - 1ull));
      const int pos = off[key] + __popcll(below);
      out[pos] = base + t;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (eq >> lane) == 1ull) off[key] += __popcll(eq);
    __builtin_amdgcn_wave_barrier();
  }
}

void launch_select(const Problem& pb, const void* Q, const void* K, const float* planes_s,
                   uint16_t* qc, uint16_t* kc, int32_t* qperm, int32_t* kperm,
                   hipStream_t st) {
  const int BH = pb.B * pb.H;
  dim3 hg((pb.N + 255) / 256, BH, 2);
  if (pb.bf16)
    ELSAA_LAUNCH("hash", hash_kernel<__bf16>, hg, dim3(256), 0, st, (const __bf16*)Q,
                       (const __bf16*)K, planes_s, qc, kc, pb.H, pb.N, pb.d, pb.hash_bits);
  else
    ELSAA_LAUNCH("hash", hash_kernel<float>, hg, dim3(256), 0, st, (const float*)Q,
                       (const float*)K, planes_s, qc, kc, pb.H, pb.N, pb.d, pb.hash_bits);
  const int nseg = pb.causal ? (1 << pb.levels) - 1 : 1;
  const size_t lds = sizeof(int) * ((size_t)kSortWaves * (1 << pb.hash_bits) + 256);
  if (nseg > 0)
    ELSAA_LAUNCH("sort", sort_kernel, dim3(nseg, BH, 2), dim3(256), lds, st, qc, kc, qperm, kperm,
                       pb.N, (int)pb.causal, pb.levels, pb.hash_bits);
}

}  // namespace elsaa
