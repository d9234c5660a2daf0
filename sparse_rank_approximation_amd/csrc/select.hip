// select.hip -- sortLSH selection: hash codes and sorted orders (ELSAA paper,
// Section 3.2: queries and keys are hashed, sorted by hash and cut into
// equal-size blocks; causally, per level of the past/future divide-and-conquer).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

// The sortLSH hyperplanes widened to fp64 once per call, [H][bits][D].
__global__ void __launch_bounds__(256) planes_f64_kernel(const float* __restrict__ planes, int n,
                                                         double* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = (double)planes[i];
}

// Bits P0 .. P0 + NB - 1 of the code of the row at xr (LDS, CH pieces of 16 bytes):
// bit b is the sign of the fp64 fused-multiply-add chain over the row against
// hyperplane b, in index order from +0.0. The hyperplanes are the same for every
// lane and are read with scalar loads (operands in scalar registers).
template <typename T, int D, int P0, int NB>
__device__ __forceinline__ unsigned hash_bits(const uint4* xr, const double* pl) {
  constexpr int CH = D * (int)sizeof(T) / 16, EPP = 16 / (int)sizeof(T);
  if constexpr (NB == 0) {
    return 0u;
  } else {
    double acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0;
    for (int c = 0; c < CH; ++c) {
      const uint4 v = xr[c];
      float xv[EPP];
      if constexpr (sizeof(T) == 2) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[2 * e] = __uint_as_float(w4[e] << 16);
          xv[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
        }
      } else {
        xv[0] = __uint_as_float(v.x);
        xv[1] = __uint_as_float(v.y);
        xv[2] = __uint_as_float(v.z);
        xv[3] = __uint_as_float(v.w);
      }
      double xd[EPP];
#pragma unroll
      for (int e = 0; e < EPP; ++e) xd[e] = (double)xv[e];
      double pv[NB][EPP];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < EPP; ++e) pv[b][e] = pl[(P0 + b) * D + c * EPP + e];
#pragma unroll
      for (int e = 0; e < EPP; ++e)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = __builtin_fma(xd[e], pv[b][e], acc[b]);
    }
    unsigned code = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (acc[b] > 0.0) code |= 1u << (P0 + b);
    return code;
  }
}

// One row per (token, tensor) and two threads per row: wave 0 forms the first
// half of the code's bits and wave 1 the rest, each bit its own chain in the
// order above (correctly rounded FMA in a fixed order makes every bit
// reproducible by any other correctly rounded implementation). The workgroup's
// 64 rows are first copied into LDS with 16-byte row-contiguous loads (row
// stride padded by 16 bytes so that each thread's 16-byte reads of its own row
// are free of bank conflicts). Workgroups of 64 rows (17 KB of LDS at d_h = 128)
// let twice as many share a CU as 128 rows did, so more of one's loads overlap
// another's fp64 chains (144 -> 136 us at the headline workload).
constexpr int kHashRows = 64;
template <typename T, int D, int BITS>
__global__ void __launch_bounds__(2 * kHashRows) hash_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const double* __restrict__ planes,
                                                   uint16_t* __restrict__ qc,
                                                   uint16_t* __restrict__ kc, int H, int N,
                                                   int rounds) {
  constexpr int ROWS = kHashRows, NT = 2 * ROWS, CH = D * (int)sizeof(T) / 16;
  constexpr int RW = D * (int)sizeof(T) / 4 + 4;  // row stride in dwords
  constexpr int IT = ROWS * CH / NT, B0 = (BITS + 1) / 2;
  __shared__ uint4 xs[ROWS * RW / 4];
  __shared__ unsigned hib[ROWS];
  // blockIdx.z = 2 round + (0: queries, 1: keys); round r hashes with its own
  // hyperplanes into its own codes.
  const int bh = blockIdx.y, h = bh % H, tid = threadIdx.x;
  const int isk = blockIdx.z & 1, r = blockIdx.z >> 1;
  const int tok0 = blockIdx.x * ROWS;
  const T* X = (isk ? K : Q) + (size_t)bh * N * D;
  const double* pl = planes + ((size_t)h * rounds + r) * BITS * D;
  {
    uint4 buf[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int p = tid + NT * i, r = p / CH, c = p % CH;
      const int tok = min(tok0 + r, N - 1);
      buf[i] = reinterpret_cast<const uint4*>(X + (size_t)tok * D)[c];
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int p = tid + NT * i, r = p / CH, c = p % CH;
      xs[r * (RW / 4) + c] = buf[i];
    }
  }
  __syncthreads();
  const int row = tid & (ROWS - 1);
  const uint4* xr = &xs[row * (RW / 4)];
  if (tid >= ROWS) hib[row] = hash_bits<T, D, B0, BITS - B0>(xr, pl);  // wave 1
  const unsigned lo = tid < ROWS ? hash_bits<T, D, 0, B0>(xr, pl) : 0u;
  __syncthreads();
  const int t = tok0 + row;
  if (tid < ROWS && t < N)
    (isk ? kc : qc)[((size_t)bh * rounds + r) * N + t] = (uint16_t)(lo | hib[row]);
}

// Stable counting sort of one segment half by Gray rank (ties by token index).
// Grid: x = segment over all levels (causal: level l has 2^l segments, id =
// 2^l - 1 + g), y = batch*head, z = 0 (queries, future half) / 1 (keys, past
// half). Four waves each take a contiguous quarter of the tokens; counts are
// kept per (wave, bin) so offsets are bin-major, wave-minor, and inside a wave
// 64 tokens at a time are placed with ballots (lanes with equal rank are
// ordered by lane), which keeps the order stable without atomics on positions.
constexpr int kSortWaves = 4;

template <bool STAGED>
__global__ void __launch_bounds__(256) sort_kernel(const uint16_t* __restrict__ qc,
                                                   const uint16_t* __restrict__ kc,
                                                   int32_t* __restrict__ qperm,
                                                   int32_t* __restrict__ kperm, int N, int causal,
                                                   int levels, int bits, int rounds) {
  extern __shared__ int smem[];
  const int nbins = 1 << bits;
  int* cnt = smem;                               // [kSortWaves][nbins]
  int* part = smem + kSortWaves * nbins;         // [kSortWaves] wave totals
  // STAGED: the segment's codes are first copied into LDS (after 256 words for
  // the wave totals) with 16-byte loads all in flight, and both passes read them
  // there.
  uint16_t* cs = reinterpret_cast<uint16_t*>(part + 256);
  const int bh = blockIdx.y, isk = blockIdx.z & 1, rd = blockIdx.z >> 1;  // z = 2 round + isk
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
  const uint16_t* code = (isk ? kc : qc) + ((size_t)bh * rounds + rd) * N;
  int32_t* out = (isk ? kperm : qperm) + (size_t)bh * perm_stride(N, levels, causal, rounds) +
                 (size_t)rd * perm_stride(N, levels, causal) + out_off;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kSortWaves * nbins; i += blockDim.x) cnt[i] = 0;
  if constexpr (STAGED)  // count and base are multiples of 8
    for (int i = tid; i < count / 8; i += blockDim.x)
      reinterpret_cast<uint4*>(cs)[i] = reinterpret_cast<const uint4*>(code + base)[i];
  __syncthreads();
  auto code_at = [&](int t) -> unsigned {
    if constexpr (STAGED) return cs[t];
    else return code[base + t];
  };
  const int per = (count + kSortWaves - 1) / kSortWaves;
  const int beg = min(count, w * per), end = min(count, beg + per);
  for (int t = beg + lane; t < end; t += 64) atomicAdd(&cnt[w * nbins + gray_rank(code_at(t))], 1);
  __syncthreads();

  // Exclusive scan of cnt in (bin, wave) order, written back as start offsets.
  const int E = kSortWaves * nbins;
  const int chunk = (E + blockDim.x - 1) / blockDim.x;
  auto at = [&](int e) -> int& { return cnt[(e % kSortWaves) * nbins + e / kSortWaves]; };
  int s = 0;
  for (int e = tid * chunk; e < min(E, (tid + 1) * chunk); ++e) s += at(e);
  // Exclusive prefix of the per-thread sums: inclusive scan inside each wave
  // (shuffles), then the totals of the earlier waves.
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) part[w] = incl;
  __syncthreads();
  for (int i = 0; i < w; ++i) incl += part[i];
  s = incl - s;
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
    const unsigned key = valid ? gray_rank(code_at(t)) : 0u;
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

// The same sort for the causal levels whose segment halves hold at most
// kSmallHalf tokens: one wave per segment half, four to a workgroup, with no
// barrier across waves (segment id = first_id + 4 blockIdx.x + wave; ids past the
// last segment leave their wave idle). Counts per bin, their exclusive scan and the
// ballot placement are those of sort_kernel for a single wave.
constexpr int kSmallHalf = 512;

__global__ void __launch_bounds__(256) sort_small_kernel(const uint16_t* __restrict__ qc,
                                                         const uint16_t* __restrict__ kc,
                                                         int32_t* __restrict__ qperm,
                                                         int32_t* __restrict__ kperm, int N,
                                                         int levels, int bits, int rounds,
                                                         int first_id, int nseg) {
  extern __shared__ int smem[];
  const int nbins = 1 << bits;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  int* cnt = smem + w * nbins;  // this wave's bins
  const int id = first_id + 4 * blockIdx.x + w;
  if (id >= nseg) return;  // (whole waves: nothing below synchronizes across waves)
  const int bh = blockIdx.y, isk = blockIdx.z & 1, rd = blockIdx.z >> 1;
  const int l = 31 - __clz(id + 1);
  const int g = id + 1 - (1 << l);
  const int n = N >> l, half = n >> 1;
  const int base = g * n + (isk ? 0 : half), count = half;
  const uint16_t* code = (isk ? kc : qc) + ((size_t)bh * rounds + rd) * N + base;
  int32_t* out = (isk ? kperm : qperm) + (size_t)bh * perm_stride(N, levels, true, rounds) +
                 (size_t)rd * perm_stride(N, levels, true) + (size_t)l * (N / 2) + (size_t)g * half;
  for (int i = lane; i < nbins; i += 64) cnt[i] = 0;
  __builtin_amdgcn_wave_barrier();
  unsigned keys[kSmallHalf / 64];
#pragma unroll
  for (int j = 0; j < kSmallHalf / 64; ++j) {
    const int t = 64 * j + lane;
    keys[j] = t < count ? gray_rank(code[t]) : 0u;
  }
#pragma unroll
  for (int j = 0; j < kSmallHalf / 64; ++j)
    if (64 * j + lane < count) atomicAdd(&cnt[keys[j]], 1);
  __builtin_amdgcn_wave_barrier();
  // Exclusive scan of the bins: lane takes a run of per consecutive bins.
  const int per = (nbins + 63) / 64;
  int sum = 0;
  for (int e = lane * per; e < min(nbins, (lane + 1) * per); ++e) sum += cnt[e];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  int run = incl - sum;
  __builtin_amdgcn_wave_barrier();
  for (int e = lane * per; e < min(nbins, (lane + 1) * per); ++e) {
    const int v = cnt[e];
    cnt[e] = run;
    run += v;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < kSmallHalf / 64; ++j) {
    const int t = 64 * j + lane;
    if (64 * j >= count) break;
    const bool valid = t < count;
    const unsigned key = keys[j];
    unsigned long long eq = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const unsigned long long m = __ballot(valid && ((key >> b) & 1u));
      eq &= ((key >> b) & 1u) ? m : ~m;
    }
    if (valid) {
      const unsigned long long below = (lane == 0) ? 0ull : (eq & ((1ull << lane) - 1ull));
      out[cnt[key] + __popcll(below)] = base + t;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (eq >> lane) == 1ull) cnt[key] += __popcll(eq);
    __builtin_amdgcn_wave_barrier();
  }
}

// Scratch of the allocation-free selection (elsaa_select_noalloc): the fp64
// hyperplanes go to this fixed array instead of a caller's workspace. Every GPU
// the library runs on holds its own copy until the process ends; calls on one
// GPU share it, so such calls must not overlap (they would race on it). Nothing
// in it has to start at zero: each call writes all of what it then reads.
constexpr size_t kNoallocScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) double scratch[kNoallocScratchBytes / sizeof(double)];

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    // The device address of this device's copy (in host code `scratch` names a
    // host-side stand-in, not device memory).
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

size_t select_ws_bytes(const Problem& pb) {
  return (sizeof(double) * pb.H * pb.rounds * pb.hash_bits * pb.d + 255) & ~(size_t)255;
}

// Block index of every token in every (round, level) order of a head, as a query
// (qb) and as a key (kb): entry t of order c = r levels + l lies in block
// (t mod half) / s of its segment's half (half = N >> (l + 1) causal, N when not);
// entries of tokens absent from an order (the other half, causal) are not written
// and not read. [B H][rounds levels][N]. The sparse kernels compare these to take
// a pair that an earlier round already holds out of a later round's block.
__global__ void __launch_bounds__(256)
    block_ids_kernel(const int32_t* __restrict__ qperm, const int32_t* __restrict__ kperm, int N,
                     int levels, int causal, int rounds, int s, int32_t* __restrict__ qb,
                     int32_t* __restrict__ kb) {
  const int bh = blockIdx.y;
  const int len = causal ? N / 2 : N;
  const int nord = causal ? rounds * levels : rounds;
  const size_t P = perm_stride(N, levels, causal, rounds);
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < (size_t)nord * len;
       e += (size_t)gridDim.x * 256) {
    const int c = (int)(e / len), t = (int)(e % len);
    const int half = causal ? (N >> ((c % levels) + 1)) : N;
    const int b = (t % half) / s;
    const size_t base = ((size_t)bh * nord + c) * N;
    qb[base + qperm[(size_t)bh * P + e]] = b;
    kb[base + kperm[(size_t)bh * P + e]] = b;
  }
}

size_t block_ids_bytes(const Problem& pb) {
  if (pb.rounds <= 1 && pb.E == 0) return 0;
  const size_t nord = pb.causal ? (size_t)pb.rounds * pb.levels : (size_t)pb.rounds;
  return 2 * sizeof(int32_t) * (size_t)pb.B * pb.H * nord * pb.N;
}

void launch_block_ids(const Problem& pb, const int32_t* qperm, const int32_t* kperm, int32_t* qb,
                      int32_t* kb, hipStream_t st) {
  const size_t nord = pb.causal ? (size_t)pb.rounds * pb.levels : (size_t)pb.rounds;
  const size_t n = nord * (pb.causal ? pb.N / 2 : pb.N);
  if (n == 0 || pb.B * pb.H == 0) return;  // (no level: the leaves need no block index)
  const int gx = (int)std::min<size_t>((n + 255) / 256, 1024);
  ELSAA_LAUNCH("block_ids", block_ids_kernel, dim3(gx, pb.B * pb.H), dim3(256), 0, st, qperm,
               kperm, pb.N, pb.levels, (int)pb.causal, pb.rounds, pb.s, qb, kb);
}

void launch_select(const Problem& pb, const void* Q, const void* K, const float* planes_s,
                   uint16_t* qc, uint16_t* kc, int32_t* qperm, int32_t* kperm, void* ws,
                   hipStream_t st) {
  const int BH = pb.B * pb.H;
  double* pld = (double*)ws;
  const int np = pb.H * pb.rounds * pb.hash_bits * pb.d;
  ELSAA_LAUNCH("planes_f64", planes_f64_kernel, dim3((np + 255) / 256), dim3(256), 0, st, planes_s,
               np, pld);
  const dim3 hg((pb.N + kHashRows - 1) / kHashRows, BH, 2 * pb.rounds);
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      auto run = [&](auto bc) {
        constexpr int BITS = ELSAA_C(bc);
        ELSAA_LAUNCH("hash", (hash_kernel<T, D, BITS>), hg, dim3(2 * kHashRows), 0, st, (const T*)Q,
                     (const T*)K, (const double*)pld, qc, kc, pb.H, pb.N, pb.rounds);
      };
      switch (pb.hash_bits) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 5: run(std::integral_constant<int, 5>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 7: run(std::integral_constant<int, 7>{}); break;
        case 8: run(std::integral_constant<int, 8>{}); break;
        case 9: run(std::integral_constant<int, 9>{}); break;
        case 10: run(std::integral_constant<int, 10>{}); break;
        case 11: run(std::integral_constant<int, 11>{}); break;
        default: run(std::integral_constant<int, kMaxHashBits>{}); break;
      }
    });
  });
  const int nseg = pb.causal ? (1 << pb.levels) - 1 : 1;
  // Causal levels l whose halves N >> (l + 1) hold at most kSmallHalf tokens go to
  // the one-wave-per-segment kernel (segment ids from 2^l_small - 1 on).
  int nbig = nseg;
  if (pb.causal)
    for (int l = 0; l < pb.levels; ++l)
      if ((pb.N >> (l + 1)) <= kSmallHalf) {
        nbig = (1 << l) - 1;
        break;
      }
  const size_t lds = sizeof(int) * ((size_t)kSortWaves * (1 << pb.hash_bits) + 256);
  const size_t seg_codes = sizeof(uint16_t) * (size_t)(pb.causal ? pb.N / 2 : pb.N);
  if (nbig > 0) {
    if (lds + seg_codes <= 64 * 1024)
      ELSAA_LAUNCH("sort", sort_kernel<true>, dim3(nbig, BH, 2 * pb.rounds), dim3(256),
                   lds + seg_codes, st, qc, kc, qperm, kperm, pb.N, (int)pb.causal, pb.levels,
                   pb.hash_bits, pb.rounds);
    else
      ELSAA_LAUNCH("sort", sort_kernel<false>, dim3(nbig, BH, 2 * pb.rounds), dim3(256), lds, st,
                   qc, kc, qperm, kperm, pb.N, (int)pb.causal, pb.levels, pb.hash_bits,
                   pb.rounds);
  }
  if (nseg > nbig)
    ELSAA_LAUNCH("sort_small", sort_small_kernel, dim3((nseg - nbig + 3) / 4, BH, 2 * pb.rounds),
                 dim3(256), sizeof(int) * 4 * ((size_t)1 << pb.hash_bits), st, qc, kc, qperm,
                 kperm, pb.N, pb.levels, pb.hash_bits, pb.rounds, nbig, nseg);
}

}  // namespace elsaa
