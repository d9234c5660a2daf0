// extra.hip -- extra edges of the sparse support: keys listed per query that join
// what sortLSH selects (Appendix C of the ELSAA paper augments the LSH support,
// Omega = Omega_LSH u Omega_safe with Omega_safe,ij ~ Bernoulli(p); the random
// draw is the caller's and the edges come in as E keys per query, -1 padded).
// The support is a set, so every kept pair is one the sortLSH support does not
// already hold and that the query's list does not repeat.
//
//   extra_prep_kernel     per listed entry: is it a key the query may see, its
//                         first occurrence in the list, and outside the sortLSH
//                         support (same causal leaf, or a shared block at the
//                         level where query and key part, in any round)? Writes
//                         the kept keys per query (-1 otherwise) and, for the
//                         backward, (key, query) pairs with key N for the rest.
//   radix_*_kernel        stable LSD radix sort (8-bit digits) of those pairs by
//                         key, per head: the queries of each key end up listed
//                         in ascending order, so the key-side sums below run in a
//                         fixed order (no atomics on gradients).
//   extra_fwd_kernel      per query: the softmax partial (normalized output and
//                         log-sum-exp) over its kept keys, merged like the
//                         sortLSH blocks' partials.
//   extra_bwd_q_kernel    per query: the dQ part sum_j dS_ij (K_j - Q_i).
//   extra_bwd_k_kernel    per key: the dK and dV parts over the queries that kept
//                         it (found by binary search in the sorted pairs).
//
// The gather kernels give each row D/8 lanes holding 8 channels each; dot
// products are reduced across those lanes with butterfly shuffles. The work is a
// gather of E rows per query (or per key): bound by memory latency and HBM, not
// by arithmetic, so there is nothing here for the matrix cores.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

constexpr int kSortTile = 2048;  // elements per radix tile (256 threads x 8)

// Sum over the LPR lanes of a row group (aligned groups of LPR lanes).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ void __launch_bounds__(256)
    extra_prep_kernel(const int32_t* __restrict__ extra, const int32_t* __restrict__ qbid,
                      const int32_t* __restrict__ kbid, int N, int E, int EP, int causal, int s,
                      int levels, int rounds, int32_t* __restrict__ jq, int32_t* __restrict__ skey,
                      int32_t* __restrict__ sval) {
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int per_wave = 64 / EP, e = lane % EP;
  const int i = (blockIdx.x * 4 + (threadIdx.x >> 6)) * per_wave + lane / EP;
  const bool row = i < N, here = row && e < E;
  const size_t at = ((size_t)bh * N + (row ? i : 0)) * E + e;
  const int j = here ? extra[at] : -1;
  bool keep = here && j >= 0 && j < N && (!causal || j <= i);
  // Only the first occurrence of a key in the list counts (uniform loop: every
  // lane takes part in the shuffles).
  const int base = lane - e;
  for (int t = 0; t < EP - 1; ++t) {
    const int jt = __shfl(j, base + t);
    keep = keep && !(t < e && jt == j);
  }
  if (keep) {
    const int nord = causal ? rounds * levels : rounds;
    if (causal && (i ^ j) < s) {
      keep = false;  // the query's causal leaf holds every key of its block up to it
    } else {
      // (causal: the level where i and j part, i in the future half, j in the past)
      const int lev = causal ? (31 - __clz(N)) - 1 - (31 - __clz(i ^ j)) : 0;
      for (int r = 0; r < rounds && keep; ++r) {
        const size_t o = ((size_t)bh * nord + (causal ? r * levels + lev : r)) * N;
        keep = qbid[o + i] != kbid[o + j];
      }
    }
  }
  if (here) {
    jq[at] = keep ? j : -1;
    if (skey) {
      skey[at] = keep ? j : N;
      sval[at] = i;
    }
  }
}

// Digit counts of one tile: table[bh][digit][tile].
__global__ void __launch_bounds__(256)
    radix_hist_kernel(const int32_t* __restrict__ keys, int M, int shift, int tiles,
                      int32_t* __restrict__ table) {
  __shared__ int h[256];
  const int bh = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int32_t* k = keys + (size_t)bh * M;
#pragma unroll
  for (int r = 0; r < kSortTile / 256; ++r) {
    const int idx = tile * kSortTile + r * 256 + tid;
    if (idx < M) atomicAdd(&h[(k[idx] >> shift) & 255], 1);
  }
  __syncthreads();
  table[((size_t)bh * 256 + tid) * tiles + tile] = h[tid];
}

// Exclusive prefix sum over a head's table in (digit, tile) order: the output
// position of each tile's first element of each digit.
__global__ void __launch_bounds__(256) radix_scan_kernel(int32_t* __restrict__ table, int tiles) {
  __shared__ int part[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int n = 256 * tiles, per = (n + 255) / 256;
  int32_t* t = table + (size_t)bh * n;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int x = lo; x < hi; ++x) sum += t[x];
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int x = lo; x < hi; ++x) {
    const int c = t[x];
    t[x] = run;
    run += c;
  }
}

// Stable scatter of one tile: the tile's elements go in order, 256 at a time;
// within a wave an element's rank among the lanes with the same digit comes from
// eight ballots, and the waves of a round are placed in wave order.
__global__ void __launch_bounds__(256)
    radix_scatter_kernel(const int32_t* __restrict__ kin, const int32_t* __restrict__ vin, int M,
                         int shift, int tiles, const int32_t* __restrict__ table,
                         int32_t* __restrict__ kout, int32_t* __restrict__ vout) {
  __shared__ int run[256];
  __shared__ int wc[4][256];
  __shared__ int wb[4][256];
  const int bh = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  run[tid] = table[((size_t)bh * 256 + tid) * tiles + tile];
#pragma unroll
  for (int x = 0; x < 4; ++x) wc[x][tid] = 0;
  __syncthreads();
  const size_t hb = (size_t)bh * M;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < kSortTile / 256; ++r) {
    const int idx = tile * kSortTile + r * 256 + tid;
    const bool valid = idx < M;
    const int key = valid ? kin[hb + idx] : 0;
    const int val = valid ? vin[hb + idx] : 0;
    const int dg = (key >> shift) & 255;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const unsigned long long bb = __ballot((dg >> b) & 1);
      peers &= ((dg >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) wc[w][dg] = __popcll(peers);
    __syncthreads();
    {
      const int c0 = wc[0][tid], c1 = wc[1][tid], c2 = wc[2][tid], c3 = wc[3][tid];
      const int t = run[tid];
      wb[0][tid] = t;
      wb[1][tid] = t + c0;
      wb[2][tid] = t + c0 + c1;
      wb[3][tid] = t + c0 + c1 + c2;
      run[tid] = t + c0 + c1 + c2 + c3;
#pragma unroll
      for (int x = 0; x < 4; ++x) wc[x][tid] = 0;
    }
    __syncthreads();
    if (valid) {
      const int pos = wb[w][dg] + rank;
      kout[hb + pos] = key;
      vout[hb + pos] = val;
    }
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
    extra_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                     const int32_t* __restrict__ jq, int N, int E, float scale,
                     T* __restrict__ Ox, float* __restrict__ Lx) {
  constexpr int LPR = D / 8, RPB = 256 / LPR, EB = 4;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int i = blockIdx.x * RPB + tid / LPR, c8 = (tid % LPR) * 8;
  const bool row = i < N;
  const size_t hb = (size_t)bh * N;
  const size_t qrow = (hb + (row ? i : 0)) * D + c8;
  float qv[8];
  load8(Q + qrow, qv);
  const int32_t* js = jq + (hb + (row ? i : 0)) * E;
  const float c2 = scale * kLog2e;
  float m = -INFINITY, l = 0.0f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int e0 = 0; e0 < E; e0 += EB) {
    int j[EB];
    float kv[EB][8], vv[EB][8];
#pragma unroll
    for (int b = 0; b < EB; ++b) j[b] = row && e0 + b < E ? js[e0 + b] : -1;
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const size_t kr = (hb + (j[b] >= 0 ? j[b] : 0)) * D + c8;
      load8(K + kr, kv[b]);
      load8(V + kr, vv[b]);
    }
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      float dot = 0.0f;
#pragma unroll
      for (int x = 0; x < 8; ++x) dot = fmaf(qv[x], kv[b][x], dot);
      dot = group_sum<LPR>(dot);
      if (j[b] >= 0) {
        const float sc = dot * c2, mn = fmaxf(m, sc);
        const float a = __builtin_amdgcn_exp2f(m - mn), p = __builtin_amdgcn_exp2f(sc - mn);
        l = l * a + p;
#pragma unroll
        for (int x = 0; x < 8; ++x) o[x] = o[x] * a + p * vv[b][x];
        m = mn;
      }
    }
  }
  if (row) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] *= inv;
    store8(Ox + qrow, o);
    if (c8 == 0) Lx[hb + i] = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
    extra_bwd_q_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                       const T* __restrict__ dO, const float* __restrict__ lse,
                       const float* __restrict__ rc, const float* __restrict__ rD,
                       const int32_t* __restrict__ jq, int N, int E, float scale,
                       T* __restrict__ dQx) {
  constexpr int LPR = D / 8, RPB = 256 / LPR, EB = 4;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int i = blockIdx.x * RPB + tid / LPR, c8 = (tid % LPR) * 8;
  const bool row = i < N;
  const size_t hb = (size_t)bh * N, ri = hb + (row ? i : 0);
  float qv[8], ov[8];
  load8(Q + ri * D + c8, qv);
  load8(dO + ri * D + c8, ov);
  const float c = rc[ri], lq = lse[ri], dq = rD[ri];
#pragma unroll
  for (int x = 0; x < 8; ++x) ov[x] *= c;
  const int32_t* js = jq + ri * E;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, sig = 0.0f;
  for (int e0 = 0; e0 < E; e0 += EB) {
    int j[EB];
    float kv[EB][8], vv[EB][8];
#pragma unroll
    for (int b = 0; b < EB; ++b) j[b] = row && e0 + b < E ? js[e0 + b] : -1;
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const size_t kr = (hb + (j[b] >= 0 ? j[b] : 0)) * D + c8;
      load8(K + kr, kv[b]);
      load8(V + kr, vv[b]);
    }
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      float sd = 0.0f, dp = 0.0f;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        sd = fmaf(qv[x], kv[b][x], sd);
        dp = fmaf(ov[x], vv[b][x], dp);
      }
      sd = group_sum<LPR>(sd);
      dp = group_sum<LPR>(dp);
      const float p = j[b] >= 0 ? fast_exp(sd * scale - lq) : 0.0f;
      const float ds = p * (dp - dq);
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] = fmaf(ds, kv[b][x], acc[x]);
      sig += ds;
    }
  }
  if (row) {
    // (relative to the query: the query's own sortLSH block adds the support-wide
    // sum of dS times Q_i)
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = (acc[x] - sig * qv[x]) * scale;
    store8(dQx + ri * D + c8, acc);
  }
}

// First position in keys[0, M) holding a value >= v (keys ascending).
__device__ __forceinline__ int lower_bound(const int32_t* keys, int M, int v) {
  int lo = 0, hi = M;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (keys[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
    extra_bwd_k_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                       const T* __restrict__ dO, const float* __restrict__ lse,
                       const float* __restrict__ rc, const float* __restrict__ rD,
                       const int32_t* __restrict__ skey, const int32_t* __restrict__ sval, int M,
                       int N, float scale, T* __restrict__ dKx, T* __restrict__ dVx) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int j = blockIdx.x * RPB + tid / LPR, c8 = (tid % LPR) * 8;
  const bool row = j < N;
  const size_t hb = (size_t)bh * N, rj = hb + (row ? j : 0);
  const int32_t* sk = skey + (size_t)bh * M;
  const int32_t* sv = sval + (size_t)bh * M;
  const int lo = row ? lower_bound(sk, M, j) : 0;
  const int hi = row ? lower_bound(sk, M, j + 1) : 0;
  float kv[8], vv[8];
  load8(K + rj * D + c8, kv);
  load8(V + rj * D + c8, vv);
  float ak[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float av[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // (the lanes of a key share its trip count; the loop runs while any key of the
  // wave has queries left, so the shuffles stay convergent)
  for (int t = lo; __any(t < hi); ++t) {
    const bool act = t < hi;
    const int i = act ? sv[t] : 0;
    const size_t ri = hb + i;
    float qv[8], ov[8];
    load8(Q + ri * D + c8, qv);
    load8(dO + ri * D + c8, ov);
    const float c = rc[ri], lq = lse[ri], dq = rD[ri];
    float sd = 0.0f, dpr = 0.0f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      sd = fmaf(qv[x], kv[x], sd);
      dpr = fmaf(ov[x], vv[x], dpr);
    }
    sd = group_sum<LPR>(sd);
    dpr = group_sum<LPR>(dpr);
    const float p = act ? fast_exp(sd * scale - lq) : 0.0f;
    const float ds = p * (c * dpr - dq), pc = p * c;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      av[x] = fmaf(pc, ov[x], av[x]);
      ak[x] = fmaf(ds, qv[x], ak[x]);
    }
  }
  if (row) {
#pragma unroll
    for (int x = 0; x < 8; ++x) ak[x] *= scale;
    store8(dKx + rj * D + c8, ak);
    store8(dVx + rj * D + c8, av);
  }
}

}  // namespace

ExtraLayout extra_layout(const Problem& pb, bool bwd) {
  ExtraLayout l{};
  if (pb.E == 0) return l;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t BH = (size_t)pb.B * pb.H, N = pb.N, M = N * pb.E;
  size_t off = 0;
  l.jq = off; off += al(sizeof(int32_t) * BH * M);
  l.rows = off; off += al((bwd ? 3 : 1) * BH * N * pb.d * pb.elem);
  if (!bwd) {
    l.lse = off; off += al(sizeof(float) * BH * N);
  } else {
    const size_t tiles = (M + kSortTile - 1) / kSortTile;
    for (int x = 0; x < 4; ++x) {
      l.sort[x] = off;
      off += al(sizeof(int32_t) * BH * M);
    }
    l.table = off; off += al(sizeof(int32_t) * BH * 256 * tiles);
  }
  l.total = off;
  return l;
}

void launch_extra_prep(const Problem& pb, const int32_t* extra, const int32_t* qbid,
                       const int32_t* kbid, int32_t* jq, int32_t* skey, int32_t* sval,
                       hipStream_t st) {
  const int EP = pb.E <= 1 ? 1 : 1 << (32 - __builtin_clz(pb.E - 1));
  const int rows_per_block = 4 * (64 / EP);
  ELSAA_LAUNCH("extra_prep", extra_prep_kernel,
               dim3((pb.N + rows_per_block - 1) / rows_per_block, pb.B * pb.H), dim3(256), 0, st,
               extra, qbid, kbid, pb.N, pb.E, EP, (int)pb.causal, pb.s, pb.levels, pb.rounds, jq,
               skey, sval);
}

void launch_extra_sort(const Problem& pb, int32_t* const (&buf)[4], int32_t* table,
                       const int32_t** keys, const int32_t** vals, hipStream_t st) {
  const int BH = pb.B * pb.H, M = pb.N * pb.E;
  const int tiles = (M + kSortTile - 1) / kSortTile;
  const int bits = 32 - __builtin_clz((unsigned)pb.N);  // keys lie in [0, N]
  int32_t *ki = buf[0], *vi = buf[1], *ko = buf[2], *vo = buf[3];
  for (int shift = 0; shift < bits; shift += 8) {
    ELSAA_LAUNCH("radix_hist", radix_hist_kernel, dim3(tiles, BH), dim3(256), 0, st, ki, M, shift,
                 tiles, table);
    ELSAA_LAUNCH("radix_scan", radix_scan_kernel, dim3(BH), dim3(256), 0, st, table, tiles);
    ELSAA_LAUNCH("radix_scatter", radix_scatter_kernel, dim3(tiles, BH), dim3(256), 0, st, ki, vi,
                 M, shift, tiles, table, ko, vo);
    std::swap(ki, ko);
    std::swap(vi, vo);
  }
  *keys = ki;
  *vals = vi;
}

void launch_extra_fwd(const Problem& pb, const void* Q, const void* K, const void* V,
                      const int32_t* jq, void* Ox, float* Lx, hipStream_t st) {
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      constexpr int RPB = 256 / (D / 8);
      ELSAA_LAUNCH("extra_fwd", (extra_fwd_kernel<T, D>),
                   dim3((pb.N + RPB - 1) / RPB, pb.B * pb.H), dim3(256), 0, st, (const T*)Q,
                   (const T*)K, (const T*)V, jq, pb.N, pb.E, pb.scale, (T*)Ox, Lx);
    });
  });
}

void launch_extra_bwd(const Problem& pb, const void* Q, const void* K, const void* V,
                      const void* dO, const float* lse, const float* rc, const float* rD,
                      const int32_t* jq, const int32_t* skey, const int32_t* sval, void* dQx,
                      void* dKx, void* dVx, hipStream_t st) {
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      constexpr int RPB = 256 / (D / 8);
      const dim3 grid((pb.N + RPB - 1) / RPB, pb.B * pb.H);
      ELSAA_LAUNCH("extra_bwd_q", (extra_bwd_q_kernel<T, D>), grid, dim3(256), 0, st,
                   (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, lse, rc, rD, jq, pb.N,
                   pb.E, pb.scale, (T*)dQx);
      ELSAA_LAUNCH("extra_bwd_k", (extra_bwd_k_kernel<T, D>), grid, dim3(256), 0, st,
                   (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, lse, rc, rD, skey, sval,
                   pb.N * pb.E, pb.N, pb.scale, (T*)dKx, (T*)dVx);
    });
  });
}

}  // namespace elsaa
