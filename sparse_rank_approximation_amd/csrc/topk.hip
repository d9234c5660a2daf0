// topk.hip -- exact per-query top-k key selection on Q K^T (the top-k kind of
// sparse selector the ELSAA paper lists next to sortLSH in Section 3; here the
// exact one, without learning).
//
// For query i the candidate keys are every j (or j <= i when causal); the score of
// (i, j) is the fp64 fused-multiply-add chain acc = fma(Q_i[c], K_j[c], acc) over
// c = 0 .. d-1 from +0.0, and the selected set holds the min(k, #candidates) keys
// of largest score, ties to the lower key index (the same definition any other
// correctly rounded fp64 FMA implementation reproduces bit for bit).
//
// Three kernels, none of which keeps a heap:
//   topk_stream_kernel   workgroups of 4 waves (128 queries) stream 64-key tiles
//   (radix passes)       through LDS; each wave forms S^T = K Q^T for its 32
//                        queries on MFMA in fp32 (lane = query). Three radix passes
//                        on the scores' order-preserving bit patterns, 6 bits each,
//                        give the 18-bit prefix (sign, exponent, 9 mantissa bits)
//                        of the k-th largest fp32 score and T_i, the lowest float
//                        with that prefix. At least k keys have an fp32 score
//                        >= T_i, so the exact k-th best score is >= T_i - b (b:
//                        the fp32 dot product's rounding bound (d + 8) 2^-23
//                        |Q_i| max_j |K_j|), and every key of the exact top k has
//                        an fp32 score >= T_i - 2 b.
//   topk_stream_kernel   the same scores once more; the keys at or above
//   (listing pass)       T_i - 2 b are listed per query with their fp32 scores
//                        (at most 320).
//   topk_finish_kernel   one wave per query: F, the k-th largest listed fp32 score;
//                        keys with f > F + 2b are in, keys with f < F - 2b out, and
//                        only the few in between are rescored with the fp64 chain
//                        and ranked exactly (score, then lower index); the set is
//                        written in ascending key order.
// A query whose list overflows (many fp32 scores within 2 b of the threshold:
// large runs of tied keys) marks its 32-query tile, and topk_heap_kernel redoes
// that tile: it streams the key tiles, lists the keys whose fp32 score is not
// provably below its query's current k-th best (a binary heap in LDS of exact
// scores), rescores them with the fp64 chain and offers them to the heap.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

// Heap entries of one query: score and key; "worse" orders by score, then by the
// larger key (which loses a tie). heap[0] is the worst entry.
__device__ __forceinline__ bool worse(double sa, int ja, double sb, int jb) {
  return sa < sb || (sa == sb && ja > jb);
}

// Row stride (elements) of the LDS copies of query and key rows: D + 8 keeps the
// lanes' 16-byte reads of different rows on different banks.
template <typename T>
constexpr int chain_ld(int D) { return D + 8; }

// The fp64 fused-multiply-add chain of two rows in LDS, two chains interleaved
// (independent, so their latencies overlap); each is the exact index-order chain.
template <typename T, int D>
__device__ __forceinline__ void score_chains(const T* q0, const T* k0, const T* q1, const T* k1,
                                             double& a0, double& a1) {
  a0 = 0.0;
  a1 = 0.0;
#pragma unroll 2
  for (int c8 = 0; c8 < D; c8 += 8) {
    float x0[8], y0[8], x1[8], y1[8];
    load8(q0 + c8, x0);
    load8(k0 + c8, y0);
    load8(q1 + c8, x1);
    load8(k1 + c8, y1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a0 = __builtin_fma((double)x0[e], (double)y0[e], a0);
      a1 = __builtin_fma((double)x1[e], (double)y1[e], a1);
    }
  }
}

template <typename T, int D, int KMAX>
struct TopkSmem {
  static constexpr int LDC = chain_ld<T>(D);
  double hs[KMAX][32];   // heap scores, [entry][query]
  int hj[KMAX][32];      // heap keys
  alignas(16) T qs[32][LDC];  // the wave's query rows
  alignas(16) T ks[32][LDC];  // the key tile's rows
  double cs[1024];       // exact scores of the tile's candidates
  short cq[1024], ck[1024];  // candidate (query, key row) pairs, grouped by query
  int off[33];           // start of each query's candidates
  int cnt[2][32];        // candidates per (lane half, query)
  float knorm[32];
};

template <typename T, int D, int KMAX>
__global__ void __launch_bounds__(64)
    topk_heap_kernel(const T* __restrict__ Q, const T* __restrict__ K, int N, int causal,
                     int ktop, const int32_t* __restrict__ redo, int32_t* __restrict__ out) {
  typedef MF<T> M;
  typedef TopkSmem<T, D, KMAX> Sm;
  __shared__ Sm sm;
  const int bh = blockIdx.y, q0 = blockIdx.x * 32;
  if (redo[(size_t)bh * gridDim.x + blockIdx.x] == 0) return;  // (uniform)
  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int i = q0 + col;  // this lane's query
  const bool qvalid = i < N;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;

  // The query's row fragments (B operand), its LDS copy and its norm (fp32 sum of
  // squares of each half, the halves added).
  typename M::frag qf[D / M::KSTEP];
  prefetch_row_frags<T, D>(Qh + (size_t)(qvalid ? i : 0) * D, qf, h);
  float qq = 0.0f;
#pragma unroll
  for (int ks = 0; ks < D / M::KSTEP; ++ks) {
    if constexpr (M::KPL == 8) {
      *reinterpret_cast<typename M::frag*>(&sm.qs[col][ks * 16 + 8 * h]) = qf[ks];
#pragma unroll
      for (int e = 0; e < 8; ++e) qq = fmaf((float)qf[ks][e], (float)qf[ks][e], qq);
    } else {
      sm.qs[col][ks * 2 + h] = qf[ks];
      qq = fmaf(qf[ks], qf[ks], qq);
    }
  }
  qq = sum_halves(qq);
  // Rounding bound of an fp32 dot product of d terms with exact or once-rounded
  // products: (d - 1) 2^-24 sum |q_c k_c| for the sum and d 2^-24 for the
  // products; (d + 8) 2^-23 |q| |k| covers both (Cauchy-Schwarz), the norms being
  // taken 1e-5 larger than computed; 2^-120 covers flushed denormals.
  const double dq = (double)(D + 8) * 0x1p-23 * (double)sqrtf(qq) * 1.00001;

  int count = 0;            // entries in the query's heap (both lanes agree)
  double tau = -INFINITY;   // exact score of the root once the heap is full
  const int nkt = causal ? min(N, q0 + 32) : N;  // keys to visit: [0, nkt)
  // The key tile's rows as A operands, one tile ahead.
  typename M::frag kn[D / M::KSTEP];
  prefetch_row_frags<T, D>(Kh + (size_t)min(col, N - 1) * D, kn, h);
  for (int k0 = 0; k0 < nkt; k0 += 32) {
    // S^T tile (rows = keys k0 .. k0 + 31, columns = queries), the keys' rows to
    // LDS and their norms; then the next tile's rows are requested.
    floatx16 s = zero16();
    typename M::frag kf[D / M::KSTEP];
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks) kf[ks] = kn[ks];
    prefetch_row_frags<T, D>(Kh + (size_t)min(k0 + 32 + col, N - 1) * D, kn, h);
    float kk = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks) {
      s = M::mma(kf[ks], qf[ks], s);
      if constexpr (M::KPL == 8) {
        *reinterpret_cast<typename M::frag*>(&sm.ks[col][ks * 16 + 8 * h]) = kf[ks];
#pragma unroll
        for (int e = 0; e < 8; ++e) kk = fmaf((float)kf[ks][e], (float)kf[ks][e], kk);
      } else {
        sm.ks[col][ks * 2 + h] = kf[ks];
        kk = fmaf(kf[ks], kf[ks], kk);
      }
    }
    kk = sum_halves(kk);
    if (h == 0) sm.knorm[col] = sqrtf(kk) * 1.00001f;
    __syncthreads();
    // Candidates: every valid key while the heap is not full, then those whose
    // fp32 score is not provably below the root's exact score.
    unsigned flags = 0;
    if (qvalid) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = acc_row(v, h), j = k0 + r;
        const bool ok = j < N && !(causal && j > i);
        const double bound = dq * (double)sm.knorm[r] + 0x1p-120;
        if (ok && (count < ktop || (double)s[v] >= tau - bound)) flags |= 1u << v;
      }
    }
    // Offsets of the queries' candidate groups: an inclusive scan of the per-query
    // counts over the 32 queries (lane half 0 holds query col's total).
    {
      const int mine = __popc(flags);
      sm.cnt[h][col] = mine;
      int tot = mine + __shfl_xor(mine, 32, 64);
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const int y = __shfl_up(tot, o, 32);
        if (col >= o) tot += y;
      }
      if (h == 0) sm.off[col + 1] = tot;
      if (lane == 0) sm.off[0] = 0;
    }
    __syncthreads();
    {  // this lane's candidates, after its query's half-0 ones
      int pos = sm.off[col] + (h ? sm.cnt[0][col] : 0);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (flags & (1u << v)) {
          sm.cq[pos] = (short)col;
          sm.ck[pos] = (short)acc_row(v, h);
          ++pos;
        }
    }
    __syncthreads();
    // Exact scores of all candidates, two per lane at a time.
    const int L = sm.off[32];
    for (int e = lane; e < L; e += 128) {
      const int e1 = min(e + 64, L - 1);
      double a0, a1;
      score_chains<T, D>(&sm.qs[sm.cq[e]][0], &sm.ks[sm.ck[e]][0], &sm.qs[sm.cq[e1]][0],
                         &sm.ks[sm.ck[e1]][0], a0, a1);
      sm.cs[e] = a0;
      if (e + 64 < L) sm.cs[e1] = a1;
    }
    __syncthreads();
    // Each query's lane of half 0 offers its candidates to its heap.
    if (h == 0 && qvalid) {
      for (int e = sm.off[col]; e < sm.off[col + 1]; ++e) {
        const double sc = sm.cs[e];
        const int j = k0 + sm.ck[e];
        if (count < ktop) {
          // Append and sift up.
          int p = count++;
          while (p > 0) {
            const int par = (p - 1) >> 1;
            if (!worse(sc, j, sm.hs[par][col], sm.hj[par][col])) break;
            sm.hs[p][col] = sm.hs[par][col];
            sm.hj[p][col] = sm.hj[par][col];
            p = par;
          }
          sm.hs[p][col] = sc;
          sm.hj[p][col] = j;
        } else if (worse(sm.hs[0][col], sm.hj[0][col], sc, j)) {
          // Replace the root and sift down.
          int p = 0;
          for (;;) {
            const int c1 = 2 * p + 1, c2 = c1 + 1;
            if (c1 >= ktop) break;
            int w = c1;
            if (c2 < ktop && worse(sm.hs[c2][col], sm.hj[c2][col], sm.hs[c1][col], sm.hj[c1][col]))
              w = c2;
            if (!worse(sm.hs[w][col], sm.hj[w][col], sc, j)) break;
            sm.hs[p][col] = sm.hs[w][col];
            sm.hj[p][col] = sm.hj[w][col];
            p = w;
          }
          sm.hs[p][col] = sc;
          sm.hj[p][col] = j;
        }
      }
      if (count == ktop) tau = sm.hs[0][col];
    }
    // Half 1 takes half 0's heap state.
    const int pc = __shfl_xor(count, 32, 64);
    const double pt = __shfl_xor(tau, 32, 64);
    if (h == 1) {
      count = pc;
      tau = pt;
    }
    __syncthreads();  // the key tile, the list and knorm are rewritten next
  }

  // The set in ascending key order: entry e goes to position #{entries with a
  // smaller key}; each lane half ranks half of the entries. Positions past the
  // count are -1.
  if (qvalid) {
    int32_t* o = out + ((size_t)bh * N + i) * ktop;
    for (int e = h; e < count; e += 2) {
      const int je = sm.hj[e][col];
      int rank = 0;
      for (int f = 0; f < count; ++f) rank += sm.hj[f][col] < je;
      o[rank] = je;
    }
    for (int e = count + h; e < ktop; e += 2) o[e] = -1;
  }
}


constexpr int kSelBits = 6, kSelBins = 1 << kSelBits;
constexpr int kSelPasses = 3;    // 18 of the 32 bits: the sign, exponent and 9 mantissa bits
constexpr int kListExtra = 64;   // listed keys per query beyond k
constexpr int kStreamWaves = 4;  // waves (of 32 queries) per streaming workgroup
constexpr int kStreamKeys = 64;  // keys per LDS tile

// fp32 -> uint32, monotone (larger float, larger key; -0 just below +0).
__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// The query's fragments (B operand) and the fp32 sum of squares of its row.
template <typename T, int D>
__device__ __forceinline__ float query_frags(const T* row,
                                             typename MF<T>::frag (&qf)[D / MF<T>::KSTEP], int h) {
  typedef MF<T> M;
  prefetch_row_frags<T, D>(row, qf, h);
  float qq = 0.0f;
#pragma unroll
  for (int ks = 0; ks < D / M::KSTEP; ++ks) {
    if constexpr (M::KPL == 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qq = fmaf((float)qf[ks][e], (float)qf[ks][e], qq);
    } else {
      qq = fmaf(qf[ks], qf[ks], qq);
    }
  }
  return sum_halves(qq);
}

template <typename T, int D>
struct StreamSmem {
  static constexpr int LD = tile_ld<T>(D);
  T Ks[kStreamKeys][LD];
  // Per wave and query: radix histogram (a padded row, so that the 32 queries'
  // counters of one bin lie on different banks) or listed-key count.
  int hist[kStreamWaves][32][kSelBins + 1];
};

// Streams the key tiles past the workgroup's 128 queries (4 waves of 32): each
// 64-key tile is loaded once into LDS (its rows for the next tile in flight in
// registers meanwhile) and every wave forms S^T = K Q^T for its 32 queries (lane
// = query, rows = keys) on MFMA in fp32.
//   LIST = false: kSelPasses radix passes over the scores' order bits give each
//     query the prefix of its k-th largest score, then thr = T - 2 b (T the lowest
//     float with that prefix; -inf when the query has at most k candidate keys).
//   LIST = true: the keys whose score reaches thr are listed (at most C), the
//     count is stored, and a 32-query tile with an overflowing list is marked.
template <typename T, int D, bool LIST>
__global__ void __launch_bounds__(64 * kStreamWaves)
    topk_stream_kernel(const T* __restrict__ Q, const T* __restrict__ K, int N, int causal,
                       int ktop, int C, double* __restrict__ thr, int32_t* __restrict__ list,
                       int32_t* __restrict__ cnt, int32_t* __restrict__ redo) {
  typedef MF<T> M;
  typedef StreamSmem<T, D> Sm;
  constexpr int LD = Sm::LD, NT = 64 * kStreamWaves, CH = D / 8;
  constexpr int PIECES = kStreamKeys * CH, PIT = (PIECES + NT - 1) / NT;
  __shared__ Sm sm;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int bh = blockIdx.y, q0 = blockIdx.x * 32 * kStreamWaves;
  const int qw = q0 + 32 * w;  // the wave's first query
  const int i = qw + col;
  const bool qvalid = i < N;
  const T* Kh = K + (size_t)bh * N * D;
  typename M::frag qf[D / M::KSTEP];
  const float qq = query_frags<T, D>(Q + ((size_t)bh * N + (qvalid ? i : 0)) * D, qf, h);
  const int nk = causal ? min(N, q0 + 32 * kStreamWaves) : N;  // keys to visit: [0, nk)
  const int wlast = causal ? min(N, qw + 32) : N;             // this wave's keys: [0, wlast)
  double t = -INFINITY;
  if constexpr (LIST) t = qvalid ? thr[(size_t)bh * N + i] : INFINITY;
  uint32_t pref = 0;  // the k-th largest's order bits found so far
  int krem = ktop;    // its rank among the keys with that prefix
  bool all = false;   // at most k candidates: every one is listed
  float kmax = 0.0f;  // largest squared key norm seen
  constexpr int PASSES = LIST ? 1 : kSelPasses;
  for (int pass = 0; pass < PASSES; ++pass) {
    for (int b = tid; b < kStreamWaves * 32 * (kSelBins + 1); b += NT) (&sm.hist[0][0][0])[b] = 0;
    const int sh = 32 - kSelBits * (pass + 1);  // the digit's lowest bit
    Vec8<T> buf[PIT];
    auto load_tile = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < PIT; ++it) {
        const int piece = tid + NT * it, r = min(piece / CH, kStreamKeys - 1);
        buf[it].load(Kh + (size_t)min(k0 + r, N - 1) * D + (piece % CH) * 8);
      }
    };
    load_tile(0);
    for (int k0 = 0; k0 < nk; k0 += kStreamKeys) {
      __syncthreads();  // the previous tile's reads (and the counters' zeroing) done
#pragma unroll
      for (int it = 0; it < PIT; ++it) {
        const int piece = tid + NT * it;
        if (piece < PIECES) buf[it].store(&sm.Ks[piece / CH][(piece % CH) * 8]);
      }
      __syncthreads();
      if (k0 + kStreamKeys < nk) load_tile(k0 + kStreamKeys);
#pragma unroll
      for (int sub = 0; sub < kStreamKeys / 32; ++sub) {
        const int kb = k0 + 32 * sub;
        if (kb >= wlast) break;  // (uniform: past this wave's last query, causal)
        floatx16 s = zero16();
        float kk = 0.0f;
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks) {
          const typename M::frag kf = row_frag<T>(&sm.Ks[0][0], LD, 32 * sub, 0, ks, lane);
          s = M::mma(kf, qf[ks], s);
          if (!LIST && pass == 0) {
            if constexpr (M::KPL == 8) {
#pragma unroll
              for (int e = 0; e < 8; ++e) kk = fmaf((float)kf[e], (float)kf[e], kk);
            } else {
              kk = fmaf(kf, kf, kk);
            }
          }
        }
        if (!LIST && pass == 0) kmax = fmaxf(kmax, sum_halves(kk));
        // (a subtile wholly inside every query's candidates needs no per-key test)
        const bool full = kb + 32 <= N && (!causal || kb + 32 <= qw + 1);
        if (qvalid && !all) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = kb + acc_row(v, h);
            const bool cand = full || (j < N && !(causal && j > i));
            if constexpr (LIST) {
              if (cand && (double)s[v] >= t) {
                const int p = atomicAdd(&sm.hist[w][col][0], 1);
                if (p < C)
                  reinterpret_cast<int2*>(list)[((size_t)bh * N + i) * C + p] =
                      make_int2(j, __float_as_int(s[v]));
              }
            } else {
              const uint32_t u = order_bits(s[v]);
              if (cand && (pass == 0 || (u >> (sh + kSelBits)) == pref))
                atomicAdd(&sm.hist[w][col][(u >> sh) & (kSelBins - 1)], 1);
            }
          }
        }
      }
    }
    __syncthreads();
    if constexpr (!LIST) {
      // The bin holding the krem-th largest, counted from the top (lane half 0 of
      // each query; half 1 takes the result).
      if (h == 0 && qvalid && !all) {
        int above = 0, b = kSelBins - 1;
        for (; b >= 0; --b) {
          const int c = sm.hist[w][col][b];
          if (above + c >= krem) break;
          above += c;
        }
        if (b < 0) {
          all = true;  // (fewer than krem candidates)
        } else {
          pref = (pref << kSelBits) | (uint32_t)b;
          krem -= above;
        }
      }
      pref = __shfl(pref, col, 64);
      krem = __shfl(krem, col, 64);
      all = __shfl((int)all, col, 64) != 0;
    }
  }
  if constexpr (LIST) {
    if (qvalid && h == 0) {
      const int n = sm.hist[w][col][0];
      cnt[(size_t)bh * N + i] = n;
      if (n > C) redo[(size_t)bh * ((N + 31) / 32) + qw / 32] = 1;
    }
  } else {
    // kmax over the 32 key rows of every tile the wave formed: the largest key norm
    // among its candidates.
    for (int o = 16; o > 0; o >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, o, 64));
    if (qvalid && h == 0) {
      const double b = (double)(D + 8) * 0x1p-23 * (double)sqrtf(qq) * 1.00001 *
                           (double)sqrtf(kmax) * 1.00001 + 0x1p-120;
      const double tt = (double)order_float(pref << (32 - kSelBits * kSelPasses));
      thr[(size_t)bh * N + i] = all ? -INFINITY : tt - 2.0 * b;
      thr[(size_t)(gridDim.y) * N + (size_t)bh * N + i] = b;  // (the bound, for the finish)
    }
  }
}

// One wave per query. The listed keys come with their fp32 scores f; F is the k-th
// largest of those and b the query's rounding bound. A key with f > F + 2b is in
// the exact top k (a key of larger exact score has f > F, and fewer than k have);
// a key with f < F - 2b is out (at least k keys have exact scores >= F - b). Only
// the keys in between (a handful) get their exact score (the fp64 chain); the
// best of them by (score, then lower index) fill the remaining places. The set is
// written in ascending key order (-1 past the candidates). A query whose list
// overflowed is left to the heap kernel.
template <typename T, int D, int C>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4)))
    topk_finish_kernel(const T* __restrict__ Q, const T* __restrict__ K, int N, int ktop,
                       const double* __restrict__ thr, const int32_t* __restrict__ list,
                       const int32_t* __restrict__ cnt, int32_t* __restrict__ out) {
  __shared__ alignas(16) T qs[D];
  __shared__ float fs[C];
  __shared__ int kj[C];
  __shared__ double ex[C];   // exact scores (zone keys only)
  __shared__ int st[C];      // 2: in for sure, 1: zone, 0: out
  __shared__ int sl[C];      // selected
  __shared__ float Fk;
  __shared__ int nsure;
  const int lane = threadIdx.x, bh = blockIdx.y, i = blockIdx.x;
  const size_t qi = (size_t)bh * N + i;
  const int n = cnt[qi];
  if (n > C) return;  // (uniform)
  const int2* li = reinterpret_cast<const int2*>(list) + qi * C;
  const double b2 = 2.0 * thr[(size_t)gridDim.y * N + qi];
  for (int c = lane; c < D / 8; c += 64) copy8(&qs[8 * c], Q + qi * D + 8 * c);
  for (int e = lane; e < n; e += 64) {
    const int2 x = li[e];
    kj[e] = x.x;
    fs[e] = __int_as_float(x.y);
  }
  if (lane == 0) {
    Fk = -INFINITY;
    nsure = 0;
  }
  __syncthreads();
  if (n > ktop) {
    // F: the value whose count of larger values is below k and count of values at
    // least as large is k or more.
    for (int e = lane; e < n; e += 64) {
      const float fe = fs[e];
      int gt = 0, ge = 0;
      for (int g = 0; g < n; ++g) {
        gt += fs[g] > fe;
        ge += fs[g] >= fe;
      }
      if (gt < ktop && ge >= ktop) Fk = fe;  // (every writer writes the same value)
    }
    __syncthreads();
    const double F = (double)Fk;
    for (int e = lane; e < n; e += 64) {
      const double fe = (double)fs[e];
      const int sv = fe > F + b2 ? 2 : fe >= F - b2 ? 1 : 0;
      st[e] = sv;
      if (sv == 2) atomicAdd(&nsure, 1);
      if (sv == 1) {
        const T* kr = K + ((size_t)bh * N + kj[e]) * D;
        double a = 0.0;
#pragma unroll 2
        for (int c8 = 0; c8 < D; c8 += 8) {
          float x[8], y[8];
          load8(&qs[c8], x);
          load8(kr + c8, y);
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) a = __builtin_fma((double)x[e2], (double)y[e2], a);
        }
        ex[e] = a;
      }
    }
    __syncthreads();
    // Zone keys: selected when fewer than k - nsure zone keys beat them.
    const int room = ktop - nsure;
    for (int e = lane; e < n; e += 64) {
      int sel = st[e] == 2;
      if (st[e] == 1) {
        const double se = ex[e];
        const int je = kj[e];
        int better = 0;
        for (int g = 0; g < n; ++g)
          better += st[g] == 1 && (ex[g] > se || (ex[g] == se && kj[g] < je));
        sel = better < room;
      }
      sl[e] = sel;
    }
  } else {
    for (int e = lane; e < n; e += 64) sl[e] = 1;  // at most k candidates: all
  }
  __syncthreads();
  int32_t* o = out + qi * ktop;
  for (int e = lane; e < n; e += 64) {
    if (!sl[e]) continue;
    const int je = kj[e];
    int pos = 0;
    for (int g = 0; g < n; ++g) pos += sl[g] && kj[g] < je;
    o[pos] = je;
  }
  for (int p = min(n, ktop) + lane; p < ktop; p += 64) o[p] = -1;
}

__global__ void __launch_bounds__(256) topk_zero_kernel(int32_t* __restrict__ x, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    x[e] = 0;
}

}  // namespace

// Workspace: thresholds and bounds, list counts, tiles to redo, the lists of (key,
// fp32 score) (sized for k <= 256).
size_t topk_ws_bytes(const Problem& pb) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t q = (size_t)pb.B * pb.H * pb.N, tiles = (size_t)pb.B * pb.H * ((pb.N + 31) / 32);
  return al(2 * q * sizeof(double)) + al(q * sizeof(int32_t)) + al(tiles * sizeof(int32_t)) +
         al(q * (256 + kListExtra) * 2 * sizeof(int32_t));
}

bool launch_topk(const Problem& pb, const void* Q, const void* K, int ktop, int32_t* out,
                 void* ws, hipStream_t st, bool dry) {
  bool ok = true;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int BH = pb.B * pb.H, ntile = (pb.N + 31) / 32;
  const size_t q = (size_t)BH * pb.N;
  char* base = (char*)ws;
  double* thr = (double*)base;
  int32_t* cnt = (int32_t*)(base + al(2 * q * sizeof(double)));
  int32_t* redo = (int32_t*)((char*)cnt + al(q * sizeof(int32_t)));
  int32_t* list = (int32_t*)((char*)redo + al((size_t)BH * ntile * sizeof(int32_t)));
  const dim3 grid(ntile, BH);
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      auto run = [&](auto kc) {
        // (the lists take every k the same room, 256 + kListExtra keys: the room
        // beyond k makes overflows, and so the heap kernel's redo, rare)
        constexpr int KMAX = ELSAA_C(kc), C = 256 + kListExtra;
        if (dry) return;
        ELSAA_LAUNCH("topk_zero", topk_zero_kernel, dim3(std::min(BH * ntile / 256 + 1, 1024)),
                     dim3(256), 0, st, redo, (size_t)BH * ntile);
        const dim3 sgrid((pb.N + 32 * kStreamWaves - 1) / (32 * kStreamWaves), BH);
        ELSAA_LAUNCH("topk_thresh", (topk_stream_kernel<T, D, false>), sgrid,
                     dim3(64 * kStreamWaves), 0, st, (const T*)Q, (const T*)K, pb.N,
                     (int)pb.causal, ktop, C, thr, list, cnt, redo);
        ELSAA_LAUNCH("topk_collect", (topk_stream_kernel<T, D, true>), sgrid,
                     dim3(64 * kStreamWaves), 0, st, (const T*)Q, (const T*)K, pb.N,
                     (int)pb.causal, ktop, C, thr, list, cnt, redo);
        ELSAA_LAUNCH("topk_finish", (topk_finish_kernel<T, D, C>), dim3(pb.N, BH), dim3(64), 0,
                     st, (const T*)Q, (const T*)K, pb.N, ktop, thr, list, cnt, out);
        ELSAA_LAUNCH("topk_redo", (topk_heap_kernel<T, D, KMAX>), grid, dim3(64), 0, st,
                     (const T*)Q, (const T*)K, pb.N, (int)pb.causal, ktop, redo, out);
      };
      if (ktop <= 64) run(std::integral_constant<int, 64>{});
      else if (ktop <= 128) run(std::integral_constant<int, 128>{});
      else if (ktop <= 256) run(std::integral_constant<int, 256>{});
      else ok = false;
    });
  });
  return ok;
}

}  // namespace elsaa
