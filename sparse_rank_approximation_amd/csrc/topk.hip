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
// One wave per tile of 32 queries streams the key tiles: S^T = K Q^T on MFMA in
// fp32 (lane = query, 16 keys per lane); each query keeps a binary heap in LDS of
// the k best (exact score, key) pairs so far, its root being the worst of them. A
// key whose fp32 score is below the root's exact score by more than the fp32
// rounding bound of its dot product, (d + 8) 2^-23 |Q_i| |K_j|, cannot enter and
// is skipped. The tile's other keys are listed (grouped by query), rescored with
// the fp64 chain by all 64 lanes, two chains per lane at a time, from LDS copies
// of the rows, and offered to their query's heap by one lane per query (replacing
// the root when better). A heap of a strict total order keeps exactly the k best
// of what it is offered, whatever the order, so the sets are exact. At the end
// each query's set is written in ascending key order.
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
    topk_kernel(const T* __restrict__ Q, const T* __restrict__ K, int N, int causal, int ktop,
                int32_t* __restrict__ out) {
  typedef MF<T> M;
  typedef TopkSmem<T, D, KMAX> Sm;
  __shared__ Sm sm;
  const int bh = blockIdx.y, q0 = blockIdx.x * 32;
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


}  // namespace

bool launch_topk(const Problem& pb, const void* Q, const void* K, int ktop, int32_t* out,
                 hipStream_t st, bool dry) {
  bool ok = true;
  const dim3 grid((pb.N + 31) / 32, pb.B * pb.H);
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      auto run = [&](auto kc) {
        constexpr int KMAX = ELSAA_C(kc);
        if (dry) return;
        ELSAA_LAUNCH("topk", (topk_kernel<T, D, KMAX>), grid, dim3(64), 0, st, (const T*)Q,
                     (const T*)K, pb.N, (int)pb.causal, ktop, out);
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
