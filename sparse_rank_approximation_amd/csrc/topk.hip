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
// fp32 (lane = query, 16 keys per lane), then a per-query binary heap in LDS of
// the k best (score, key) pairs so far, its root being the worst of them. A key
// whose fp32 score is below the root's exact score by more than the fp32
// rounding bound of its dot product, (d + 8) 2^-23 |Q_i| |K_j|, cannot enter and
// is skipped; every other key is rescored with the fp64 chain and offered to the
// heap (replacing the root when better). The two lanes of a query take turns on
// its heap. At the end each query's set is written in ascending key order.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

// Heap entries of one query: score and key; "worse" orders by score, then by the
// larger key (which loses a tie). heap[0] is the worst entry.
__device__ __forceinline__ bool worse(double sa, int ja, double sb, int jb) {
  return sa < sb || (sa == sb && ja > jb);
}

template <typename T, int D>
__device__ __forceinline__ double score_chain(const T* q, const T* k) {
  double acc = 0.0;
#pragma unroll 4
  for (int c8 = 0; c8 < D; c8 += 8) {
    float qv[8], kv[8];
    load8(q + c8, qv);
    load8(k + c8, kv);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fma((double)qv[e], (double)kv[e], acc);
  }
  return acc;
}

template <typename T, int D, int KMAX>
__global__ void __launch_bounds__(64)
    topk_kernel(const T* __restrict__ Q, const T* __restrict__ K, int N, int causal, int ktop,
                int32_t* __restrict__ out) {
  typedef MF<T> M;
  __shared__ double hs[KMAX][32];
  __shared__ int hj[KMAX][32];
  __shared__ float knorm[32];
  const int bh = blockIdx.y, q0 = blockIdx.x * 32;
  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int i = q0 + col;  // this lane's query
  const bool qvalid = i < N;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* qrow = Qh + (size_t)(qvalid ? i : 0) * D;

  // The query's row fragments and its norm (fp32 sum of squares of its half,
  // both halves added).
  typename M::frag qf[D / M::KSTEP];
  prefetch_row_frags<T, D>(qrow, qf, h);
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
  qq = sum_halves(qq);
  // Rounding bound of an fp32 dot product of d terms with exact or once-rounded
  // products: (d - 1) 2^-24 sum |q_c k_c| for the sum and d 2^-24 for the
  // products; (d + 8) 2^-23 |q| |k| covers both (Cauchy-Schwarz), the norms being
  // taken 1e-5 larger than computed; 2^-120 covers flushed denormals.
  const double dq = (double)(D + 8) * 0x1p-23 * (double)sqrtf(qq) * 1.00001;

  int count = 0;            // entries in the heap (both lanes of a query agree)
  double tau = -INFINITY;   // exact score of the root once the heap is full
  const int nkt = causal ? min(N, q0 + 32) : N;  // keys to visit: [0, nkt)
  for (int k0 = 0; k0 < nkt; k0 += 32) {
    // S^T tile (rows = keys k0 .. k0 + 31, columns = queries) and the keys' norms.
    floatx16 s = zero16();
    typename M::frag kf[D / M::KSTEP];
    const int krow = min(k0 + col, N - 1);
    prefetch_row_frags<T, D>(Kh + (size_t)krow * D, kf, h);
    float kk = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks) {
      s = M::mma(kf[ks], qf[ks], s);
      if constexpr (M::KPL == 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kk = fmaf((float)kf[ks][e], (float)kf[ks][e], kk);
      } else {
        kk = fmaf(kf[ks], kf[ks], kk);
      }
    }
    kk = sum_halves(kk);
    if (h == 0) knorm[col] = sqrtf(kk) * 1.00001f;
    __syncthreads();
    // The two lanes of a query take turns on its heap.
#pragma unroll
    for (int turn = 0; turn < 2; ++turn) {
      if (h == turn && qvalid) {
        for (int v = 0; v < 16; ++v) {
          const int r = acc_row(v, h), j = k0 + r;
          if (j >= N || (causal && j > i)) continue;
          const double bound = dq * (double)knorm[r] + 0x1p-120;
          if (count == ktop && (double)s[v] < tau - bound) continue;
          const double sc = score_chain<T, D>(qrow, Kh + (size_t)j * D);
          if (count < ktop) {
            // Append and sift up.
            int p = count++;
            while (p > 0) {
              const int par = (p - 1) >> 1;
              if (!worse(sc, j, hs[par][col], hj[par][col])) break;
              hs[p][col] = hs[par][col];
              hj[p][col] = hj[par][col];
              p = par;
            }
            hs[p][col] = sc;
            hj[p][col] = j;
          } else if (worse(hs[0][col], hj[0][col], sc, j)) {
            // Replace the root and sift down.
            int p = 0;
            for (;;) {
              const int c1 = 2 * p + 1, c2 = c1 + 1;
              if (c1 >= ktop) break;
              int w = c1;
              if (c2 < ktop && worse(hs[c2][col], hj[c2][col], hs[c1][col], hj[c1][col])) w = c2;
              if (!worse(hs[w][col], hj[w][col], sc, j)) break;
              hs[p][col] = hs[w][col];
              hj[p][col] = hj[w][col];
              p = w;
            }
            hs[p][col] = sc;
            hj[p][col] = j;
          }
          if (count == ktop) tau = hs[0][col];
        }
      }
      // The other half takes this half's heap state.
      const int pc = __shfl_xor(count, 32, 64);
      const double pt = __shfl_xor(tau, 32, 64);
      if (h != turn) {
        count = pc;
        tau = pt;
      }
    }
    __syncthreads();  // knorm is rewritten by the next tile
  }

  // The set in ascending key order: entry e goes to position #{entries with a
  // smaller key}; each lane half ranks half of the entries. Positions past the
  // count are -1.
  if (qvalid) {
    int32_t* o = out + ((size_t)bh * N + i) * ktop;
    for (int e = h; e < count; e += 2) {
      const int je = hj[e][col];
      int rank = 0;
      for (int f = 0; f < count; ++f) rank += hj[f][col] < je;
      o[rank] = je;
    }
    for (int e = count + h; e < ktop; e += 2) o[e] = -1;
  }
}

template <int KMAX>
constexpr size_t topk_lds() { return (sizeof(double) + sizeof(int)) * KMAX * 32 + 128; }

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
