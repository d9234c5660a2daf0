// bwd.hip -- backward of the ELSAA operator on gfx950 (training), the chain rule
// through Eq. 4, Eq. 5, the exact block softmaxes of the sparse branch (Section
// 3.2) and the RACE readout (Section 3.1), with the selection held fixed.
//
// With m_i = d_s / (d_s + lambda d_lr + eps), d_s = exp(lse), a_i = <dO_i, O_s,i>,
// b_i = <dO_i, O_lr,i>, dm_i = g_s a_i:
//   sparse branch: upstream c_i dO_i with c_i = g_s m_i and, through the lse,
//     ds_ij = p_ij (<c_i dO_i, V_j> - D_i), D_i = g_s a_i m_i^2;
//   low-rank branch: dnum_i = (g_lr / d_lr,i) dO_i and
//     dd_lr,i = -g_lr b_i / d_lr,i - dm_i lambda m_i^2 / d_s;
//   dlambda = -sum_i dm_i d_lr,i m_i^2 / d_s; dg_s,i = m_i a_i; dg_lr,i = b_i.
// m_i^2 / d_s is evaluated as exp(lse - 2 log(d_s + lambda d_lr + eps)).
//
// dQ_i = scale sum_j dS_ij K_j is formed relative to the query: since p_i sums
// to 1 over the support, sum_j dS_ij = c_i a_i - D_i = g_s a_i m_i (1 - m_i)
// =: sigma_i exactly, so dQ_i = scale (sum_j dS_ij (K_j - Q_i) + sigma_i Q_i).
// Each block stores its part of the first sum (its own block, the causal leaf
// or the only non-causal one, adds sigma_i Q_i). When a query's selected keys
// lie near it, as sortLSH makes them, these parts are small and cancel little
// across levels, so storing them per level in the element type loses little;
// the plain parts sum_j dS_ij K_j share a large component along the keys' mean
// that cancels between levels.
//
// Kernels, in launch order:
//   bwd_rows_kernel      per-row terms above, dg_s, dg_lr, per-block dlambda sums;
//   dlam_reduce_kernel   dlambda per head (fixed order: deterministic);
//   lr_sums + lr_scan    (lowrank.hip) G = sum_i phi(Q_i) dnum_i^T, g = sum_i
//                        phi(Q_i) dd_lr,i per chunk, combined as the exclusive suffix
//                        over chunks (causal) or the total;
//   sparse_bwd3_kernel   per selected block: dQ, dK, dV partials per level slot
//   / sparse_bwd2_kernel (bf16 blocks of 128 with one hash round: sparse_bwd3 on
//   / sparse_bwd_kernel  16-key tiles, 8 waves; other bf16 blocks of at most 128:
//                        sparse_bwd2; else sparse_bwd_kernel, in one launch or a
//                        key launch and a query launch);
//   lr_bwd_q_kernel      query side of the low-rank branch, walking each chunk
//                        forwards with the running key statistics A, z:
//                        dphi(Q_i) = sum_{j<=i} (<dnum_i, V_j> + dd_lr,i) phi(K_j),
//                        then through the features to the low-rank part of dQ;
//   lr_bwd_k_kernel      key side, walking each chunk backwards with the running
//                        query statistics G, g:
//                        dphi(K_j) = sum_{i>=j} (<dnum_i, V_j> + dd_lr,i) phi(Q_i),
//                        dV_j += sum_{i>=j} (phi(Q_i).phi(K_j)) dnum_i: the low-rank
//                        parts of dK, dV;
//   combine_kernel       (merge.hip) adds the sparse partial rows: dQ, then dK, dV.
// Features are processed in groups of at most 8 tables (128 features); with two
// groups the first launch leaves an fp32 running sum that the second completes.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

// Compact index of query i within level l's future halves, and of key j within its
// past halves. N is a power of two whenever there are levels, so the segment
// length n is one and masks and shifts replace divisions.
__device__ __forceinline__ int compact_future_b(int i, int N, int l) {
  const int n = N >> l;
  return ((i & -n) >> 1) + (i & (n - 1)) - (n >> 1);
}
__device__ __forceinline__ int compact_past(int j, int N, int l) {
  const int n = N >> l;
  return ((j & -n) >> 1) + (j & (n - 1));
}

// Writes the low-rank part of one gradient row held in the accumulator layout
// (lane = token): lr + the fp32 running sum of earlier feature groups (unless
// first), stored as T (last group) or as the fp32 running sum. The sparse partial
// rows are added afterwards (combine_kernel). SINGLE: one feature group, stored
// straight to out (no running-sum load, so nothing here waits for memory; the
// two lanes of a token must be active together).
template <typename T, int D, int NDT = D / 32, bool SINGLE = false>
__device__ __forceinline__ void write_grad_row(const floatx16 (&lr)[NDT], float* scratch, T* out,
                                               size_t row, int h, bool first, bool last,
                                               int dt0 = 0) {
  if constexpr (SINGLE) {
    // One feature group: straight to out, 16 bytes per lane.
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) store_tile_row(out + row + 32 * (dt0 + dt), lr[dt], h);
    return;
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const size_t o = row + 32 * (dt0 + dt) + 8 * g + 4 * h;
      float v[4];
      if (!first) load4(scratch + o, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (first ? 0.0f : v[e]) + lr[dt][4 * g + e];
      if (last) store4(out + o, v);
      else store4(scratch + o, v);
    }
}

// RT[h][d][p] = R[h][p][d] for p < 4 L, zero up to the row stride pw.
__global__ void planes_transpose_kernel(const float* __restrict__ R, int L, int D, int pw,
                                        float* __restrict__ RT) {
  const int h = blockIdx.x;
  for (int i = threadIdx.x; i < D * pw; i += blockDim.x) {
    const int d = i / pw, p = i % pw;
    RT[(size_t)h * D * pw + i] = p < 4 * L ? R[((size_t)h * 4 * L + p) * D + d] : 0.0f;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Row terms.
template <typename T, int D>
__global__ void __launch_bounds__(256)
    bwd_rows_kernel(const T* __restrict__ dO, const float* __restrict__ Os, const T* __restrict__ Olr,
                    const float* __restrict__ lse, const float* __restrict__ dlr,
                    const float* __restrict__ lambda, const float* __restrict__ gs,
                    const float* __restrict__ glr, float eps, int H, int N, float* __restrict__ rc,
                    float* __restrict__ rD, float* __restrict__ rsig, float* __restrict__ re,
                    float* __restrict__ rdd,
                    float* __restrict__ dgs, float* __restrict__ dglr, float* __restrict__ dlam_part) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  __shared__ float red[RPB];
  const int bh = blockIdx.y, head = bh % H;
  const int tid = threadIdx.x, rloc = tid / TPR, part = tid % TPR;
  const int i = blockIdx.x * RPB + rloc;
  const bool valid = i < N;
  float a = 0.0f, b = 0.0f;
  if (valid) {
    const size_t row = ((size_t)bh * N + i) * D + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = to_f(dO[row + e]);
      a += x * Os[row + e];
      b += x * to_f(Olr[row + e]);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
  }
  float dl = 0.0f;
  if (valid && part == 0) {
    const size_t k = (size_t)bh * N + i;
    const float L = lse[k], den = dlr[k], lam = lambda[head];
    const float g1 = gs ? gs[k] : 1.0f, g2 = glr ? glr[k] : 1.0f;
    const float lo = __logf(lam * den + eps);  // -inf when lambda d_lr + eps == 0
    const float mx = fmaxf(L, lo);
    const float lt = mx + __logf(fast_exp(L - mx) + fast_exp(lo - mx));  // log(d_s + lambda d_lr + eps)
    const float m = fast_exp(L - lt);
    const float w2 = fast_exp(L - 2.0f * lt);  // m^2 / d_s
    const float dm = g1 * a;
    rc[k] = g1 * m;
    rD[k] = g1 * a * m * m;
    // sum over the support of dS_ij = c a - D (p_i sums to 1), with 1 - m formed
    // as (lambda d_lr + eps) / (d_s + lambda d_lr + eps)
    rsig[k] = g1 * a * m * fast_exp(lo - lt);
    re[k] = g2 / den;
    rdd[k] = -g2 * b / den - dm * lam * w2;
    dl = -dm * den * w2;
    if (dgs) dgs[k] = m * a;
    if (dglr) dglr[k] = b;
  }
  if (part == 0) red[rloc] = dl;
  __syncthreads();
  if (tid == 0) {
    float s = 0.0f;
    for (int r = 0; r < RPB; ++r) s += red[r];
    dlam_part[(size_t)bh * gridDim.x + blockIdx.x] = s;
  }
}

// dlambda per head: one workgroup per head; thread t sums the entries t, t+256,
// ... in order, then a fixed pairwise tree in LDS (deterministic).
__global__ void __launch_bounds__(256) dlam_reduce_kernel(const float* __restrict__ part, int B,
                                                          int H, int nblk,
                                                          float* __restrict__ dlambda) {
  __shared__ float red[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int total = B * nblk;
  float s = 0.0f;
  for (int i = tid; i < total; i += 256) {
    const int b = i / nblk, k = i % nblk;
    s += part[((size_t)b * H + h) * nblk + k];
  }
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) dlambda[h] = red[0];
}

// ---------------------------------------------------------------------------
// Sparse branch, one workgroup per selected block (s queries x s keys).
// The block's K, V, Q and c dO rows are gathered into LDS row-major (16-byte
// row-contiguous copies, one barrier); then two kinds of waves work without
// further synchronisation, reading every operand from LDS (row fragments, or
// transposed fragments through ds_read_b64_tr_b16):
//   key waves (32 keys each): S = Q K^T and dP = (c dO) V^T put the keys in lanes,
//     so P and dS feed dV^T += (c dO)^T P and dK^T += Q^T dS from registers; dV and
//     dK are accumulated in two passes over the queries to bound register use;
//   query waves (32 queries each): S^T = K Q^T and dP^T = V (c dO)^T put the
//     queries in lanes, so dS^T feeds dQ^T += K^T dS^T.
// ROLE selects key waves (1), query waves (2) or both (3, one launch); with one
// role per launch only the tiles that role reads are staged.
template <typename T, int D, int SB, int ROLE, bool MR = false>
struct SbwdSmem {
  static constexpr int KT = SB < 32 ? 32 : SB;
  static constexpr int LD = tile_ld<T>(D);
  static constexpr bool HK = (ROLE & 2) != 0;  // all keys staged (query waves)
  static constexpr bool HQ = (ROLE & 1) != 0;  // all queries staged (key waves)
  T Ks[HK ? KT : 1][LD];
  T Vs[HK ? KT : 1][LD];
  T Qs[HQ ? KT : 1][LD];
  T Os[HQ ? KT : 1][LD];  // c * dO
  float lse[KT], Dd[KT], cq[KT], sig[KT];
  int kidx[KT], qidx[KT];
  // Several hash rounds: the rows' block indices in the earlier rounds' orders.
  int qbe[MR ? kMaxRounds - 1 : 1][MR ? KT : 1], kbe[MR ? kMaxRounds - 1 : 1][MR ? KT : 1];
};

template <int SB>
constexpr int sbwd_threads(int role) {
  return 64 * (SB < 32 ? 1 : SB / 32) * (role == 3 ? 2 : 1);
}

// Row fragments of one token row read from global memory (x must point to a
// readable row), scaled by sc when SCALED, zero when !valid. Every load is issued
// before any value is used, so that they are in flight together.
template <typename T, int D, bool SCALED = false>
__device__ __forceinline__ void row_frags(const T* x, bool valid, float sc,
                                          typename MF<T>::frag (&f)[D / MF<T>::KSTEP], int h) {
  typedef MF<T> M;
  typename M::frag raw[D / M::KSTEP];
  prefetch_row_frags<T, D>(x, raw, h);
#pragma unroll
  for (int ks = 0; ks < D / M::KSTEP; ++ks) {
    if constexpr (SCALED) {
      const float c = valid ? sc : 0.0f;
      float v[M::KPL];
      if constexpr (M::KPL == 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)raw[ks][e] * c;
      } else {
        v[0] = raw[ks] * c;
      }
      f[ks] = M::from_floats(v);
    } else {
      f[ks] = valid ? raw[ks] : M::zero();
    }
  }
}

template <typename T, int D, int SB, int ROLE, bool MR>
__global__ void __launch_bounds__(sbwd_threads<SB>(ROLE))
    sparse_bwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                      const T* __restrict__ dO, const float* __restrict__ lse,
                      const float* __restrict__ rc, const float* __restrict__ rD,
                      const float* __restrict__ rsig, const int32_t* __restrict__ qperm,
                      const int32_t* __restrict__ kperm, int N, int causal, int levels,
                      int rounds, const int32_t* __restrict__ qbid,
                      const int32_t* __restrict__ kbid, float scale, T* __restrict__ dQp,
                      T* __restrict__ dKp, T* __restrict__ dVp) {
  typedef MF<T> M;
  typedef SbwdSmem<T, D, SB, ROLE, MR> Sm;
  constexpr int KT = Sm::KT, NW = KT / 32, LD = Sm::LD;
  constexpr int NT = sbwd_threads<SB>(ROLE);
  __shared__ Sm sm;
  const int bh = blockIdx.y, item = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = wave_id();  // wave index, uniform (scalar) so that role branches stay uniform
  const size_t P = perm_stride(N, levels, causal, rounds);
  const size_t slots = partial_slots(N, levels, causal, rounds);
  const size_t rowbase = (size_t)bh * N;

  // Orders (round, level): causal rounds x levels, order-major items then the
  // leaves; otherwise one order per round.
  const int nord = causal ? rounds * levels : rounds;
  const int per_level = causal ? (N / 2) / SB : 0;
  const int nlev_items = causal ? nord * per_level : 0;
  const int32_t* qsrc = nullptr;
  const int32_t* ksrc = nullptr;
  int ord = -1, lev = 0, rnd = 0, tok0 = 0;
  bool leaf = false;
  if (causal && item < nlev_items) {
    ord = item / per_level;
    lev = ord % levels;
    rnd = ord / levels;
    const int b = item % per_level;
    qsrc = qperm + (size_t)bh * P + (size_t)ord * (N / 2) + (size_t)b * SB;
    ksrc = kperm + (size_t)bh * P + (size_t)ord * (N / 2) + (size_t)b * SB;
  } else if (causal) {
    leaf = true;
    tok0 = (item - nlev_items) * SB;
  } else {
    ord = rnd = item / (N / SB);
    qsrc = qperm + (size_t)bh * P + (size_t)item * SB;
    ksrc = kperm + (size_t)bh * P + (size_t)item * SB;
  }
  // The query's own block (its causal leaf, or its first round's block) adds
  // sigma_i Q_i to its dQ part.
  const bool own = causal ? leaf : rnd == 0;
  for (int t = tid; t < KT; t += NT) {
    const int kj = t < SB ? (leaf ? tok0 + t : ksrc[t]) : -1;
    const int qi = t < SB ? (leaf ? tok0 + t : qsrc[t]) : -1;
    sm.kidx[t] = kj;
    sm.qidx[t] = qi;
    sm.lse[t] = qi >= 0 ? lse[rowbase + qi] : 0.0f;
    sm.Dd[t] = qi >= 0 ? rD[rowbase + qi] : 0.0f;
    sm.cq[t] = qi >= 0 ? rc[rowbase + qi] : 0.0f;
    sm.sig[t] = qi >= 0 ? rsig[rowbase + qi] : 0.0f;
    if constexpr (MR) {
      for (int r = 0; r < rnd; ++r) {
        const size_t base = ((size_t)bh * nord + (causal ? r * levels + lev : r)) * N;
        sm.qbe[r][t] = qi >= 0 ? qbid[base + qi] : -1;
        sm.kbe[r][t] = kj >= 0 ? kbid[base + kj] : -2;
      }
    }
  }
  __syncthreads();
  // A pair that shares a block in an earlier round is held there (several rounds).
  auto dup = [&](int qr, int kr) __attribute__((always_inline)) {
    bool d = false;
    if constexpr (MR) {
      for (int r = 0; r < rnd; ++r) d = d || sm.qbe[r][qr] == sm.kbe[r][kr];
    }
    return d;
  };
  if constexpr (Sm::HK) {
    T* const dst[2] = {&sm.Ks[0][0], &sm.Vs[0][0]};
    const T* const src[2] = {K, V};
    const float* const sc[2] = {nullptr, nullptr};
    gather_rows<T, D, KT, NT, 2>(dst, LD, src, sc, sm.kidx, rowbase, tid);
  }
  if constexpr (Sm::HQ) {
    T* const dst[2] = {&sm.Qs[0][0], &sm.Os[0][0]};
    const T* const src[2] = {Q, dO};
    const float* const sc[2] = {nullptr, sm.cq};
    gather_rows<T, D, KT, NT, 2>(dst, LD, src, sc, sm.qidx, rowbase, tid);
  }
  __syncthreads();

  const bool key_wave = (ROLE & 1) && w < NW;
  if (key_wave) {
    if constexpr (Sm::HQ) {
      const int key = 32 * w + col;
      const int jk = sm.kidx[key];
      const bool kvalid = jk >= 0;
      typename M::frag kf[D / M::KSTEP], vf[D / M::KSTEP];
      if constexpr (Sm::HK) {
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks) kf[ks] = row_frag<T>(&sm.Ks[0][0], LD, 32 * w, 0, ks, lane);
      } else {
        row_frags<T, D>(K + (rowbase + (kvalid ? jk : 0)) * D, kvalid, 1.0f, kf, h);
      }
      const int qt0 = leaf ? w : 0;
      const size_t ksl = !causal ? (size_t)rnd * N + jk
                         : leaf  ? (size_t)jk
                                 : (size_t)N + (size_t)ord * (N / 2) + compact_past(jk, N, lev);
      // Pass 0: dV^T = (c dO)^T P.   Pass 1: dK^T = Q^T dS.
#pragma unroll 1
      for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
          if constexpr (Sm::HK) {
#pragma unroll
            for (int ks = 0; ks < D / M::KSTEP; ++ks) vf[ks] = row_frag<T>(&sm.Vs[0][0], LD, 32 * w, 0, ks, lane);
          } else {
            row_frags<T, D>(V + (rowbase + (kvalid ? jk : 0)) * D, kvalid, 1.0f, vf, h);
          }
        }
        floatx16 acc[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
        for (int qt = qt0; qt < KT / 32; ++qt) {
          floatx16 s = zero16();
          // Fragments read four k-steps at a time so that their LDS reads overlap.
          constexpr int KB = D / M::KSTEP < 4 ? D / M::KSTEP : 4;
#pragma unroll
          for (int k4 = 0; k4 < D / M::KSTEP; k4 += KB) {
            typename M::frag qa[KB];
#pragma unroll
            for (int j = 0; j < KB; ++j) qa[j] = row_frag<T>(&sm.Qs[0][0], LD, 32 * qt, 0, k4 + j, lane);
#pragma unroll
            for (int j = 0; j < KB; ++j) s = M::mma(qa[j], kf[k4 + j], s);
          }
          floatx16 dp = zero16();
          if (pass == 1) {
#pragma unroll
            for (int k4 = 0; k4 < D / M::KSTEP; k4 += KB) {
              typename M::frag oa[KB];
#pragma unroll
              for (int j = 0; j < KB; ++j) oa[j] = row_frag<T>(&sm.Os[0][0], LD, 32 * qt, 0, k4 + j, lane);
#pragma unroll
              for (int j = 0; j < KB; ++j) dp = M::mma(oa[j], vf[k4 + j], dp);
            }
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qr = 32 * qt + acc_row(v, h);
            // Masked pairs get exp(-inf) = 0 (no branch around the exponential);
            // every row of a block of 32 or more is valid.
            const bool ok = kvalid & (SB >= 32 || sm.qidx[qr] >= 0) & !(leaf & (key > qr)) &
                            !dup(qr, key);
            const float p = fast_exp(ok ? s[v] * scale - sm.lse[qr] : -INFINITY);
            s[v] = pass == 0 ? p : p * (dp[v] - sm.Dd[qr]);
          }
          const T* X = pass == 0 ? &sm.Os[0][0] : &sm.Qs[0][0];
#pragma unroll
          for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
            const typename M::frag pf = M::from_acc(s, ks2);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
              acc[dt] = M::mma(tr_frag<T>(X, LD, 32 * qt, 32 * dt, ks2, lane, true), pf, acc[dt]);
          }
        }
        if (kvalid) {  // (the same for the two lanes of a key)
          T* dst = (pass == 0 ? dVp : dKp) + ((size_t)bh * slots + ksl) * D;
          const float f = pass == 0 ? 1.0f : scale;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            float x[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) x[v] = acc[dt][v] * f;
            store_tile_row(dst + 32 * dt, x, h);
          }
        }
      }
    }
  } else {
    if constexpr (Sm::HK) {
      const int qw = (ROLE & 1) ? w - NW : w;
      const int query = 32 * qw + col;
      const int iq = sm.qidx[query];
      const bool qvalid = iq >= 0;
      typename M::frag qf[D / M::KSTEP], of[D / M::KSTEP];
      if constexpr (Sm::HQ) {
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks) {
          qf[ks] = row_frag<T>(&sm.Qs[0][0], LD, 32 * qw, 0, ks, lane);
          of[ks] = row_frag<T>(&sm.Os[0][0], LD, 32 * qw, 0, ks, lane);
        }
      } else {
        row_frags<T, D>(Q + (rowbase + (qvalid ? iq : 0)) * D, qvalid, 1.0f, qf, h);
        row_frags<T, D, true>(dO + (rowbase + (qvalid ? iq : 0)) * D, qvalid, sm.cq[query], of, h);
      }
      const float lq = sm.lse[query], dq = sm.Dd[query];
      floatx16 acc[D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
      // The query's row in the accumulator layout (for the shift below), in
      // flight during the products.
      DRow<T, D / 32> qrow;
      qrow.load(Q + (rowbase + (qvalid ? iq : 0)) * D, h);
      float sig = 0.0f;  // sum over the block's keys of dS (as rounded for the product)
      const int nkt = leaf ? qw + 1 : KT / 32;
      for (int kt = 0; kt < nkt; ++kt) {
        floatx16 s = zero16(), dp = zero16();
        constexpr int KB = D / M::KSTEP < 4 ? D / M::KSTEP : 4;
#pragma unroll
        for (int k4 = 0; k4 < D / M::KSTEP; k4 += KB) {
          typename M::frag ka[KB], va[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            ka[j] = row_frag<T>(&sm.Ks[0][0], LD, 32 * kt, 0, k4 + j, lane);
            va[j] = row_frag<T>(&sm.Vs[0][0], LD, 32 * kt, 0, k4 + j, lane);
          }
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            s = M::mma(ka[j], qf[k4 + j], s);
            dp = M::mma(va[j], of[k4 + j], dp);
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kr = 32 * kt + acc_row(v, h);
          const bool ok = qvalid & (SB >= 32 || sm.kidx[kr] >= 0) & !(leaf & (kr > query)) &
                          !dup(query, kr);
          const float p = fast_exp(ok ? s[v] * scale - lq : -INFINITY);
          s[v] = p * (dp[v] - dq);
        }
#pragma unroll
        for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
          const typename M::frag sf = M::from_acc(s, ks2);
          sig = frag_sum<T>(sf, sig);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            acc[dt] = M::mma(tr_frag<T>(&sm.Ks[0][0], LD, 32 * kt, 32 * dt, ks2, lane, true), sf, acc[dt]);
        }
      }
      // (the query's own block, its leaf or its only block, adds the support-wide
      // sum back)
      sig = sum_halves(sig) - (own ? sm.sig[query] : 0.0f);
      float qv[D / 32][4][4];
      qrow.unpack(qv);
      if (qvalid) {
        const size_t sl = !causal ? (size_t)rnd * N + iq
                          : leaf  ? (size_t)iq
                                  : (size_t)N + (size_t)ord * (N / 2) + compact_future_b(iq, N, lev);
        T* dst = dQp + ((size_t)bh * slots + sl) * D;  // (qvalid: the same for a query's two lanes)
        // The block's dQ part relative to the query: sum_j dS_ij (K_j - Q_i).
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          float x[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) x[v] = (acc[dt][v] - sig * qv[dt][v >> 2][v & 3]) * scale;
          store_tile_row(dst + 32 * dt, x, h);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sparse branch, single pass (bf16, blocks of at most 128 tokens). Persistent
// workgroups take the selected blocks g, g + G, g + 2G, ... (G = grid size; the
// blocks of one head are adjacent in g, so concurrent workgroups share a head's
// rows in the last-level cache). While block g computes, the next block's Q, dO
// and K rows (and each key wave's V rows) are loaded into registers, and the block
// after that's row indices.
//
// Key wave w owns keys 32 w .. 32 w + 31 (K from LDS, V in registers) and walks
// the query tiles: S = Q K^T and dP_raw = dO V^T with the keys in lanes, then
// P = exp(scale S - lse), dS = P (c dP_raw - D) (c = g_s m per query row),
// dV^T += dO^T (c P) and dK^T += Q^T dS from registers, and dS^T goes to LDS.
// After a barrier, wave w forms dQ^T = K^T dS^T for query tile w.
template <int D, int SB, bool MR = false>
struct Sb2Smem {
  static constexpr int KT = SB < 32 ? 32 : SB;
  static constexpr int LD = tile_ld<__bf16>(D), LDK = tile_ld<__bf16>(KT);
  // The per-row arrays come first: their addresses are then small constants
  // from one per-thread base (instruction offsets), not separate registers.
  alignas(16) float lse[KT];  // lse log2 e; +inf for rows past the block (P = 0)
  alignas(16) float Dd[KT];
  alignas(16) float cq[KT];
  float sig[KT];              // sum over the query's whole support of dS_ij
  int qidx[KT], kidx[KT];    // token of each row of this block, -1 past the block
  int qnext[KT], knext[KT];  // the same for the next block
  alignas(16) __bf16 Qs[KT][LD];
  __bf16 Os[KT][LD];    // dO (the row factor c is applied in registers)
  __bf16 Ks[KT][LD];
  __bf16 dST[KT][LDK];  // dS^T, [key][query]
  // Several hash rounds: the rows' block indices in the earlier rounds' orders.
  alignas(16) int qbe[MR ? kMaxRounds - 1 : 1][MR ? KT : 1];
  int kbe[MR ? kMaxRounds - 1 : 1][MR ? KT : 1];
};

template <int D, int SB, bool MR>
__global__ void __launch_bounds__(64 * (SB < 32 ? 1 : SB / 32), D <= 64 ? 2 : 1)
    sparse_bwd2_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                       const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                       const float* __restrict__ lse, const float* __restrict__ rc,
                       const float* __restrict__ rD, const float* __restrict__ rsig,
                       const int32_t* __restrict__ qperm,
                       const int32_t* __restrict__ kperm, int N, int causal, int levels,
                       int rounds, const int32_t* __restrict__ qbid,
                       const int32_t* __restrict__ kbid, float scale, int items, int total,
                       __bf16* __restrict__ dQp, __bf16* __restrict__ dKp,
                       __bf16* __restrict__ dVp) {
  typedef __bf16 T;
  typedef MF<T> M;
  typedef Sb2Smem<D, SB, MR> Sm;
  constexpr int KT = Sm::KT, NW = KT / 32, NT = 64 * NW, LD = Sm::LD, LDK = Sm::LDK;
  constexpr int CH = D / 8, GIT = KT * CH / NT, KS = D / M::KSTEP;
  __shared__ Sm sm;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = wave_id();  // wave index, uniform (scalar) so that role branches stay uniform
  const int G = gridDim.x;
  const size_t P = perm_stride(N, levels, causal, rounds);
  const size_t slots = partial_slots(N, levels, causal, rounds);
  // Orders (round, level): causal rounds x levels, order-major items then the
  // leaves; otherwise one order per round.
  const int nord = causal ? rounds * levels : rounds;
  const int per_level = causal ? (N / 2) / SB : 0;
  const int nlev = causal ? nord * per_level : 0;

  // Block g (in the XCD-aware order): head, order (-1 for a causal leaf), rows.
  // G is a multiple of 8, so a workgroup's blocks are all of its own XCD's share.
  auto head_of = [&](int g) __attribute__((always_inline)) {
    int it;
    return xcd_item(g, items, per_level, nord, it);
  };
  // Rows of block g: row t's query and key tokens are (a, b) when alt < -1, else
  // both are alt (a causal leaf: the token itself; -1 past the block). The order
  // entries are read on every path (a leaf or a row past the block reads the
  // head's first entry and discards it), so that the prefetches are issued in the
  // same number on every path and the waits for them are exact; the choice is
  // made only where the rows are used, so that nothing waits for the loads early.
  struct Rows {
    int a, b, alt;
  };
  auto rows_of = [&](int g, int t) __attribute__((always_inline)) {
    int it;
    const int bh = xcd_item(g, items, per_level, nord, it);
    const bool lf = causal && it >= nlev, past = t >= SB;
    const size_t off = (size_t)bh * P + (lf || past ? (size_t)0
                                         : causal ? (size_t)(it / per_level) * (N / 2) +
                                                        (size_t)(it % per_level) * SB + t
                                                  : (size_t)it * SB + t);
    return Rows{qperm[off], kperm[off], past ? -1 : lf ? (it - nlev) * SB + t : -2};
  };

  // Registers holding the next block.
  Vec8<T> pq[GIT], po[GIT], pk[GIT];
  typename M::frag pv[KS];
  float plse = 0.0f, pD = 0.0f, pc = 0.0f, psig = 0.0f;
  bool pvalid = false;
  int pqb[kMaxRounds - 1], pkb[kMaxRounds - 1];  // (several rounds) block indices
  Rows prow{-1, -1, -1};
  auto gather = [&](int gn) __attribute__((always_inline)) {
    int itn;
    const int bhn = xcd_item(gn, items, per_level, nord, itn);
    const size_t rb = (size_t)bhn * N;
#pragma unroll
    for (int i = 0; i < GIT; ++i) {
      const int piece = tid + NT * i, r = piece / CH, c8 = (piece % CH) * 8;
      const int qi = sm.qnext[r], kj = sm.knext[r];
      // Rows past the block (s < 32 only) read row 0: their lse (+inf) and key
      // masks make them contribute nothing.
      pq[i].load(Q + (rb + max(qi, 0)) * D + c8);
      po[i].load(dO + (rb + max(qi, 0)) * D + c8);
      pk[i].load(K + (rb + max(kj, 0)) * D + c8);
    }
    {  // row terms of query row tid % KT (used by threads tid < KT)
      const int qi = sm.qnext[tid % KT];
      const size_t k = rb + max(qi, 0);
      pvalid = qi >= 0;
      plse = lse[k];
      pD = rD[k];
      pc = rc[k];
      psig = rsig[k];
    }
    if constexpr (MR) {
      // The row's block indices in the earlier rounds' orders of the next block's
      // level (used by threads tid < KT).
      const bool lfn = causal && itn >= nlev;
      const int ordn = lfn ? -1 : causal ? itn / per_level : itn / (N / SB);
      const int levn = causal && ordn >= 0 ? ordn % levels : 0;
      const int rndn = ordn < 0 ? 0 : causal ? ordn / levels : ordn;
      const int qi = sm.qnext[tid % KT], kj = sm.knext[tid % KT];
#pragma unroll
      for (int r = 0; r < kMaxRounds - 1; ++r) {
        pqb[r] = -1;
        pkb[r] = -2;
        if (r < rndn) {
          const size_t base = ((size_t)bhn * nord + (causal ? r * levels + levn : r)) * N;
          if (qi >= 0) pqb[r] = qbid[base + qi];
          if (kj >= 0) pkb[r] = kbid[base + kj];
        }
      }
    }
  };

  // V rows of the next block's keys of this wave, as MFMA operands (issued once
  // the current block no longer needs the registers).
  auto gather_v = [&](size_t rb) __attribute__((always_inline)) {
    const int kv = sm.knext[32 * w + col];
    prefetch_row_frags<T, D>(V + (rb + max(kv, 0)) * D, pv, h);
  };

  int g = blockIdx.x;
  if (g >= total) return;
  if (tid < KT) {
    const Rows r0 = rows_of(g, tid);
    sm.qnext[tid] = r0.alt < -1 ? r0.a : r0.alt;
    sm.knext[tid] = r0.alt < -1 ? r0.b : r0.alt;
  }
  __syncthreads();
  gather(g);
  // Past the last block, the prefetches repeat the last block (never used).
  prow = rows_of(min(g + G, total - 1), tid);
  gather_v((size_t)head_of(g) * N);

  for (; g < total; g += G) {
    __syncthreads();  // the previous block is done with LDS
    // Stage block g from registers.
#pragma unroll
    for (int i = 0; i < GIT; ++i) {
      const int piece = tid + NT * i, r = piece / CH, c8 = (piece % CH) * 8;
      pq[i].store(&sm.Qs[r][c8]);
      po[i].store(&sm.Os[r][c8]);
      pk[i].store(&sm.Ks[r][c8]);
    }
    if (tid < KT) {
      sm.qidx[tid] = sm.qnext[tid];
      sm.kidx[tid] = sm.knext[tid];
      sm.qnext[tid] = prow.alt < -1 ? prow.a : prow.alt;
      sm.knext[tid] = prow.alt < -1 ? prow.b : prow.alt;
      sm.lse[tid] = pvalid ? plse * kLog2e : INFINITY;  // (base 2)
      sm.Dd[tid] = pvalid ? pD : 0.0f;
      sm.cq[tid] = pvalid ? pc : 0.0f;
      sm.sig[tid] = pvalid ? psig : 0.0f;
      if constexpr (MR) {
#pragma unroll
        for (int r = 0; r < kMaxRounds - 1; ++r) {
          sm.qbe[r][tid] = pqb[r];
          sm.kbe[r][tid] = pkb[r];
        }
      }
    }

    int it;
    const int bh = xcd_item(g, items, per_level, nord, it);
    const bool leaf = causal && it >= nlev;
    // The block's order (-1: a leaf), its level (the segment geometry) and round.
    const int ord = leaf ? -1 : causal ? it / per_level : it / (N / SB);
    const int lev = causal && ord >= 0 ? ord % levels : 0;
    const int rnd = ord < 0 ? 0 : causal ? ord / levels : ord;
    // The query's own block (its causal leaf, or its first round's block) adds
    // sigma_i Q_i to its dQ part.
    const bool own = causal ? leaf : rnd == 0;
    // (several rounds: the rows' block indices in the earlier rounds' orders of the
    // same level, staged above from the prefetch; a pair that shares a block there
    // is held there, not here)
    __syncthreads();
    // Phase 1: key wave w.
    const int key = 32 * w + col;
    floatx16 dv[D / 32], dk[D / 32];
    {
      const int jk = sm.kidx[key];
      const bool kvalid = jk >= 0;
      // Several rounds: bit v of dup[qt] marks the pair (row v of query tile qt,
      // this lane's key) as one an earlier round holds; formed for all tiles at
      // once so that the LDS reads are in flight together, not in the softmax.
      uint32_t dup[NW];
#pragma unroll
      for (int qt = 0; qt < NW; ++qt) dup[qt] = 0u;
      if constexpr (MR) {
        if (rnd > 0) {
#pragma unroll
          for (int r = 0; r < kMaxRounds - 1; ++r)
            if (r < rnd) {
              const int kb = sm.kbe[r][key % KT];
#pragma unroll
              for (int qt = 0; qt < NW; ++qt)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                  const int4 q4 =
                      *reinterpret_cast<const int4*>(&sm.qbe[r][32 * qt + 8 * gg + 4 * h]);
                  const int qe[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    if (qe[e] == kb) dup[qt] |= 1u << (4 * gg + e);
                }
            }
        }
      }
      const float c2 = scale * kLog2e;  // P = 2^(c2 S - lse log2 e)
      typename M::frag kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = row_frag<T>(&sm.Ks[0][0], LD, 32 * w, 0, ks, lane);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) dv[dt] = dk[dt] = zero16();
      auto qtile = [&](int qt, uint32_t dq) __attribute__((always_inline)) {
        floatx16 s = zero16(), dp = zero16();
        // Fragments read KB k-steps at a time so that their LDS reads overlap.
        constexpr int KB = KS < 4 ? KS : 4;
#pragma unroll
        for (int k4 = 0; k4 < KS; k4 += KB) {
          typename M::frag qa[KB], oa[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            qa[j] = row_frag<T>(&sm.Qs[0][0], LD, 32 * qt, 0, k4 + j, lane);
            oa[j] = row_frag<T>(&sm.Os[0][0], LD, 32 * qt, 0, k4 + j, lane);
          }
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            s = M::mma(qa[j], kf[k4 + j], s);
            dp = M::mma(oa[j], pv[k4 + j], dp);
          }
        }
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int r0 = 32 * qt + 8 * gg + 4 * h;
          const floatx4 L4 = *reinterpret_cast<const floatx4*>(&sm.lse[r0]);
          const floatx4 D4 = *reinterpret_cast<const floatx4*>(&sm.Dd[r0]);
          const floatx4 C4 = *reinterpret_cast<const floatx4*>(&sm.cq[r0]);
          float dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * gg + e;
            // Masked pairs get exp(-inf) = 0 (no branch around the exponential).
            bool ok = kvalid & !(leaf & (key > r0 + e));
            if constexpr (MR) ok = ok && !((dq >> v) & 1u);
            const float p = __builtin_amdgcn_exp2f(ok ? fmaf(s[v], c2, -L4[e]) : -INFINITY);
            dsv[e] = p * (C4[e] * dp[v] - D4[e]);
            s[v] = C4[e] * p;
            dp[v] = dsv[e];
          }
          store4(&sm.dST[key][r0], dsv);
        }
#pragma unroll
        for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
          const typename M::frag pf = M::from_acc(s, ks2);
          const typename M::frag sf = M::from_acc(dp, ks2);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            dv[dt] = M::mma(tr_frag<T>(&sm.Os[0][0], LD, 32 * qt, 32 * dt, ks2, lane, true), pf, dv[dt]);
            dk[dt] = M::mma(tr_frag<T>(&sm.Qs[0][0], LD, 32 * qt, 32 * dt, ks2, lane, true), sf, dk[dt]);
          }
        }
      };
      // Leaf blocks: query tiles from the diagonal on; otherwise all of them, the
      // loop unrolled so that one tile's products overlap the next tile's reads.
      if (leaf) {
        for (int qt = w; qt < NW; ++qt) qtile(qt, 0u);  // (a leaf is in every round)
      } else {
#pragma unroll
        for (int qt = 0; qt < NW; ++qt) qtile(qt, dup[qt]);
      }
    }
    // Loads for the next block (rows, issued now that phase 1 no longer needs the
    // registers; phase 2 and the stores cover their latency) and the one after
    // (indices).
    const int gn = min(g + G, total - 1);
    const size_t nrb = (size_t)head_of(gn) * N;
    gather(gn);
    prow = rows_of(min(g + 2 * G, total - 1), tid);
    gather_v(nrb);
    // The rows of phase 2's query tile (for the dQ parts relative to the query),
    // read before the barrier after which Qs holds dV.
    DRow<T, D / 32> qrow;
    qrow.load(&sm.Qs[key][0], h);
    __syncthreads();  // dS^T complete; Qs and Os no longer read
    // dV and dK tiles to LDS (rows = keys of the block) for row-contiguous stores.
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        float xv[4], xk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[e] = dv[dt][4 * gg + e];
          xk[e] = dk[dt][4 * gg + e] * scale;
        }
        const int c = 32 * dt + 8 * gg + 4 * h;
        store4(&sm.Qs[key][c], xv);
        store4(&sm.Os[key][c], xk);
      }
    // Phase 2: dQ^T = K^T dS^T for query tile w (leaf blocks: keys up to the tile),
    // with sig = the sum of the tile's dS^T over the keys as rounded for the
    // product.
    floatx16 dq[D / 32];
    float sig = 0.0f;
    {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) dq[dt] = zero16();
      // Leaf blocks: keys up to the tile (an even number of k-steps: 32 keys each
      // two); the k-steps go two at a time so that their LDS reads overlap.
      const int nks = leaf ? 2 * (w + 1) : KT / M::KSTEP;
      for (int ks = 0; ks < nks; ks += 2) {
        typename M::frag bq[2], ka[2][D / 32];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bq[j] = tr_frag<T>(&sm.dST[0][0], LDK, 0, 32 * w, ks + j, lane, false);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            ka[j][dt] = tr_frag<T>(&sm.Ks[0][0], LD, 0, 32 * dt, ks + j, lane, false);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          sig = frag_sum<T>(bq[j], sig);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) dq[dt] = M::mma(ka[j][dt], bq[j], dq[dt]);
        }
      }
    }
    // (the query's own block, its leaf or its only block, adds the support-wide
    // sum back)
    sig = sum_halves(sig) - (own ? sm.sig[key] : 0.0f);
    float qv[D / 32][4][4];
    qrow.unpack(qv);
    __syncthreads();  // Ks no longer read; dV, dK tiles complete
    // dQ tile to LDS (rows = queries of the block), relative to the query; the
    // three gradient tiles then go out to their slots with row-contiguous 16-byte
    // stores.
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        float xq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xq[e] = (dq[dt][4 * gg + e] - sig * qv[dt][gg][e]) * scale;
        store4(&sm.Ks[key][32 * dt + 8 * gg + 4 * h], xq);
      }
    __syncthreads();
    {
      const size_t hb = (size_t)bh * slots;
      // Two row pieces at a time: their six LDS reads are issued before any of
      // their stores, so that one wait covers them.
      constexpr int PB = GIT % 2 == 0 ? 2 : 1;
#pragma unroll
      for (int i0 = 0; i0 < GIT; i0 += PB) {
        Vec8<T> a[PB], b2[PB], c[PB];
        int jk[PB], iq[PB], rr[PB], c8[PB];
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const int piece = tid + NT * (i0 + j);
          rr[j] = piece / CH;
          c8[j] = (piece % CH) * 8;
          jk[j] = sm.kidx[rr[j]];
          iq[j] = sm.qidx[rr[j]];
          a[j].load(&sm.Qs[rr[j]][c8[j]]);
          b2[j].load(&sm.Os[rr[j]][c8[j]]);
          c[j].load(&sm.Ks[rr[j]][c8[j]]);
        }
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          // Every row of a block of 32 or more is valid: the stores are then
          // issued on every path, which keeps the waits for the prefetches exact.
          if (SB >= 32 || jk[j] >= 0) {
            const size_t sl = !causal ? (size_t)rnd * N + jk[j]
                              : leaf  ? (size_t)jk[j]
                                      : (size_t)N + (size_t)ord * (N / 2) + compact_past(jk[j], N, lev);
            a[j].store_nt(dVp + (hb + sl) * D + c8[j]);
            b2[j].store_nt(dKp + (hb + sl) * D + c8[j]);
          }
          if (SB >= 32 || iq[j] >= 0) {
            const size_t sl = !causal ? (size_t)rnd * N + iq[j]
                              : leaf  ? (size_t)iq[j]
                                      : (size_t)N + (size_t)ord * (N / 2) +
                                            compact_future_b(iq[j], N, lev);
            c[j].store_nt(dQp + (hb + sl) * D + c8[j]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sparse backward with 16-key tiles: the same blocks, LDS tiles and slot stores
// as sparse_bwd2_kernel (bf16, s = 128, one hash round), computed by 8 waves on
// the 16x16x32 bf16 MFMA. Wave w takes keys 16w .. 16w + 15 in the key phase and
// queries 16w .. 16w + 15 in the dQ phase, so that its dV, dK accumulators (16
// keys x D channels each) and operands fit two waves per SIMD.
//
// 16x16x32 operand layout (lane = 16 g + s): A[m][k] is held by lane (m = s) at
// k = 8 g + e; B[k][n] by lane (n = s) at k = 8 g + e; D[m][n] by lane (n = s) at
// m = 4 g + e, e < 4.
__device__ __forceinline__ floatx4 mma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Operand whose lanes run over 16 columns (n0 + s) of a row-major LDS matrix X and
// whose K elements are X's rows kb1 .. kb1 + 3 (e < 4) and kb2 .. kb2 + 3 (e >= 4),
// read with two ds_read_b64_tr_b16 (each 16-lane group may pass its own rows).
__device__ __forceinline__ bf16x8 tr16(const __bf16* X, int ld, int kb1, int kb2, int n0, int lane) {
  const int s = lane & 15;
  typedef __attribute__((address_space(3))) bf16x4_tr* lds_ptr;
  const int nb = n0 + 4 * (s & 3);
  const bf16x4_tr a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_ptr)(X + (size_t)(kb1 + (s >> 2)) * ld + nb));
  const bf16x4_tr b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_ptr)(X + (size_t)(kb2 + (s >> 2)) * ld + nb));
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[e] = a[e]; f[4 + e] = b[e]; }
  return f;
}
__device__ __forceinline__ floatx4 zero4() {
  floatx4 z;
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = 0.0f;
  return z;
}

template <int D>
__global__ void __launch_bounds__(512)
    sparse_bwd3_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                       const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                       const float* __restrict__ lse, const float* __restrict__ rc,
                       const float* __restrict__ rD, const float* __restrict__ rsig,
                       const int32_t* __restrict__ qperm, const int32_t* __restrict__ kperm,
                       int N, int causal, int levels, float scale, int items, int total,
                       __bf16* __restrict__ dQp, __bf16* __restrict__ dKp,
                       __bf16* __restrict__ dVp) {
  typedef __bf16 T;
  constexpr int SB = 128;
  typedef Sb2Smem<D, SB, false> Sm;
  constexpr int KT = SB, NT = 512, LD = Sm::LD, LDK = Sm::LDK;
  constexpr int CH = D / 8, GIT = KT * CH / NT, KS = D / 32, CT = D / 16;
  __shared__ Sm sm;
  const int tid = threadIdx.x, lane = tid & 63, s = lane & 15, g4 = lane >> 4;
  const int w = wave_id();
  const int G = gridDim.x;
  const size_t P = perm_stride(N, levels, causal);
  const size_t slots = partial_slots(N, levels, causal);
  const int nord = causal ? levels : 1;
  const int per_level = causal ? (N / 2) / SB : 0;
  const int nlev = causal ? nord * per_level : 0;

  auto head_of = [&](int gg) __attribute__((always_inline)) {
    int it;
    return xcd_item(gg, items, per_level, nord, it);
  };
  // Rows of block gg (as in sparse_bwd2_kernel): query and key tokens (a, b) when
  // alt < -1, else both are alt (a causal leaf's token); threads t >= SB read the
  // head's first entry and discard it.
  struct Rows {
    int a, b, alt;
  };
  auto rows_of = [&](int gg, int t) __attribute__((always_inline)) {
    int it;
    const int bh = xcd_item(gg, items, per_level, nord, it);
    const bool lf = causal && it >= nlev, past = t >= SB;
    const size_t off = (size_t)bh * P + (lf || past ? (size_t)0
                                         : causal ? (size_t)(it / per_level) * (N / 2) +
                                                        (size_t)(it % per_level) * SB + t
                                                  : (size_t)it * SB + t);
    return Rows{qperm[off], kperm[off], past ? -1 : lf ? (it - nlev) * SB + t : -2};
  };

  Vec8<T> pq[GIT], po[GIT], pk[GIT];
  bf16x8 pv[KS];
  float plse = 0.0f, pD = 0.0f, pc = 0.0f, psig = 0.0f;
  bool pvalid = false;
  Rows prow{-1, -1, -1};
  auto gather = [&](int gn) __attribute__((always_inline)) {
    const size_t rb = (size_t)head_of(gn) * N;
#pragma unroll
    for (int i = 0; i < GIT; ++i) {
      const int piece = tid + NT * i, r = piece / CH, c8 = (piece % CH) * 8;
      const int qi = sm.qnext[r], kj = sm.knext[r];
      pq[i].load(Q + (rb + qi) * D + c8);
      po[i].load(dO + (rb + qi) * D + c8);
      pk[i].load(K + (rb + kj) * D + c8);
    }
    const int qi = sm.qnext[tid % KT];
    const size_t k = rb + qi;
    pvalid = qi >= 0;
    plse = lse[k];
    pD = rD[k];
    pc = rc[k];
    psig = rsig[k];
  };
  // V rows of this wave's 16 keys of the next block, as B operands (lane (key s,
  // group g) holds channels 32 ks + 8 g .. + 7).
  auto gather_v = [&](size_t rb) __attribute__((always_inline)) {
    const int kv = sm.knext[16 * w + s];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      pv[ks] = *reinterpret_cast<const bf16x8*>(V + (rb + kv) * D + 32 * ks + 8 * g4);
  };

  int g = blockIdx.x;
  if (g >= total) return;
  if (tid < KT) {
    const Rows r0 = rows_of(g, tid);
    sm.qnext[tid] = r0.alt < -1 ? r0.a : r0.alt;
    sm.knext[tid] = r0.alt < -1 ? r0.b : r0.alt;
  }
  __syncthreads();
  gather(g);
  prow = rows_of(min(g + G, total - 1), tid);
  gather_v((size_t)head_of(g) * N);

  for (; g < total; g += G) {
    __syncthreads();  // the previous block is done with LDS
#pragma unroll
    for (int i = 0; i < GIT; ++i) {
      const int piece = tid + NT * i, r = piece / CH, c8 = (piece % CH) * 8;
      pq[i].store(&sm.Qs[r][c8]);
      po[i].store(&sm.Os[r][c8]);
      pk[i].store(&sm.Ks[r][c8]);
    }
    if (tid < KT) {
      sm.qidx[tid] = sm.qnext[tid];
      sm.kidx[tid] = sm.knext[tid];
      sm.qnext[tid] = prow.alt < -1 ? prow.a : prow.alt;
      sm.knext[tid] = prow.alt < -1 ? prow.b : prow.alt;
      sm.lse[tid] = pvalid ? plse * kLog2e : INFINITY;
      sm.Dd[tid] = pvalid ? pD : 0.0f;
      sm.cq[tid] = pvalid ? pc : 0.0f;
      sm.sig[tid] = pvalid ? psig : 0.0f;
    }
    int it;
    const int bh = xcd_item(g, items, per_level, nord, it);
    const bool leaf = causal && it >= nlev;
    const int ord = leaf ? -1 : causal ? it / per_level : 0;
    const int lev = causal && ord >= 0 ? ord : 0;
    const bool own = causal ? leaf : true;
    __syncthreads();

    // Key phase: wave w, keys 16 w + s. S (queries x keys) and dP tiles of 16
    // queries; dV^T, dK^T (channels x keys) accumulate over the block's queries.
    const int key = 16 * w + s;
    floatx4 dv[CT], dk[CT];
    {
      const bool kvalid = sm.kidx[key] >= 0;
      const float c2 = scale * kLog2e;
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8*>(&sm.Ks[key][32 * ks + 8 * g4]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) dv[ct] = dk[ct] = zero4();
      auto qtile = [&](int qt) __attribute__((always_inline)) {
        floatx4 sa[2], da[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sa[t] = zero4();
          da[t] = zero4();
          const int q = 32 * qt + 16 * t + s;
          bf16x8 qa[KS], oa[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            qa[ks] = *reinterpret_cast<const bf16x8*>(&sm.Qs[q][32 * ks + 8 * g4]);
            oa[ks] = *reinterpret_cast<const bf16x8*>(&sm.Os[q][32 * ks + 8 * g4]);
          }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            sa[t] = mma16(qa[ks], kf[ks], sa[t]);
            da[t] = mma16(oa[ks], pv[ks], da[t]);
          }
        }
        bf16x8 pf, sf;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r0 = 32 * qt + 16 * t + 4 * g4;
          const floatx4 L4 = *reinterpret_cast<const floatx4*>(&sm.lse[r0]);
          const floatx4 D4 = *reinterpret_cast<const floatx4*>(&sm.Dd[r0]);
          const floatx4 C4 = *reinterpret_cast<const floatx4*>(&sm.cq[r0]);
          float dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = kvalid & !(leaf & (key > r0 + e));
            const float p = __builtin_amdgcn_exp2f(ok ? fmaf(sa[t][e], c2, -L4[e]) : -INFINITY);
            dsv[e] = p * (C4[e] * da[t][e] - D4[e]);
            pf[4 * t + e] = (__bf16)(C4[e] * p);
            sf[4 * t + e] = (__bf16)dsv[e];
          }
          store4(&sm.dST[key][r0], dsv);
        }
        // K order of pf / sf: queries 32 qt + 4 g + e (e < 4), 32 qt + 16 + 4 g + e - 4.
        const int kb1 = 32 * qt + 4 * g4, kb2 = kb1 + 16;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          dv[ct] = mma16(tr16(&sm.Os[0][0], LD, kb1, kb2, 16 * ct, lane), pf, dv[ct]);
          dk[ct] = mma16(tr16(&sm.Qs[0][0], LD, kb1, kb2, 16 * ct, lane), sf, dk[ct]);
        }
      };
      if (leaf) {
        for (int qt = w >> 1; qt < 4; ++qt) qtile(qt);
      } else {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) qtile(qt);
      }
    }
    // Loads for the next block and the indices of the one after.
    const int gn = min(g + G, total - 1);
    const size_t nrb = (size_t)head_of(gn) * N;
    gather(gn);
    prow = rows_of(min(g + 2 * G, total - 1), tid);
    gather_v(nrb);
    // This wave's dQ-phase queries (16 w + s): their channels 16 ct + 4 g .. + 3,
    // read before Qs is reused.
    bf16x4 qv[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      qv[ct] = *reinterpret_cast<const bf16x4*>(&sm.Qs[16 * w + s][16 * ct + 4 * g4]);
    __syncthreads();  // dS^T complete; Qs and Os no longer read
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float xv[4], xk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[e] = dv[ct][e];
        xk[e] = dk[ct][e] * scale;
      }
      store4(&sm.Qs[key][16 * ct + 4 * g4], xv);
      store4(&sm.Os[key][16 * ct + 4 * g4], xk);
    }
    // dQ phase: dQ^T (channels x queries 16 w + s) = K^T dS^T over the block's keys
    // (leaf blocks: keys up to the wave's last query).
    floatx4 dq[CT];
    float sig = 0.0f;
    {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) dq[ct] = zero4();
      const int nks = leaf ? (w >> 1) + 1 : KT / 32;
      for (int ks = 0; ks < nks; ++ks) {
        const int kb = 32 * ks + 8 * g4;
        const bf16x8 bq = tr16(&sm.dST[0][0], LDK, kb, kb + 4, 16 * w, lane);
        sig = frag_sum<T>(bq, sig);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          dq[ct] = mma16(tr16(&sm.Ks[0][0], LD, kb, kb + 4, 16 * ct, lane), bq, dq[ct]);
      }
    }
    sig += __shfl_xor(sig, 16);
    sig += __shfl_xor(sig, 32);
    sig -= own ? sm.sig[16 * w + s] : 0.0f;
    __syncthreads();  // Ks no longer read; dV, dK tiles complete
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float xq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) xq[e] = (dq[ct][e] - sig * (float)qv[ct][e]) * scale;
      store4(&sm.Ks[16 * w + s][16 * ct + 4 * g4], xq);
    }
    __syncthreads();
    {
      const size_t hb = (size_t)bh * slots;
      constexpr int PB = GIT % 2 == 0 ? 2 : 1;
#pragma unroll
      for (int i0 = 0; i0 < GIT; i0 += PB) {
        Vec8<T> a[PB], b2[PB], c[PB];
        int jk[PB], iq[PB], rr[PB], c8[PB];
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const int piece = tid + NT * (i0 + j);
          rr[j] = piece / CH;
          c8[j] = (piece % CH) * 8;
          jk[j] = sm.kidx[rr[j]];
          iq[j] = sm.qidx[rr[j]];
          a[j].load(&sm.Qs[rr[j]][c8[j]]);
          b2[j].load(&sm.Os[rr[j]][c8[j]]);
          c[j].load(&sm.Ks[rr[j]][c8[j]]);
        }
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const size_t slk = !causal ? (size_t)jk[j]
                             : leaf  ? (size_t)jk[j]
                                     : (size_t)N + (size_t)ord * (N / 2) + compact_past(jk[j], N, lev);
          a[j].store_nt(dVp + (hb + slk) * D + c8[j]);
          b2[j].store_nt(dKp + (hb + slk) * D + c8[j]);
          const size_t slq = !causal ? (size_t)iq[j]
                             : leaf  ? (size_t)iq[j]
                                     : (size_t)N + (size_t)ord * (N / 2) + compact_future_b(iq[j], N, lev);
          c[j].store_nt(dQp + (hb + slq) * D + c8[j]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Low-rank branch, query side: one head and span per workgroup, walked forwards in
// steps of STEP tokens by 8 waves. Each query tile of the step is shared by a
// wave of half 0 (waves 0..3, tiles in order) and one of half 1 (waves 4..7, tiles
// in reverse order): each forms dphi(Q) for half of the feature
// tiles and takes it back through its half of the tables; the hyperplane
// gradients da go through LDS so that each wave then forms dQ for half of the
// channels. LDS (WalkSmem): V (XS) and phi(K) (FS) of the step's keys, the
// running key statistics S = sum_j phi(K_j) V_j^T (SF) and z (zr).
template <int LPG>
struct QdaLds {
  float da[4][2][32][2 * LPG];  // [query tile][lane half][token][table pair * 4 + t]
};

template <typename T, int D, int LPG, int STEP, bool SINGLE>
__global__ void __launch_bounds__(512)
    lr_bwd_q_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                    const T* __restrict__ dO, const float* __restrict__ planes,
                    const float* __restrict__ A, const float* __restrict__ z,
                    const float* __restrict__ re, const float* __restrict__ rdd,
                    const T* __restrict__ dQp, float* __restrict__ scratch, T* __restrict__ dQ,
                    const float* __restrict__ RT, int pw, int H, int N, int L, int span,
                    int levels, int causal, float scale, float tau, int grp, int first, int last) {
  typedef MF<T> M;
  typedef Features<T, D, LPG> Feat;
  typedef WalkSmem<T, D, LPG, STEP> Sm;
  constexpr int NW = 8, RP = 16 * LPG, NFT = RP / 32, LDD = Sm::LDD, LDR = Sm::LDR;
  constexpr int QT = STEP / 32, NST = NFT * (D / 32), SPW = (NST + NW - 1) / NW;
  constexpr int NFH = NFT > 1 ? NFT / 2 : 1;            // feature tiles per half
  constexpr int NDA = D / 32, NDH = NDA > 1 ? NDA / 2 : 1;  // channel tiles per half
  constexpr int VCH = D / 8, VIT = (STEP * VCH + 255) / 256;
  __shared__ Sm sm;
  __shared__ T RTs[D * rt_lds_width<LPG>()];
  __shared__ PlanesLds<T, D, LPG> PLs;
  __shared__ QdaLds<LPG> DA;
  const int bh = blockIdx.y, c = blockIdx.x, head = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = tid >> 6;
  // Waves w and w + 4 share a SIMD; the causal part of a query tile grows with
  // its index, so the second half takes the tiles in reverse order and every SIMD
  // gets the same work.
  const int half = w >> 2, qt = half ? 3 - (w & 3) : (w & 3);
  const bool qwave = qt < QT;
  const int r = 16 * L, f0 = 128 * grp, Lg = min(8, L - 8 * grp);
  const float* pl = planes + ((size_t)head * L + 8 * grp) * 4 * D;
  const int t_beg = c * span, t_end = min(N, t_beg + span);
  const float c2 = 2.0f * scale / tau;
  const size_t sidx = causal ? (size_t)bh * (N / span) + c : (size_t)bh;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * D;
  const T* dOh = dO + (size_t)bh * N * D;

  floatx16 st[SPW];
  load_stats<T, D, LPG, SPW, NW>(A + sidx * D * r, r, f0, w, lane, st, &sm.SF[0][0], LDD);
  stage_rt<T, D, LPG, 512>(RT + (size_t)head * D * pw + 32 * grp, pw, RTs, tid);
  stage_planes<T, D, LPG, 512>(pl, Lg, PLs, tid);
  const T* PH = &PLs.p[0][0][0];
  const T* PLo = &PLs.p[PlanesLds<T, D, LPG>::NPART - 1][0][0];
  constexpr int LDP = PlanesLds<T, D, LPG>::LDP;
  for (int f = tid; f < RP; f += 512) sm.zr[f] = f0 + f < r ? z[sidx * r + f0 + f] : 0.0f;
  __syncthreads();  // hyperplanes and statistics staged

  // The walk, compiled per half so that each wave keeps only its half's
  // registers; both halves pass the same barriers.
  auto walk = [&](auto hc) __attribute__((always_inline)) {
    constexpr int HALF = decltype(hc)::value;
    // Rows of one step: the wave's query tile (Q, dO, dd_lr, scale of dnum; both
    // halves), its key tile (K; half 0) and a share of the V rows (half 1). Tokens
    // past the span read a stand-in row; their dnum and dd_lr are zeroed where used
    // and their phi(K) rows are stored as zero.
    typename M::frag qx[D / M::KSTEP], ox[D / M::KSTEP], kx[D / M::KSTEP];
    Vec8<T> vb[VIT];
    float eq = 0.0f, ddq = 0.0f;
    const int ts = tid - 256;  // V staging thread (half 1)
    // (The row terms first: they are used first, so waiting for them leaves the
    // row loads in flight.)
    auto load_q = [&](int s0) __attribute__((always_inline)) {
      const int tok = min(s0 + 32 * qt + col, N - 1);
      const size_t rrow = (size_t)tok * D;
      eq = re[(size_t)bh * N + tok];
      ddq = rdd[(size_t)bh * N + tok];
      prefetch_row_frags<T, D>(Qh + rrow, qx, h);
      prefetch_row_frags<T, D>(dOh + rrow, ox, h);
    };
    // (Also issued when not causal, where they are unused: the loads are then the
    // same on every path, which keeps the waits for them exact.)
    auto load_keys = [&](int s0) __attribute__((always_inline)) {
      if constexpr (HALF == 0)
        prefetch_row_frags<T, D>(Kh + (size_t)min(s0 + 32 * qt + col, N - 1) * D, kx, h);
      if constexpr (HALF == 1) {
  #pragma unroll
        for (int i = 0; i < VIT; ++i) {
          const int it = ts + 256 * i;
          if (it < STEP * VCH) vb[i].load(Vh + (size_t)min(s0 + it / VCH, N - 1) * D + (it % VCH) * 8);
        }
      }
    };
    // The same order as in the walk (keys, then queries), so that the waits for
    // them are the same on the first step as on every other.
    load_keys(t_beg);
    load_q(t_beg);

    for (int s0 = t_beg; s0 < t_end; s0 += STEP) {
      const int qtok = s0 + 32 * qt + col;
      const bool qvalid = qwave && qtok < t_end;
      const float e_q = qvalid ? eq : 0.0f, dd_q = qvalid ? ddq : 0.0f;
      // One step for one half, compiled per half so that only that half's tables
      // are kept. Both halves pass the same two barriers.
      {
        constexpr bool ACTIVE_A = HALF == 0 || NFT >= 2;
        // Staging: phi(K) of key tile qt (half 0) or a share of the V rows (half 1).
        if (causal) {
          if constexpr (HALF == 0) {
            if (qwave)
              Feat::compute_to_row(kx, PH, PLo, LDP, Lg, scale, tau, lane, qvalid, &sm.FS[32 * qt + col][0]);
          } else {
  #pragma unroll
            for (int i = 0; i < VIT; ++i) {
              const int it = ts + 256 * i;
              if (it < STEP * VCH) vb[i].store(&sm.XS[it / VCH][(it % VCH) * 8]);
            }
          }
        }
        // phi(Q) of the query tile, from registers. (dnum = e_q dO: the products
        // below take the dO rows as they are and scale their columns, one per
        // query, by e_q afterwards.)
        Feat Fq;
        if (qwave && ACTIVE_A) {
          // (only this half's tables: the backward below takes only those)
          Fq.template compute<HALF * NFH, NFH>(qx, PH, PLo, LDP, Lg, scale, tau, lane);
        }
        // The next step's keys, issued as soon as this step's are staged so that
        // their latency hides behind the rest of the step (past the span: loads
        // nothing that matters); its queries follow before the statistics update.
        load_keys(s0 + STEP);
        __syncthreads();

        // dphi(Q)^T for this half's feature tiles (rows = features, columns =
        // queries) = S dnum^T + z dd^T + the causally masked part of the step, then
        // back through this half's tables; da to LDS.
        if (qwave && ACTIVE_A) {
          floatx16 df[NFH];
  #pragma unroll
          for (int i = 0; i < NFH; ++i) {
            const int ft = HALF * NFH + i;
            df[i] = zero16();
  #pragma unroll
            for (int ks = 0; ks < D / M::KSTEP; ++ks)
              df[i] = M::mma(row_frag<T>(&sm.SF[0][0], LDD, 32 * ft, 0, ks, lane), ox[ks], df[i]);
  #pragma unroll
            for (int v = 0; v < 16; ++v) df[i][v] = df[i][v] * e_q + sm.zr[32 * ft + acc_row(v, h)] * dd_q;
          }
          if (causal) {
            for (int kt = 0; kt <= qt; ++kt) {
              floatx16 gt = zero16();
  #pragma unroll
              for (int ks = 0; ks < D / M::KSTEP; ++ks)
                gt = M::mma(row_frag<T>(&sm.XS[0][0], LDD, 32 * kt, 0, ks, lane), ox[ks], gt);
  #pragma unroll
              for (int v = 0; v < 16; ++v) {
                gt[v] = gt[v] * e_q + dd_q;
                if (kt == qt && acc_row(v, h) > col) gt[v] = 0.0f;
              }
  #pragma unroll
              for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
                const typename M::frag gf = M::from_acc(gt, ks2);
  #pragma unroll
                for (int i = 0; i < NFH; ++i)
                  df[i] = M::mma(tr_frag<T>(&sm.FS[0][0], LDR, 32 * kt, 32 * (HALF * NFH + i), ks2, lane,
                                            true),
                                 gf, df[i]);
              }
            }
          }
  #pragma unroll
          for (int i = 0; i < NFH; ++i) {
            const int ft = HALF * NFH + i;
            float dphi[16], da4[4];
            tile_to_table(df[i], h, dphi);
            Fq.backward_table(ft, dphi, da4);
            *reinterpret_cast<floatx4*>(&DA.da[qt][h][col][4 * ft]) =
                floatx4{da4[0], da4[1], da4[2], da4[3]};
          }
        }
        __syncthreads();  // da of every table in LDS

        // dQ for this half's channel tiles from every table's da.
        if (qwave && (NDA > 1 || HALF == 0)) {
          float da[LPG / 2][4];
  #pragma unroll
          for (int jp = 0; jp < LPG / 2; ++jp) {
            const floatx4 x = *reinterpret_cast<const floatx4*>(&DA.da[qt][h][col][4 * jp]);
  #pragma unroll
            for (int t = 0; t < 4; ++t) da[jp][t] = x[t];
          }
          floatx16 dx[NDH];
          features_dx<T, D, LPG, T, NDH>(da, RTs, rt_lds_width<LPG>(), c2, lane, dx, HALF * NDH);
          if (qvalid)
            write_grad_row<T, D, NDH, SINGLE>(dx, scratch, dQ, ((size_t)bh * N + qtok) * D, h, first != 0,
                                      last != 0, HALF * NDH);
        }
      }
      load_q(s0 + STEP);
      if (!causal) continue;  // fixed statistics
      advance_stats<T, D, LPG, SPW, STEP, true, NW>(&sm.XS[0][0], LDD, &sm.FS[0][0], LDR, nullptr, w,
                                                    lane, st, &sm.SF[0][0], sm.zr);
      __syncthreads();
    }
  };
  if (half == 0) walk(std::integral_constant<int, 0>{});
  else walk(std::integral_constant<int, 1>{});
}

// ---------------------------------------------------------------------------
// Low-rank branch, key side: one head and span per workgroup, walked backwards in
// steps of STEP tokens by 8 waves. half = w % 2, key tile kt = (w / 2) % 2 for
// waves 0 .. 3 and the reverse for waves 4 .. 7 (see below): waves 0 .. 3 form dK (each half takes half of the feature tiles of dphi(K) and
// its tables; the hyperplane gradients da meet in LDS and each half then forms
// half of the channels of dK), waves 4 .. 7 form dV (each half takes half of the
// channels). LDS (WalkSmem): dnum (XS) and phi(Q) (FS) of the step's queries,
// dd_lr of the step (dd), the running query statistics G = sum_i phi(Q_i) dnum_i^T
// (SF) and g = sum_i phi(Q_i) dd_lr,i (zr); phi(K) of the step's keys (KFs).
template <int LPG>
struct KdaLds {
  float da[2][2][32][2 * LPG];  // [key tile][lane half][token][table pair * 4 + t]
};

template <typename T, int D, int LPG, int STEP, bool SINGLE>
__global__ void __launch_bounds__(512)
    lr_bwd_k_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                    const T* __restrict__ dO, const float* __restrict__ planes,
                    const float* __restrict__ G, const float* __restrict__ gzs,
                    const float* __restrict__ re, const float* __restrict__ rdd,
                    const T* __restrict__ dKp, const T* __restrict__ dVp, float* __restrict__ scrK,
                    float* __restrict__ scrV, T* __restrict__ dK, T* __restrict__ dV,
                    const float* __restrict__ RT, int pw, int H, int N, int L, int span,
                    int levels, int causal, float scale, float tau, int grp, int first, int last) {
  typedef MF<T> M;
  typedef Features<T, D, LPG> Feat;
  typedef WalkSmem<T, D, LPG, STEP> Sm;
  constexpr int NW = 8, RP = 16 * LPG, NFT = RP / 32, LDD = Sm::LDD, LDR = Sm::LDR;
  constexpr int QT = STEP / 32, NST = NFT * (D / 32), SPW = (NST + NW - 1) / NW;
  constexpr int NFH = NFT > 1 ? NFT / 2 : 1;
  constexpr int NJH = LPG / 2 > 1 ? LPG / 4 : 1;  // table pairs per half
  constexpr int NDA = D / 32, NDH = NDA > 1 ? NDA / 2 : 1;
  constexpr int VCH = D / 8, OIT = (STEP * VCH + 255) / 256;  // dnum pieces per dV thread
  __shared__ Sm sm;
  __shared__ T KFs[STEP][LDR];  // phi(K) of the step's keys, [key][feature]
  __shared__ T FSn[STEP][LDR];  // phi(Q): steps of odd index here, even in sm.FS
  __shared__ T RTs[D * rt_lds_width<LPG>()];
  __shared__ PlanesLds<T, D, LPG> PLs;
  __shared__ KdaLds<LPG> DA;
  const int bh = blockIdx.y, c = blockIdx.x, head = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = tid >> 6;
  // role 0: dK, 1: dV. Waves w and w + 4 share a SIMD; the causal part of a key
  // tile shrinks with its index, so the dV waves take the key tiles in reverse
  // order and every SIMD gets the same work.
  const int role = w >> 2, half = w & 1, kt = role ? 1 - ((w >> 1) & 1) : (w >> 1) & 1;
  const bool kwave = kt < QT;
  const int r = 16 * L, f0 = 128 * grp, Lg = min(8, L - 8 * grp);
  const float* pl = planes + ((size_t)head * L + 8 * grp) * 4 * D;
  const int t_beg = c * span, t_end = min(N, t_beg + span);
  const float c2 = 2.0f * scale / tau;
  const size_t sidx = causal ? (size_t)bh * (N / span) + c : (size_t)bh;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * D;
  const T* dOh = dO + (size_t)bh * N * D;
  const int ts = tid - 256;  // dnum staging thread (dV waves)

  floatx16 st[SPW];
  load_stats<T, D, LPG, SPW, NW>(G + sidx * D * r, r, f0, w, lane, st, &sm.SF[0][0], LDD);
  stage_rt<T, D, LPG, 512>(RT + (size_t)head * D * pw + 32 * grp, pw, RTs, tid);
  stage_planes<T, D, LPG, 512>(pl, Lg, PLs, tid);
  const T* PH = &PLs.p[0][0][0];
  const T* PLo = &PLs.p[PlanesLds<T, D, LPG>::NPART - 1][0][0];
  constexpr int LDP = PlanesLds<T, D, LPG>::LDP;
  for (int f = tid; f < RP; f += 512) sm.zr[f] = f0 + f < r ? gzs[sidx * r + f0 + f] : 0.0f;
  __syncthreads();  // hyperplanes and statistics staged

  // The walk, compiled per (role, half) so that each wave keeps only its own
  // role's registers; every instantiation passes the same barriers.
  auto walk = [&](auto rc, auto hc) __attribute__((always_inline)) {
    constexpr int ROLE = decltype(rc)::value, HALF = decltype(hc)::value;
    constexpr int JP0 = HALF * NJH;
    constexpr bool FEAT_HALF = HALF == 0 || LPG / 2 > 1;  // this half owns tables
    // Rows of one step. dK waves: K and V of their key tile. dV waves: Q of query
    // tile kt (for phi(Q)) and a share of the dO rows with their dnum scale and
    // dd_lr. Tokens outside the span read a stand-in row: their phi rows are
    // stored as zero, their dnum rows and dd_lr are zeroed when staged, and no key
    // result of theirs is written.
    typename M::frag xr[D / M::KSTEP], vx[D / M::KSTEP];
    Vec8<T> ob[ROLE == 1 ? OIT : 1];
    float oe[ROLE == 1 ? OIT : 1];
    float ddv = 0.0f;
    // Two parts, each issued as soon as the registers it fills are free: the rows
    // staged at the start of a step (K for dK waves; Q, dO, dd_lr for dV waves) and
    // the V rows of the dK waves, used until the da exchange.
    auto load_v = [&](int s0) __attribute__((always_inline)) {
      if constexpr (ROLE == 0) {
        if (s0 < t_beg) return;
        prefetch_row_frags<T, D>(Vh + (size_t)min(s0 + 32 * kt + col, N - 1) * D, vx, h);
      }
    };
    // dV waves: the Q rows of a step, which they featurize during the step before
    // (in the wait for the dK waves' da) into that step's phi(Q) buffer.
    auto load_q = [&](int s0) __attribute__((always_inline)) {
      if constexpr (ROLE == 1) {
        if (s0 < t_beg) return;
        prefetch_row_frags<T, D>(Qh + (size_t)min(s0 + 32 * kt + col, N - 1) * D, xr, h);
      }
    };
    auto feat_q = [&](int s0, T* fs) __attribute__((always_inline)) {
      if constexpr (ROLE == 1) {
        if (s0 >= t_beg && kwave && FEAT_HALF)
          Feat::template compute_to_row<JP0, NJH>(xr, PH, PLo, LDP, Lg, scale, tau, lane,
                                                  s0 + 32 * kt + col < t_end,
                                                  fs + (size_t)(32 * kt + col) * LDR);
      }
    };
    auto load_rows = [&](int s0) __attribute__((always_inline)) {
      if (s0 < t_beg) return;
      const size_t trow = (size_t)min(s0 + 32 * kt + col, N - 1) * D;
      if constexpr (ROLE == 0) prefetch_row_frags<T, D>(Kh + trow, xr, h);
      if constexpr (ROLE == 1) {
#pragma unroll
        for (int i = 0; i < OIT; ++i) {
          const int it = ts + 256 * i;
          const int tc = min(s0 + it / VCH, N - 1);
          if (it < STEP * VCH) ob[i].load(dOh + (size_t)tc * D + (it % VCH) * 8);
          oe[i] = re[(size_t)bh * N + tc];
        }
        if (ts < STEP) ddv = rdd[(size_t)bh * N + min(s0 + ts, N - 1)];
      }
    };
    const int nstep = (t_end - t_beg + STEP - 1) / STEP;
    auto fs_of = [&](int si) __attribute__((always_inline)) {
      return (si & 1) ? &FSn[0][0] : &sm.FS[0][0];
    };
    load_q(t_beg + (nstep - 1) * STEP);
    feat_q(t_beg + (nstep - 1) * STEP, fs_of(nstep - 1));
    load_q(t_beg + (nstep - 2) * STEP);
    load_rows(t_beg + (nstep - 1) * STEP);
    load_v(t_beg + (nstep - 1) * STEP);

    for (int si = nstep - 1; si >= 0; --si) {
      const int s0 = t_beg + si * STEP;
      const int ktok = s0 + 32 * kt + col;
      const bool kvalid = kwave && ktok < t_end;
      const T* fsc = fs_of(si);  // phi(Q) of this step's queries
      // Staging. dK waves: phi(K) of this half's tables (kept for the backward and
      // stored to KFs). dV waves: phi(Q) of this half's tables to FS, dnum rows to
      // XS, dd_lr.
      Feat Fk;
      if constexpr (ROLE == 0) {
        if (kwave && FEAT_HALF) {
          // (only this half's tables: they are all that is stored and taken back)
          Fk.template compute<JP0, NJH>(xr, PH, PLo, LDP, Lg, scale, tau, lane);
#pragma unroll
          for (int jp = JP0; jp < JP0 + NJH; ++jp) {
            float x0[8], x1[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              x0[b] = kvalid ? Fk.phi[jp][b] : 0.0f;
              x1[b] = kvalid ? Fk.phi[jp][8 + b] : 0.0f;
            }
            store8(&KFs[32 * kt + col][Feat::feat(jp, 0, h)], x0);
            store8(&KFs[32 * kt + col][Feat::feat(jp, 8, h)], x1);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < OIT; ++i) {
          const int it = ts + 256 * i;
          if (it < STEP * VCH) {
            ob[i].scale(s0 + it / VCH < t_end ? oe[i] : 0.0f);
            ob[i].store(&sm.XS[it / VCH][(it % VCH) * 8]);
          }
        }
        if (ts < STEP) sm.dd[ts] = s0 + ts < t_end ? ddv : 0.0f;
      }
      // The next step's staged rows, issued now that this step's are consumed, so
      // that their latency hides behind the rest of the step (before the span:
      // loads nothing).
      load_rows(s0 - STEP);
      __syncthreads();

      if constexpr (ROLE == 0) {
        // dphi(K)^T for this half's feature tiles (rows = features, columns =
        // keys) = G V^T + g 1^T + the part of the step's queries at or after each
        // key; back through this half's tables; da to LDS.
        if (kwave && NFH * HALF < NFT) {
          floatx16 dkt[NFH];
#pragma unroll
          for (int i = 0; i < NFH; ++i) {
            const int ft = HALF * NFH + i;
            dkt[i] = zero16();
#pragma unroll
            for (int ks = 0; ks < D / M::KSTEP; ++ks)
              dkt[i] = M::mma(row_frag<T>(&sm.SF[0][0], LDD, 32 * ft, 0, ks, lane), vx[ks], dkt[i]);
#pragma unroll
            for (int v = 0; v < 16; ++v) dkt[i][v] += sm.zr[32 * ft + acc_row(v, h)];
          }
          if (causal) {
            for (int qt = kt; qt < QT; ++qt) {
              floatx16 gm = zero16();
#pragma unroll
              for (int ks = 0; ks < D / M::KSTEP; ++ks)
                gm = M::mma(row_frag<T>(&sm.XS[0][0], LDD, 32 * qt, 0, ks, lane), vx[ks], gm);
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                gm[v] += sm.dd[32 * qt + acc_row(v, h)];
                if (qt == kt && acc_row(v, h) < col) gm[v] = 0.0f;
              }
#pragma unroll
              for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
                const typename M::frag gf = M::from_acc(gm, ks2);
#pragma unroll
                for (int i = 0; i < NFH; ++i)
                  dkt[i] = M::mma(tr_frag<T>(fsc, LDR, 32 * qt, 32 * (HALF * NFH + i), ks2,
                                             lane, true),
                                  gf, dkt[i]);
              }
            }
          }
#pragma unroll
          for (int i = 0; i < NFH; ++i) {
            const int ft = HALF * NFH + i;
            float dphi[16], da4[4];
            tile_to_table(dkt[i], h, dphi);
            Fk.backward_table(ft, dphi, da4);
            *reinterpret_cast<floatx4*>(&DA.da[kt][h][col][4 * ft]) =
                floatx4{da4[0], da4[1], da4[2], da4[3]};
          }
        }
        load_v(s0 - STEP);  // this step's V rows are no longer needed
      } else if (kwave && (NDA > 1 || HALF == 0)) {
        // dV^T for this half's channel tiles (rows = channels, columns = keys) =
        // G^T phi(K)^T + the step's part.
        floatx16 dvt[NDH];
#pragma unroll
        for (int i = 0; i < NDH; ++i) {
          const int dt = HALF * NDH + i;
          dvt[i] = zero16();
#pragma unroll
          for (int ks = 0; ks < RP / M::KSTEP; ++ks) {
            const int fk = Feat::frag_feat(ks, 0, h);
            dvt[i] = M::mma(tr_rows(&sm.SF[0][0], LDD, fk, fk + 4, 32 * dt, lane),
                            M::load(&KFs[32 * kt + col][fk]), dvt[i]);
          }
        }
        if (causal) {
          for (int qt = kt; qt < QT; ++qt) {
            floatx16 wq = zero16();
#pragma unroll
            for (int ks = 0; ks < RP / M::KSTEP; ++ks)
              wq = M::mma(M::load(fsc + (size_t)(32 * qt + col) * LDR + Feat::frag_feat(ks, 0, h)),
                          M::load(&KFs[32 * kt + col][Feat::frag_feat(ks, 0, h)]), wq);
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (qt == kt && acc_row(v, h) < col) wq[v] = 0.0f;
#pragma unroll
            for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
              const typename M::frag wf = M::from_acc(wq, ks2);
#pragma unroll
              for (int i = 0; i < NDH; ++i)
                dvt[i] = M::mma(tr_frag<T>(&sm.XS[0][0], LDD, 32 * qt, 32 * (HALF * NDH + i), ks2,
                                           lane, true),
                                wf, dvt[i]);
            }
          }
        }
        if (kvalid)
          write_grad_row<T, D, NDH, SINGLE>(dvt, scrV, dV, ((size_t)bh * N + ktok) * D, h, first != 0,
                                    last != 0, HALF * NDH);
      }
      if constexpr (ROLE == 1) {
        // While the dK waves finish their da: phi(Q) of the next step (walking
        // backwards) into its buffer, then the Q rows of the step after it.
        if (si > 0) {
          feat_q(s0 - STEP, fs_of(si - 1));
          load_q(s0 - 2 * STEP);
        }
      }
      __syncthreads();  // da of every table in LDS

      // dK for this half's channel tiles from every table's da.
      if constexpr (ROLE == 0) {
        if (kwave && (NDA > 1 || HALF == 0)) {
          float da[LPG / 2][4];
#pragma unroll
          for (int jp = 0; jp < LPG / 2; ++jp) {
            const floatx4 x = *reinterpret_cast<const floatx4*>(&DA.da[kt][h][col][4 * jp]);
#pragma unroll
            for (int t = 0; t < 4; ++t) da[jp][t] = x[t];
          }
          floatx16 dx[NDH];
          features_dx<T, D, LPG, T, NDH>(da, RTs, rt_lds_width<LPG>(), c2, lane, dx, HALF * NDH);
          if (kvalid)
            write_grad_row<T, D, NDH, SINGLE>(dx, scrK, dK, ((size_t)bh * N + ktok) * D, h, first != 0,
                                      last != 0, HALF * NDH);
        }
      }
      if (!causal) continue;  // fixed statistics
      advance_stats<T, D, LPG, SPW, STEP, true, NW>(&sm.XS[0][0], LDD, fsc, LDR, sm.dd, w,
                                                    lane, st, &sm.SF[0][0], sm.zr);
      __syncthreads();
    }
  };
  if (role == 0) {
    if (half == 0) walk(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
  } else {
    if (half == 0) walk(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
  }
}

// ---------------------------------------------------------------------------

namespace {

int rt_stride(const Problem& pb);

// Workgroups of a persistent launch: as many as fit on the device at once.
struct BwdLayout {
  size_t rows, dlam, parts, gsum, gstate, rt, scratch, bids, extra, total;
  int nblk;
};

BwdLayout bwd_layout(const Problem& pb) {
  const size_t BH = (size_t)pb.B * pb.H, N = pb.N, D = pb.d;
  const size_t slots = partial_slots(pb.N, pb.levels, pb.causal, pb.rounds);
  const int rpb = 256 / (pb.d / 8);
  BwdLayout l;
  l.nblk = (pb.N + rpb - 1) / rpb;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  l.rows = off; off += al(sizeof(float) * 5 * BH * N);
  l.dlam = off; off += al(sizeof(float) * BH * l.nblk);
  l.parts = off; off += al(3 * BH * slots * D * pb.elem);
  l.gsum = off; off += al(summary_ws_bytes(pb));
  l.gstate = off; off += al(sizeof(float) * BH * pb.nA * (D * pb.r + pb.r));
  l.rt = off; off += al(sizeof(float) * pb.H * D * rt_stride(pb));
  const int groups = padded_tables(pb.L) > 8 ? 2 : 1;
  l.scratch = off; off += groups > 1 ? al(sizeof(float) * 3 * BH * N * D) : 0;
  l.bids = off; off += al(block_ids_bytes(pb));
  l.extra = off; off += al(extra_layout(pb, true).total);
  l.total = off;
  return l;
}


// Row stride of the transposed hyperplanes (covers the reads of every group).
int rt_stride(const Problem& pb) {
  const int w = 4 * padded_tables(pb.L);
  return w < 32 ? 32 : w;
}

}  // namespace

size_t bwd_ws_bytes(const Problem& pb) { return bwd_layout(pb).total; }

size_t bwd_lds_need(const Problem& pb) {
  const size_t e = pb.elem, d = pb.d, kt = pb.s < 32 ? 32 : pb.s;
  const size_t sb = e * (2 * kt * (d + (pb.bf16 ? 24 : 8))) + 24 * kt +  // one-role launch
                    (pb.rounds > 1 ? 8 * (kMaxRounds - 1) * kt : 0);
  size_t lr = 0;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      auto need = [&](auto lc) {
        constexpr int LPG = ELSAA_C(lc);
        constexpr size_t RTB = sizeof(T) * D * rt_lds_width<LPG>() + sizeof(PlanesLds<T, D, LPG>);
        constexpr int SQ = walk_step<T, D, LPG, 128, RTB + sizeof(QdaLds<LPG>)>();
        constexpr int SK = walk_step<T, D, LPG, 64,
                                     RTB + sizeof(KdaLds<LPG>) + 2 * sizeof(T) * 64 * tile_ld<T>(16 * LPG)>();
        const size_t a = RTB + sizeof(QdaLds<LPG>) +
                         (SQ > 0 ? sizeof(WalkSmem<T, D, LPG, SQ>) : sizeof(WalkSmem<T, D, LPG, 32>));
        const size_t b = RTB + sizeof(KdaLds<LPG>) +
                         (SK > 0 ? sizeof(WalkSmem<T, D, LPG, SK>) : sizeof(WalkSmem<T, D, LPG, 32>)) +
                         2 * sizeof(T) * (SK > 0 ? SK : 32) * tile_ld<T>(16 * LPG);
        lr = a > b ? a : b;
      };
      switch (padded_tables(pb.L)) {
        case 2: need(std::integral_constant<int, 2>{}); break;
        case 4: need(std::integral_constant<int, 4>{}); break;
        default: need(std::integral_constant<int, 8>{}); break;
      }
    });
  });
  return sb > lr ? sb : lr;
}

bool launch_bwd(const Problem& pb, const void* Q, const void* K, const void* V, const void* dO,
                const float* O_s, const void* O_lr, const float* planes_lr, const int32_t* qperm,
                const int32_t* kperm, const float* A, const float* z, const float* lse,
                const float* d_lr, const float* lambda, const float* g_s, const float* g_lr,
                const int32_t* extra, void* dQ, void* dK, void* dV, float* dlambda, float* dg_s,
                float* dg_lr, void* ws, hipStream_t st, bool dry) {
  bool ok = true;
  const BwdLayout lay = bwd_layout(pb);
  char* base = (char*)ws;
  const size_t BH = (size_t)pb.B * pb.H, N = pb.N;
  float* rc = (float*)(base + lay.rows);
  float* rD = rc + BH * N;
  float* re = rD + BH * N;
  float* rdd = re + BH * N;
  float* rsig = rdd + BH * N;
  float* dlam_part = (float*)(base + lay.dlam);
  const size_t slots = partial_slots(pb.N, pb.levels, pb.causal, pb.rounds);
  char* parts = base + lay.parts;
  const size_t pbytes = BH * slots * pb.d * pb.elem;
  void* dQp = parts;
  void* dKp = parts + pbytes;
  void* dVp = parts + 2 * pbytes;
  float* S = (float*)(base + lay.gsum);
  float* Z = S + BH * lr_tiles(pb) * pb.d * pb.r;
  float* Gs = (float*)(base + lay.gstate);
  float* gzs = Gs + BH * pb.nA * pb.d * pb.r;
  float* scr = (float*)(base + lay.scratch);
  float* RT = (float*)(base + lay.rt);
  const int pw = rt_stride(pb);
  const int groups = padded_tables(pb.L) > 8 ? 2 : 1;
  float* scrQ = scr;
  float* scrK = scr + BH * N * pb.d;
  float* scrV = scr + 2 * BH * N * pb.d;
  int32_t* qbid = (int32_t*)(base + lay.bids);
  int32_t* kbid = qbid + block_ids_bytes(pb) / (2 * sizeof(int32_t));
  const int nord = pb.causal ? pb.rounds * pb.levels : pb.rounds;
  const int items = pb.causal ? nord * (pb.N / 2) / pb.s + pb.N / pb.s : nord * (pb.N / pb.s);
  if (!dry && (pb.rounds > 1 || pb.E > 0)) launch_block_ids(pb, qperm, kperm, qbid, kbid, st);
  const ExtraLayout xl = extra_layout(pb, true);
  char* xb = base + lay.extra;
  int32_t* jq = (int32_t*)(xb + xl.jq);
  const size_t xrow = BH * N * pb.d * pb.elem;
  void* dQx = pb.E ? xb + xl.rows : nullptr;
  void* dKx = pb.E ? xb + xl.rows + xrow : nullptr;
  void* dVx = pb.E ? xb + xl.rows + 2 * xrow : nullptr;

  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      if (!dry) {
        ELSAA_LAUNCH("planes_t", planes_transpose_kernel, dim3(pb.H), dim3(256), 0, st, planes_lr,
                     pb.L, pb.d, pw, RT);
        ELSAA_LAUNCH("bwd_rows", (bwd_rows_kernel<T, D>), dim3(lay.nblk, BH), dim3(256), 0, st,
                           (const T*)dO, O_s, (const T*)O_lr, lse, d_lr, lambda, g_s,
                           g_lr, pb.eps, pb.H, pb.N, rc, rD, rsig, re, rdd, dg_s, dg_lr,
                           dlam_part);
        if (dlambda)
          ELSAA_LAUNCH("dlam_reduce", dlam_reduce_kernel, dim3(pb.H), dim3(256), 0, st, dlam_part,
                             pb.B, pb.H, lay.nblk, dlambda);
        run_lr_sums(pb, Q, dO, re, rdd, planes_lr, S, Z, st);
        run_lr_scan(pb, S, Z, pb.causal ? 2 : 0, Gs, gzs, st);
        if (pb.E > 0) {
          int32_t* const sb[4] = {(int32_t*)(xb + xl.sort[0]), (int32_t*)(xb + xl.sort[1]),
                                  (int32_t*)(xb + xl.sort[2]), (int32_t*)(xb + xl.sort[3])};
          const int32_t *skey = nullptr, *sval = nullptr;
          launch_extra_prep(pb, extra, qbid, kbid, jq, sb[0], sb[1], st);
          launch_extra_sort(pb, sb, (int32_t*)(xb + xl.table), &skey, &sval, st);
          launch_extra_bwd(pb, Q, K, V, dO, lse, rc, rD, jq, skey, sval, dQx, dKx, dVx, st);
        }
      }
      auto run_sparse = [&](auto sc) {
        constexpr int SB = ELSAA_C(sc);
        auto go = [&](auto mc) {
          constexpr bool MR = decltype(mc)::value;
          const dim3 grid(items, BH);
          // The kernels read an order entry for every row, leaves included; with no
          // level (causal, N = s) the orders are empty and may be null, and the
          // entry read (and discarded) is then the first row term.
          const int32_t* qp = qperm ? qperm : (const int32_t*)rc;
          const int32_t* kp = kperm ? kperm : (const int32_t*)rc;
          if constexpr (!(std::is_same_v<T, __bf16> && SB <= 128 &&
                          sizeof(Sb2Smem<D, SB, MR>) <= kLdsBytes) &&
                        !(sizeof(SbwdSmem<T, D, SB, 3, MR>) <= kLdsBytes && SB <= 128) &&
                        !(sizeof(SbwdSmem<T, D, SB, 1, MR>) <= kLdsBytes)) {
            ok = false;
          } else if (dry) {
          } else if constexpr (std::is_same_v<T, __bf16> && SB == 128 && !MR &&
                               (D == 64 || D == 128)) {
            const int total = items * (int)BH;
            const int G = persistent_grid((const void*)sparse_bwd3_kernel<D>, 512, total);
            ELSAA_LAUNCH("sparse_bwd", (sparse_bwd3_kernel<D>), dim3(G), dim3(512), 0, st,
                         (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, (const __bf16*)dO,
                         lse, rc, rD, rsig, qp, kp, pb.N, (int)pb.causal, pb.levels, pb.scale,
                         items, total, (__bf16*)dQp, (__bf16*)dKp, (__bf16*)dVp);
          } else if constexpr (std::is_same_v<T, __bf16> && SB <= 128 &&
                               sizeof(Sb2Smem<D, SB, MR>) <= kLdsBytes) {
            constexpr int NT = 64 * (SB < 32 ? 1 : SB / 32);
            const int total = items * (int)BH;
            const int G = persistent_grid((const void*)sparse_bwd2_kernel<D, SB, MR>, NT, total);
            ELSAA_LAUNCH("sparse_bwd", (sparse_bwd2_kernel<D, SB, MR>), dim3(G), dim3(NT), 0, st,
                         (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, lse, rc, rD, rsig, qp,
                         kp, pb.N, (int)pb.causal, pb.levels, pb.rounds, qbid, kbid, pb.scale,
                         items, total, (T*)dQp, (T*)dKp, (T*)dVp);
          } else if constexpr (sizeof(SbwdSmem<T, D, SB, 3, MR>) <= kLdsBytes && SB <= 128) {
            ELSAA_LAUNCH("sparse_bwd", (sparse_bwd_kernel<T, D, SB, 3, MR>), grid,
                         dim3(sbwd_threads<SB>(3)), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                         (const T*)dO, lse, rc, rD, rsig, qp, kp, pb.N, (int)pb.causal, pb.levels,
                         pb.rounds, qbid, kbid, pb.scale, (T*)dQp, (T*)dKp, (T*)dVp);
          } else if constexpr (sizeof(SbwdSmem<T, D, SB, 1, MR>) <= kLdsBytes) {
            ELSAA_LAUNCH("sparse_bwd", (sparse_bwd_kernel<T, D, SB, 1, MR>), grid,
                         dim3(sbwd_threads<SB>(1)), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                         (const T*)dO, lse, rc, rD, rsig, qp, kp, pb.N, (int)pb.causal, pb.levels,
                         pb.rounds, qbid, kbid, pb.scale, (T*)dQp, (T*)dKp, (T*)dVp);
            ELSAA_LAUNCH("sparse_bwd_q", (sparse_bwd_kernel<T, D, SB, 2, MR>), grid,
                         dim3(sbwd_threads<SB>(2)), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                         (const T*)dO, lse, rc, rD, rsig, qp, kp, pb.N, (int)pb.causal, pb.levels,
                         pb.rounds, qbid, kbid, pb.scale, (T*)dQp, (T*)dKp, (T*)dVp);
          }
        };
        if (pb.rounds > 1) go(std::true_type{});
        else go(std::false_type{});
      };
      switch (pb.s) {
        case 16: run_sparse(std::integral_constant<int, 16>{}); break;
        case 32: run_sparse(std::integral_constant<int, 32>{}); break;
        case 64: run_sparse(std::integral_constant<int, 64>{}); break;
        case 128: run_sparse(std::integral_constant<int, 128>{}); break;
        default: run_sparse(std::integral_constant<int, 256>{}); break;
      }
      auto run_lr = [&](auto lc) {
        constexpr int LPG = ELSAA_C(lc);
        constexpr size_t RTB = sizeof(T) * D * rt_lds_width<LPG>() + sizeof(PlanesLds<T, D, LPG>);
        constexpr int SQ = walk_step<T, D, LPG, 128, RTB + sizeof(QdaLds<LPG>)>();
        constexpr int SK = walk_step<T, D, LPG, 64,
                                     RTB + sizeof(KdaLds<LPG>) + 2 * sizeof(T) * 64 * tile_ld<T>(16 * LPG)>();
        if constexpr (SQ == 0 || SK == 0) {
          ok = false;
        } else if (!dry) {
          const int span_q = pb.causal ? pb.chunk : noncausal_span(pb.N, (int)BH, SQ);
          const int span_k = pb.causal ? pb.chunk : noncausal_span(pb.N, (int)BH, SK);
          // One feature group: the gradients go straight out (SINGLE); two: the
          // first group's part is kept in fp32 scratch and added by the second.
          auto launch_group = [&](auto sc, int g) {
            constexpr bool SINGLE = decltype(sc)::value;
            const int first = g == 0, last = g == groups - 1;
            ELSAA_LAUNCH("lr_bwd_q", (lr_bwd_q_kernel<T, D, LPG, SQ, SINGLE>),
                         dim3((pb.N + span_q - 1) / span_q, BH), dim3(512), 0, st, (const T*)Q,
                         (const T*)K, (const T*)V, (const T*)dO, planes_lr, A, z, re, rdd,
                         (const T*)dQp, scrQ, (T*)dQ, RT, pw, pb.H, pb.N, pb.L, span_q,
                         pb.levels, (int)pb.causal, pb.scale, pb.tau, g, first, last);
            ELSAA_LAUNCH("lr_bwd_k", (lr_bwd_k_kernel<T, D, LPG, SK, SINGLE>),
                         dim3((pb.N + span_k - 1) / span_k, BH), dim3(512), 0, st, (const T*)Q,
                         (const T*)K, (const T*)V, (const T*)dO, planes_lr, Gs, gzs, re, rdd,
                         (const T*)dKp, (const T*)dVp, scrK, scrV, (T*)dK, (T*)dV, RT, pw, pb.H,
                         pb.N, pb.L, span_k, pb.levels, (int)pb.causal, pb.scale, pb.tau, g,
                         first, last);
          };
          if (groups == 1) {
            launch_group(std::true_type{}, 0);
          } else {
            for (int g = 0; g < groups; ++g) launch_group(std::false_type{}, g);
          }
        }
      };
      switch (padded_tables(pb.L)) {
        case 2: run_lr(std::integral_constant<int, 2>{}); break;
        case 4: run_lr(std::integral_constant<int, 4>{}); break;
        default: run_lr(std::integral_constant<int, 8>{}); break;
      }
      if (!dry) launch_combine(pb, dQp, dKp, dVp, dQx, dKx, dVx, dQ, dK, dV, st);
    });
  });
  return ok;
}

}  // namespace elsaa
