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
// Kernels, in launch order:
//   bwd_rows_kernel      per-row terms above, dg_s, dg_lr, per-block dlambda sums;
//   dlam_reduce_kernel   dlambda per head (fixed order: deterministic);
//   lr_sums + lr_scan    (lowrank.hip) G = sum_i phi(Q_i) dnum_i^T, g = sum_i
//                        phi(Q_i) dd_lr,i per chunk, combined as the exclusive suffix
//                        over chunks (causal) or the total;
//   sparse_bwd_kernel    per selected block: dQ, dK, dV partials per level slot;
//   lr_bwd_q_kernel      query side of the low-rank branch, walking each chunk
//                        forwards with the running key statistics A, z:
//                        dphi(Q_i) = sum_{j<=i} (<dnum_i, V_j> + dd_lr,i) phi(K_j),
//                        then through the features to dQ, plus the sparse dQ
//                        partials -> dQ;
//   lr_bwd_k_kernel      key side, walking each chunk backwards with the running
//                        query statistics G, g:
//                        dphi(K_j) = sum_{i>=j} (<dnum_i, V_j> + dd_lr,i) phi(Q_i),
//                        dV_j += sum_{i>=j} (phi(Q_i).phi(K_j)) dnum_i, plus the sparse
//                        partials -> dK, dV.
// Features are processed in groups of at most 8 tables (128 features); with two
// groups the first launch leaves an fp32 running sum that the second completes.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

__device__ __forceinline__ int compact_future_b(int i, int N, int l) {
  const int n = N >> l, half = n >> 1;
  return (i / n) * half + (i % n) - half;
}
__device__ __forceinline__ int compact_past(int j, int N, int l) {
  const int n = N >> l;
  return (j / n) * (n >> 1) + (j % n);
}

// Accumulates, for this lane's token and the D-layout rows of every 32-row tile
// (d = 32 dt + 8 g + 4 h + e), the sum of the token's sparse partial slots:
// leaf/own slot, then each level where the token is a query of a future half
// (QUERY) or a key of a past half (!QUERY).
template <typename T, int D, bool QUERY>
__device__ __forceinline__ void sum_partials(const T* part, int bh, size_t slots, int tok, int N,
                                             int levels, bool causal, int h,
                                             float (&acc)[D / 32][4][4]) {
  const int logN = 31 - __clz(N);
  for (int l = -1; l < levels; ++l) {
    size_t sl;
    if (l < 0) {
      sl = (size_t)tok;
    } else {
      if (!causal) break;
      const bool fut = (tok >> (logN - 1 - l)) & 1;
      if (QUERY != fut) continue;
      sl = (size_t)N + (size_t)l * (N / 2) +
           (QUERY ? compact_future_b(tok, N, l) : compact_past(tok, N, l));
    }
    const T* src = part + ((size_t)bh * slots + sl) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
        load4(src + 32 * dt + 8 * g + 4 * h, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[dt][g][e] += x[e];
      }
  }
}

// Final write of one gradient row held in D layout (lane = token, rows = d):
// value = (first ? sparse partial sum : fp32 running sum) + lr, stored as T
// (last) or kept as the fp32 running sum for the next feature group.
template <typename T, int D, bool QUERY>
__device__ __forceinline__ void finish_row(const T* part, float* scratch, T* out, int bh,
                                           size_t slots, int tok, int N, int levels, bool causal,
                                           int h, const floatx16 (&lr)[D / 32], bool first,
                                           bool last) {
  float acc[D / 32][4][4];
  const size_t row = ((size_t)bh * N + tok) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (first) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[dt][g][e] = 0.0f;
      } else {
        load4(scratch + row + 32 * dt + 8 * g + 4 * h, acc[dt][g]);
      }
    }
  if (first) sum_partials<T, D, QUERY>(part, bh, slots, tok, N, levels, causal, h, acc);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[dt][g][e] + lr[dt][4 * g + e];
      const size_t o = row + 32 * dt + 8 * g + 4 * h;
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
    bwd_rows_kernel(const T* __restrict__ dO, const T* __restrict__ Os, const T* __restrict__ Olr,
                    const float* __restrict__ lse, const float* __restrict__ dlr,
                    const float* __restrict__ lambda, const float* __restrict__ gs,
                    const float* __restrict__ glr, float eps, int H, int N, float* __restrict__ rc,
                    float* __restrict__ rD, float* __restrict__ re, float* __restrict__ rdd,
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
      a += x * to_f(Os[row + e]);
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
template <typename T, int D, int SB, int ROLE>
struct SbwdSmem {
  static constexpr int KT = SB < 32 ? 32 : SB;
  static constexpr int LD = tile_ld<T>(D);
  static constexpr bool HK = (ROLE & 2) != 0;  // all keys staged (query waves)
  static constexpr bool HQ = (ROLE & 1) != 0;  // all queries staged (key waves)
  T Ks[HK ? KT : 1][LD];
  T Vs[HK ? KT : 1][LD];
  T Qs[HQ ? KT : 1][LD];
  T Os[HQ ? KT : 1][LD];  // c * dO
  float lse[KT], Dd[KT], cq[KT];
  int kidx[KT], qidx[KT];
};

template <int SB>
constexpr int sbwd_threads(int role) {
  return 64 * (SB < 32 ? 1 : SB / 32) * (role == 3 ? 2 : 1);
}

// Row fragments of one token row read from global memory, scaled.
template <typename T, int D>
__device__ __forceinline__ void row_frags(const T* x, bool valid, float sc,
                                          typename MF<T>::frag (&f)[D / MF<T>::KSTEP], int h) {
  typedef MF<T> M;
#pragma unroll
  for (int ks = 0; ks < D / M::KSTEP; ++ks) {
    if (!valid) {
      f[ks] = M::zero();
    } else if (sc == 1.0f) {
      f[ks] = M::load(x + ks * M::KSTEP + M::KPL * h);
    } else {
      float v[M::KPL];
      if constexpr (M::KPL == 8) load8(x + ks * M::KSTEP + M::KPL * h, v);
      else v[0] = to_f(x[ks * M::KSTEP + M::KPL * h]);
#pragma unroll
      for (int e = 0; e < M::KPL; ++e) v[e] *= sc;
      f[ks] = M::from_floats(v);
    }
  }
}

template <typename T, int D, int SB, int ROLE>
__global__ void __launch_bounds__(sbwd_threads<SB>(ROLE))
    sparse_bwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                      const T* __restrict__ dO, const float* __restrict__ lse,
                      const float* __restrict__ rc, const float* __restrict__ rD,
                      const int32_t* __restrict__ qperm, const int32_t* __restrict__ kperm, int N,
                      int causal, int levels, float scale, T* __restrict__ dQp,
                      T* __restrict__ dKp, T* __restrict__ dVp) {
  typedef MF<T> M;
  typedef SbwdSmem<T, D, SB, ROLE> Sm;
  constexpr int KT = Sm::KT, NW = KT / 32, LD = Sm::LD;
  constexpr int NT = sbwd_threads<SB>(ROLE);
  __shared__ Sm sm;
  const int bh = blockIdx.y, item = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const size_t P = perm_stride(N, levels, causal);
  const size_t slots = partial_slots(N, levels, causal);
  const size_t rowbase = (size_t)bh * N;

  const int per_level = causal ? (N / 2) / SB : 0;
  const int nlev_items = causal ? levels * per_level : 0;
  const int32_t* qsrc = nullptr;
  const int32_t* ksrc = nullptr;
  int lev = -1, tok0 = 0;
  bool leaf = false;
  if (causal && item < nlev_items) {
    lev = item / per_level;
    const int b = item % per_level;
    qsrc = qperm + (size_t)bh * P + (size_t)lev * (N / 2) + (size_t)b * SB;
    ksrc = kperm + (size_t)bh * P + (size_t)lev * (N / 2) + (size_t)b * SB;
  } else if (causal) {
    leaf = true;
    tok0 = (item - nlev_items) * SB;
  } else {
    qsrc = qperm + (size_t)bh * P + (size_t)item * SB;
    ksrc = kperm + (size_t)bh * P + (size_t)item * SB;
  }
  for (int t = tid; t < KT; t += NT) {
    const int kj = t < SB ? (leaf ? tok0 + t : ksrc[t]) : -1;
    const int qi = t < SB ? (leaf ? tok0 + t : qsrc[t]) : -1;
    sm.kidx[t] = kj;
    sm.qidx[t] = qi;
    sm.lse[t] = qi >= 0 ? lse[rowbase + qi] : 0.0f;
    sm.Dd[t] = qi >= 0 ? rD[rowbase + qi] : 0.0f;
    sm.cq[t] = qi >= 0 ? rc[rowbase + qi] : 0.0f;
  }
  __syncthreads();
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
      const size_t ksl = lev >= 0 ? (size_t)N + (size_t)lev * (N / 2) + compact_past(jk, N, lev)
                                  : (size_t)jk;
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
#pragma unroll
          for (int ks = 0; ks < D / M::KSTEP; ++ks)
            s = M::mma(row_frag<T>(&sm.Qs[0][0], LD, 32 * qt, 0, ks, lane), kf[ks], s);
          floatx16 dp = zero16();
          if (pass == 1) {
#pragma unroll
            for (int ks = 0; ks < D / M::KSTEP; ++ks)
              dp = M::mma(row_frag<T>(&sm.Os[0][0], LD, 32 * qt, 0, ks, lane), vf[ks], dp);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qr = 32 * qt + acc_row(v, h);
            const bool ok = kvalid && sm.qidx[qr] >= 0 && !(leaf && key > qr);
            const float p = ok ? fast_exp(s[v] * scale - sm.lse[qr]) : 0.0f;
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
        if (kvalid) {
          T* dst = (pass == 0 ? dVp : dKp) + ((size_t)bh * slots + ksl) * D;
          const float f = pass == 0 ? 1.0f : scale;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float x[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = acc[dt][4 * g + e] * f;
              store4(dst + 32 * dt + 8 * g + 4 * h, x);
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
        row_frags<T, D>(dO + (rowbase + (qvalid ? iq : 0)) * D, qvalid, sm.cq[query], of, h);
      }
      const float lq = sm.lse[query], dq = sm.Dd[query];
      floatx16 acc[D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
      const int nkt = leaf ? qw + 1 : KT / 32;
      for (int kt = 0; kt < nkt; ++kt) {
        floatx16 s = zero16(), dp = zero16();
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks) {
          s = M::mma(row_frag<T>(&sm.Ks[0][0], LD, 32 * kt, 0, ks, lane), qf[ks], s);
          dp = M::mma(row_frag<T>(&sm.Vs[0][0], LD, 32 * kt, 0, ks, lane), of[ks], dp);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kr = 32 * kt + acc_row(v, h);
          const bool ok = qvalid && sm.kidx[kr] >= 0 && !(leaf && kr > query);
          const float p = ok ? fast_exp(s[v] * scale - lq) : 0.0f;
          s[v] = p * (dp[v] - dq);
        }
#pragma unroll
        for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
          const typename M::frag sf = M::from_acc(s, ks2);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            acc[dt] = M::mma(tr_frag<T>(&sm.Ks[0][0], LD, 32 * kt, 32 * dt, ks2, lane, true), sf, acc[dt]);
        }
      }
      if (qvalid) {
        const size_t sl = lev >= 0 ? (size_t)N + (size_t)lev * (N / 2) + compact_future_b(iq, N, lev)
                                   : (size_t)iq;
        T* dst = dQp + ((size_t)bh * slots + sl) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[dt][4 * g + e] * scale;
            store4(dst + 32 * dt + 8 * g + 4 * h, x);
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Low-rank branch, query side. 128 tokens per step, wave w owns query tile w.
template <typename T, int D, int LPG>
struct LbqSmem {
  static constexpr int RP = 16 * LPG, STEP = 128;
  T AF[RP][D + 8];      // running key statistics A = sum phi(K) V^T, [feature][channel]
  T KFT[RP][STEP + 8];  // phi(K) of the step's keys, [feature][key]
  T VS[STEP][D + 8];    // V of the step's keys
  float zr[RP];         // running sum of phi(K)
};

template <typename T, int D, int LPG>
__global__ void __launch_bounds__(256)
    lr_bwd_q_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                    const T* __restrict__ dO, const float* __restrict__ planes,
                    const float* __restrict__ A, const float* __restrict__ z,
                    const float* __restrict__ re, const float* __restrict__ rdd,
                    const T* __restrict__ dQp, float* __restrict__ scratch, T* __restrict__ dQ,
                    const float* __restrict__ RT, int pw, int H, int N, int L, int span,
                    int levels, int causal, float scale, float tau, int grp, int first, int last) {
  typedef MF<T> M;
  typedef Features<T, D, LPG> Feat;
  constexpr int RP = 16 * LPG, STEP = 128, NFT = RP / 32;
  constexpr int NST = NFT * (D / 32), SPW = (NST + 3) / 4;
  __shared__ LbqSmem<T, D, LPG> sm;
  const int bh = blockIdx.y, c = blockIdx.x, head = bh % H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int r = 16 * L, f0 = 128 * grp, Lg = min(8, L - 8 * grp);
  const float* pl = planes + ((size_t)head * L + 8 * grp) * 4 * D;
  const int t_beg = c * span, t_end = min(N, t_beg + span);
  const size_t slots = partial_slots(N, levels, causal);
  const float c2 = 2.0f * scale / tau;
  const size_t sidx = causal ? (size_t)bh * (N / span) + c : (size_t)bh;
  const float* Ac = A + sidx * D * r;
  const float* zc = z + sidx * r;

  // State tiles (ft, dt): D layout with lanes = channels, rows = features.
  floatx16 st[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    st[i] = zero16();
    const int tix = w + 4 * i;
    if (causal && tix < NST) {
      const int dt = tix % (D / 32), ft = tix / (D / 32), d = 32 * dt + col;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int f = f0 + 32 * ft + acc_row(v, h);
        st[i][v] = f < r ? Ac[(size_t)d * r + f] : 0.0f;
      }
    }
  }
  for (int idx = tid; idx < RP * D; idx += blockDim.x) {
    const int d = idx / RP, f = idx % RP;
    sm.AF[f][d] = from_f<T>(f0 + f < r ? Ac[(size_t)d * r + f0 + f] : 0.0f);
  }
  for (int f = tid; f < RP; f += blockDim.x) sm.zr[f] = f0 + f < r ? zc[f0 + f] : 0.0f;

  for (int s0 = t_beg; s0 < t_end; s0 += STEP) {
    if (causal) {
      const int tok = s0 + 32 * w + col;
      const bool valid = tok < t_end;
      Feat Fk;
      Fk.compute(K + ((size_t)bh * N + (valid ? tok : t_beg)) * D, valid, pl, Lg, scale, tau, lane);
#pragma unroll
      for (int jp = 0; jp < LPG / 2; ++jp)
#pragma unroll
        for (int b = 0; b < 16; ++b)
          sm.KFT[Feat::feat(jp, b, h)][32 * w + col] = from_f<T>(valid ? Fk.phi[jp][b] : 0.0f);
      for (int idx = tid; idx < STEP * (D / 8); idx += blockDim.x) {
        const int t = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
        const int tk = s0 + t;
        if (tk < t_end) {
          copy8(&sm.VS[t][c8], V + ((size_t)bh * N + tk) * D + c8);
        } else {
          const float zz[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          store8(&sm.VS[t][c8], zz);
        }
      }
    }
    const int qtok = s0 + 32 * w + col;
    const bool qvalid = qtok < t_end;
    Feat Fq;
    Fq.compute(Q + ((size_t)bh * N + (qvalid ? qtok : t_beg)) * D, qvalid, pl, Lg, scale, tau, lane);
    typename M::frag dn[D / M::KSTEP];
    float ddq = 0.0f;
    {
      const float e = qvalid ? re[(size_t)bh * N + qtok] : 0.0f;
      ddq = qvalid ? rdd[(size_t)bh * N + qtok] : 0.0f;
      const T* orow = dO + ((size_t)bh * N + (qvalid ? qtok : t_beg)) * D;
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks) {
        float x[M::KPL];
        if constexpr (M::KPL == 8) {
          load8(orow + ks * M::KSTEP + M::KPL * h, x);
        } else {
          x[0] = to_f(orow[ks * M::KSTEP + M::KPL * h]);
        }
#pragma unroll
        for (int k = 0; k < M::KPL; ++k) x[k] *= e;
        dn[ks] = M::from_floats(x);
      }
    }
    __syncthreads();

    // dphi(Q)^T tiles: rows = features of tables (2 ft, 2 ft + 1), columns = queries.
    floatx16 df[NFT];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      df[ft] = zero16();
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks)
        df[ft] = M::mma(M::load(&sm.AF[32 * ft + col][ks * M::KSTEP + M::KPL * h]), dn[ks], df[ft]);
#pragma unroll
      for (int v = 0; v < 16; ++v) df[ft][v] += sm.zr[32 * ft + acc_row(v, h)] * ddq;
    }
    if (causal) {
      for (int kt = 0; kt <= w; ++kt) {
        floatx16 gt = zero16();
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks)
          gt = M::mma(M::load(&sm.VS[32 * kt + col][ks * M::KSTEP + M::KPL * h]), dn[ks], gt);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          gt[v] += ddq;
          if (kt == w && acc_row(v, h) > col) gt[v] = 0.0f;
        }
#pragma unroll
        for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
          const typename M::frag gf = M::from_acc(gt, ks2);
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
            df[ft] = M::mma(M::load_accperm(&sm.KFT[32 * ft + col][32 * kt], ks2, h), gf, df[ft]);
        }
      }
    }
    {
      float dphi[LPG / 2][16], da[LPG / 2][4];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) tile_to_table(df[ft], h, dphi[ft]);
      Fq.backward(dphi, da);
      floatx16 dx[D / 32];
      features_dx<T, D, LPG>(da, RT + (size_t)head * D * pw + 32 * grp, pw, c2, lane, dx);
      if (qvalid)
        finish_row<T, D, true>(dQp, scratch, dQ, bh, slots, qtok, N, levels, causal, h, dx,
                               first != 0, last != 0);
    }
    __syncthreads();

    if (causal) {
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int tix = w + 4 * i;
        if (tix < NST) {
          const int dt = tix % (D / 32), ft = tix / (D / 32);
#pragma unroll
          for (int ks = 0; ks < STEP / M::KSTEP; ++ks) {
            const int k0 = ks * M::KSTEP + M::KPL * h;
            float vb[M::KPL];
#pragma unroll
            for (int k = 0; k < M::KPL; ++k) vb[k] = to_f(sm.VS[k0 + k][32 * dt + col]);
            st[i] = M::mma(M::load(&sm.KFT[32 * ft + col][k0]), M::from_floats(vb), st[i]);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v)
            sm.AF[32 * ft + acc_row(v, h)][32 * dt + col] = from_f<T>(st[i][v]);
        }
      }
      for (int f = tid; f < RP; f += blockDim.x) {
        float zs = 0.0f;
        for (int t = 0; t < STEP; ++t) zs += to_f(sm.KFT[f][t]);
        sm.zr[f] += zs;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Low-rank branch, key side. 64 tokens per step walked from the end of the chunk;
// wave w owns key tile kt = w / 2 and computes dK (w even) or dV (w odd).
template <typename T, int D, int LPG>
struct LbkSmem {
  static constexpr int RP = 16 * LPG, STEP = 64;
  T GF[RP][D + 8];      // running query statistics G = sum phi(Q) dnum^T, [feature][channel]
  T GT[D][RP + 8];      // the same, [channel][feature]
  T QFT[RP][STEP + 8];  // phi(Q) of the step's queries, [feature][query]
  T QF[STEP][RP + 8];   // [query][feature]
  T dnS[STEP][D + 8];   // dnum of the step's queries
  T dnT[D][STEP + 8];
  float gz[RP];         // running sum of phi(Q) dd_lr
  float dd[STEP];
};

template <typename T, int D, int LPG>
__global__ void __launch_bounds__(256)
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
  constexpr int RP = 16 * LPG, STEP = 64, NFT = RP / 32;
  constexpr int NST = NFT * (D / 32), SPW = (NST + 3) / 4;
  __shared__ LbkSmem<T, D, LPG> sm;
  const int bh = blockIdx.y, c = blockIdx.x, head = bh % H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int kt = w >> 1, part = w & 1;
  const int r = 16 * L, f0 = 128 * grp, Lg = min(8, L - 8 * grp);
  const float* pl = planes + ((size_t)head * L + 8 * grp) * 4 * D;
  const int t_beg = c * span, t_end = min(N, t_beg + span);
  const size_t slots = partial_slots(N, levels, causal);
  const float c2 = 2.0f * scale / tau;
  const size_t sidx = causal ? (size_t)bh * (N / span) + c : (size_t)bh;
  const float* Gc = G + sidx * D * r;
  const float* gc = gzs + sidx * r;

  // State tiles (mt, nt): G^T with lanes = features, rows = channels.
  floatx16 st[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    st[i] = zero16();
    const int tix = w + 4 * i;
    if (causal && tix < NST) {
      const int mt = tix / NFT, nt = tix % NFT, f = f0 + 32 * nt + col;
      if (f < r)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[i][v] = Gc[(size_t)(32 * mt + acc_row(v, h)) * r + f];
    }
  }
  for (int idx = tid; idx < RP * D; idx += blockDim.x) {
    const int d = idx / RP, f = idx % RP;
    const T x = from_f<T>(f0 + f < r ? Gc[(size_t)d * r + f0 + f] : 0.0f);
    sm.GT[d][f] = x;
    sm.GF[f][d] = x;
  }
  for (int f = tid; f < RP; f += blockDim.x) sm.gz[f] = f0 + f < r ? gc[f0 + f] : 0.0f;

  const int nstep = (t_end - t_beg + STEP - 1) / STEP;
  for (int si = nstep - 1; si >= 0; --si) {
    const int s0 = t_beg + si * STEP;
    if (w < 2) {
      const int tok = s0 + 32 * w + col;
      const bool valid = tok < t_end;
      Feat Fq;
      Fq.compute(Q + ((size_t)bh * N + (valid ? tok : t_beg)) * D, valid, pl, Lg, scale, tau, lane);
#pragma unroll
      for (int jp = 0; jp < LPG / 2; ++jp) {
        float x[16];
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          x[b] = valid ? Fq.phi[jp][b] : 0.0f;
          sm.QFT[Feat::feat(jp, b, h)][32 * w + col] = from_f<T>(x[b]);
        }
        store8(&sm.QF[32 * w + col][Feat::feat(jp, 0, h)], *reinterpret_cast<float(*)[8]>(&x[0]));
        store8(&sm.QF[32 * w + col][Feat::feat(jp, 8, h)], *reinterpret_cast<float(*)[8]>(&x[8]));
      }
    } else {
      for (int idx = tid - 128; idx < STEP * (D / 8); idx += 128) {
        const int t = idx % STEP, c8 = (idx / STEP) * 8;  // token-fastest transposed stores
        const int tk = s0 + t;
        float x[8];
        if (tk < t_end) {
          const float e = re[(size_t)bh * N + tk];
          load8(dO + ((size_t)bh * N + tk) * D + c8, x);
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] *= e;
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = 0.0f;
        }
        store8(&sm.dnS[t][c8], x);
#pragma unroll
        for (int k = 0; k < 8; ++k) sm.dnT[c8 + k][t] = from_f<T>(x[k]);
      }
      for (int t = tid - 128; t < STEP; t += 128)
        sm.dd[t] = s0 + t < t_end ? rdd[(size_t)bh * N + s0 + t] : 0.0f;
    }
    const int ktok = s0 + 32 * kt + col;
    const bool kvalid = ktok < t_end;
    Feat Fk;
    Fk.compute(K + ((size_t)bh * N + (kvalid ? ktok : t_beg)) * D, kvalid, pl, Lg, scale, tau, lane);
    __syncthreads();

    if (part == 0) {
      // dphi(K)^T tiles: rows = features, columns = keys.
      typename M::frag vf[D / M::KSTEP];
      const T* vrow = V + ((size_t)bh * N + (kvalid ? ktok : t_beg)) * D;
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks)
        vf[ks] = kvalid ? M::load(vrow + ks * M::KSTEP + M::KPL * h) : M::zero();
      floatx16 dkt[NFT];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        dkt[ft] = zero16();
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks)
          dkt[ft] = M::mma(M::load(&sm.GF[32 * ft + col][ks * M::KSTEP + M::KPL * h]), vf[ks], dkt[ft]);
#pragma unroll
        for (int v = 0; v < 16; ++v) dkt[ft][v] += sm.gz[32 * ft + acc_row(v, h)];
      }
      if (causal) {
        for (int qt = kt; qt < STEP / 32; ++qt) {
          floatx16 gm = zero16();
#pragma unroll
          for (int ks = 0; ks < D / M::KSTEP; ++ks)
            gm = M::mma(M::load(&sm.dnS[32 * qt + col][ks * M::KSTEP + M::KPL * h]), vf[ks], gm);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            gm[v] += sm.dd[32 * qt + acc_row(v, h)];
            if (qt == kt && acc_row(v, h) < col) gm[v] = 0.0f;
          }
#pragma unroll
          for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
            const typename M::frag gf = M::from_acc(gm, ks2);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
              dkt[ft] = M::mma(M::load_accperm(&sm.QFT[32 * ft + col][32 * qt], ks2, h), gf, dkt[ft]);
          }
        }
      }
      float dphi[LPG / 2][16], da[LPG / 2][4];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) tile_to_table(dkt[ft], h, dphi[ft]);
      Fk.backward(dphi, da);
      floatx16 dx[D / 32];
      features_dx<T, D, LPG>(da, RT + (size_t)head * D * pw + 32 * grp, pw, c2, lane, dx);
      if (kvalid)
        finish_row<T, D, false>(dKp, scrK, dK, bh, slots, ktok, N, levels, causal, h, dx,
                                first != 0, last != 0);
    } else {
      floatx16 dvt[D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        dvt[dt] = zero16();
#pragma unroll
        for (int ks = 0; ks < RP / M::KSTEP; ++ks)
          dvt[dt] = M::mma(M::load(&sm.GT[32 * dt + col][Feat::frag_feat(ks, 0, h)]), Fk.frag(ks), dvt[dt]);
      }
      if (causal) {
        for (int qt = kt; qt < STEP / 32; ++qt) {
          floatx16 wq = zero16();
#pragma unroll
          for (int ks = 0; ks < RP / M::KSTEP; ++ks)
            wq = M::mma(M::load(&sm.QF[32 * qt + col][Feat::frag_feat(ks, 0, h)]), Fk.frag(ks), wq);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (qt == kt && acc_row(v, h) < col) wq[v] = 0.0f;
#pragma unroll
          for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
            const typename M::frag wf = M::from_acc(wq, ks2);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
              dvt[dt] = M::mma(M::load_accperm(&sm.dnT[32 * dt + col][32 * qt], ks2, h), wf, dvt[dt]);
          }
        }
      }
      if (kvalid)
        finish_row<T, D, false>(dVp, scrV, dV, bh, slots, ktok, N, levels, causal, h, dvt,
                                first != 0, last != 0);
    }
    __syncthreads();

    if (causal) {
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int tix = w + 4 * i;
        if (tix < NST) {
          const int mt = tix / NFT, nt = tix % NFT;
#pragma unroll
          for (int ks = 0; ks < STEP / M::KSTEP; ++ks) {
            const int k0 = ks * M::KSTEP + M::KPL * h;
            st[i] = M::mma(M::load(&sm.dnT[32 * mt + col][k0]), M::load(&sm.QFT[32 * nt + col][k0]), st[i]);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const T x = from_f<T>(st[i][v]);
            sm.GT[32 * mt + acc_row(v, h)][32 * nt + col] = x;
            sm.GF[32 * nt + col][32 * mt + acc_row(v, h)] = x;
          }
        }
      }
      for (int f = tid; f < RP; f += blockDim.x) {
        float s = 0.0f;
        for (int t = 0; t < STEP; ++t) s += to_f(sm.QFT[f][t]) * sm.dd[t];
        sm.gz[f] += s;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------

namespace {

int rt_stride(const Problem& pb);

struct BwdLayout {
  size_t rows, dlam, parts, gsum, gstate, rt, scratch, total;
  int nblk;
};

BwdLayout bwd_layout(const Problem& pb) {
  const size_t BH = (size_t)pb.B * pb.H, N = pb.N, D = pb.d;
  const size_t slots = partial_slots(pb.N, pb.levels, pb.causal);
  const int rpb = 256 / (pb.d / 8);
  BwdLayout l;
  l.nblk = (pb.N + rpb - 1) / rpb;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  l.rows = off; off += al(sizeof(float) * 4 * BH * N);
  l.dlam = off; off += al(sizeof(float) * BH * l.nblk);
  l.parts = off; off += al(3 * BH * slots * D * pb.elem);
  l.gsum = off; off += al(summary_ws_bytes(pb));
  l.gstate = off; off += al(sizeof(float) * BH * pb.nA * (D * pb.r + pb.r));
  l.rt = off; off += al(sizeof(float) * pb.H * D * rt_stride(pb));
  const int groups = padded_tables(pb.L) > 8 ? 2 : 1;
  l.scratch = off; off += groups > 1 ? al(sizeof(float) * 3 * BH * N * D) : 0;
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
  const size_t rpg = 16 * (size_t)(padded_tables(pb.L) > 8 ? 8 : padded_tables(pb.L));
  const size_t sb = e * (2 * kt * (d + 24)) + 20 * kt;  // one-role launch (two tiles)
  const size_t lq = e * (rpg * (d + 8) + rpg * 136 + 128 * (d + 8)) + 4 * rpg;
  const size_t lk = e * (2 * rpg * (d + 8) + rpg * 72 + 64 * (rpg + 8) + 64 * (d + 8) + d * 72) +
                    4 * rpg + 4 * 64;
  size_t m = sb > lq ? sb : lq;
  return lk > m ? lk : m;
}

void launch_bwd(const Problem& pb, const void* Q, const void* K, const void* V, const void* dO,
                const void* O_s, const void* O_lr, const float* planes_lr, const int32_t* qperm,
                const int32_t* kperm, const float* A, const float* z, const float* lse,
                const float* d_lr, const float* lambda, const float* g_s, const float* g_lr,
                void* dQ, void* dK, void* dV, float* dlambda, float* dg_s, float* dg_lr, void* ws,
                hipStream_t st) {
  const BwdLayout lay = bwd_layout(pb);
  char* base = (char*)ws;
  const size_t BH = (size_t)pb.B * pb.H, N = pb.N;
  float* rc = (float*)(base + lay.rows);
  float* rD = rc + BH * N;
  float* re = rD + BH * N;
  float* rdd = re + BH * N;
  float* dlam_part = (float*)(base + lay.dlam);
  const size_t slots = partial_slots(pb.N, pb.levels, pb.causal);
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
  const int items = pb.causal ? pb.levels * (pb.N / 2) / pb.s + pb.N / pb.s : pb.N / pb.s;
  const int span = pb.causal ? pb.chunk : 128;
  const int span_k = pb.causal ? pb.chunk : 64;

  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      ELSAA_LAUNCH("planes_t", planes_transpose_kernel, dim3(pb.H), dim3(256), 0, st, planes_lr,
                   pb.L, pb.d, pw, RT);
      ELSAA_LAUNCH("bwd_rows", (bwd_rows_kernel<T, D>), dim3(lay.nblk, BH), dim3(256), 0, st,
                         (const T*)dO, (const T*)O_s, (const T*)O_lr, lse, d_lr, lambda, g_s,
                         g_lr, pb.eps, pb.H, pb.N, rc, rD, re, rdd, dg_s, dg_lr, dlam_part);
      if (dlambda)
        ELSAA_LAUNCH("dlam_reduce", dlam_reduce_kernel, dim3(pb.H), dim3(256), 0, st, dlam_part,
                           pb.B, pb.H, lay.nblk, dlambda);
      run_lr_sums(pb, Q, dO, re, rdd, planes_lr, S, Z, st);
      run_lr_scan(pb, S, Z, pb.causal ? 2 : 0, Gs, gzs, st);
      auto run_sparse = [&](auto sc) {
        constexpr int SB = ELSAA_C(sc);
        const dim3 grid(items, BH);
        if constexpr (sizeof(SbwdSmem<T, D, SB, 3>) <= kLdsBytes && SB <= 128) {
          ELSAA_LAUNCH("sparse_bwd", (sparse_bwd_kernel<T, D, SB, 3>), grid,
                       dim3(sbwd_threads<SB>(3)), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                       (const T*)dO, lse, rc, rD, qperm, kperm, pb.N, (int)pb.causal, pb.levels,
                       pb.scale, (T*)dQp, (T*)dKp, (T*)dVp);
        } else if constexpr (sizeof(SbwdSmem<T, D, SB, 1>) <= kLdsBytes) {
          ELSAA_LAUNCH("sparse_bwd", (sparse_bwd_kernel<T, D, SB, 1>), grid,
                       dim3(sbwd_threads<SB>(1)), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                       (const T*)dO, lse, rc, rD, qperm, kperm, pb.N, (int)pb.causal, pb.levels,
                       pb.scale, (T*)dQp, (T*)dKp, (T*)dVp);
          ELSAA_LAUNCH("sparse_bwd_q", (sparse_bwd_kernel<T, D, SB, 2>), grid,
                       dim3(sbwd_threads<SB>(2)), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                       (const T*)dO, lse, rc, rD, qperm, kperm, pb.N, (int)pb.causal, pb.levels,
                       pb.scale, (T*)dQp, (T*)dKp, (T*)dVp);
        }
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
        for (int g = 0; g < groups; ++g) {
          const int first = g == 0, last = g == groups - 1;
          if constexpr (sizeof(LbqSmem<T, D, LPG>) <= kLdsBytes)
            ELSAA_LAUNCH("lr_bwd_q", (lr_bwd_q_kernel<T, D, LPG>),
                               dim3((pb.N + span - 1) / span, BH), dim3(256), 0, st, (const T*)Q,
                               (const T*)K, (const T*)V, (const T*)dO, planes_lr, A, z, re, rdd,
                               (const T*)dQp, scrQ, (T*)dQ, RT, pw, pb.H, pb.N, pb.L, span, pb.levels,
                               (int)pb.causal, pb.scale, pb.tau, g, first, last);
          if constexpr (sizeof(LbkSmem<T, D, LPG>) <= kLdsBytes)
            ELSAA_LAUNCH("lr_bwd_k", (lr_bwd_k_kernel<T, D, LPG>),
                               dim3((pb.N + span_k - 1) / span_k, BH), dim3(256), 0, st,
                               (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, planes_lr, Gs,
                               gzs, re, rdd, (const T*)dKp, (const T*)dVp, scrK, scrV, (T*)dK,
                               (T*)dV, RT, pw, pb.H, pb.N, pb.L, span_k, pb.levels, (int)pb.causal,
                               pb.scale, pb.tau, g, first, last);
        }
      };
      switch (padded_tables(pb.L)) {
        case 2: run_lr(std::integral_constant<int, 2>{}); break;
        case 4: run_lr(std::integral_constant<int, 4>{}); break;
        default: run_lr(std::integral_constant<int, 8>{}); break;
      }
    });
  });
}

}  // namespace elsaa
