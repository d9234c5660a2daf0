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
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[dt][g][e] += to_f(src[32 * dt + 8 * g + 4 * h + e]);
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
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[dt][g][e] = first ? 0.0f : scratch[row + 32 * dt + 8 * g + 4 * h + e];
  if (first) sum_partials<T, D, QUERY>(part, bh, slots, tok, N, levels, causal, h, acc);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[dt][g][e] + lr[dt][4 * g + e];
        const size_t o = row + 32 * dt + 8 * g + 4 * h + e;
        if (last) out[o] = from_f<T>(v);
        else scratch[o] = v;
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

__global__ void dlam_reduce_kernel(const float* __restrict__ part, int B, int H, int nblk,
                                   float* __restrict__ dlambda) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float s = 0.0f;
  for (int b = 0; b < B; ++b)
    for (int k = 0; k < nblk; ++k) s += part[((size_t)b * H + h) * nblk + k];
  dlambda[h] = s;
}

// ---------------------------------------------------------------------------
// Sparse branch, one workgroup per selected block. Wave w owns keys
// [32 w, 32 w + 32) of the block (their K and V rows stay in registers) and
// accumulates their dK^T, dV^T over the block's query tiles. Per query tile,
// S = Q K^T and dP = (c dO) V^T put the wave's keys in lanes, so P and dS are
// directly the B operands of dV^T += (c dO)^T P and dK^T += Q^T dS; dS goes to LDS
// and dQ = dS K is formed after a barrier from all keys of the block.
template <typename T, int D, int SB>
struct SbwdSmem {
  static constexpr int KT = SB < 32 ? 32 : SB;
  T Kt[D][KT + 8];
  T Qs[32][D + 8];
  T QsT[D][40];
  T dOs[32][D + 8];
  T dOsT[D][40];
  T dSs[32][KT + 8];
  float lse[32], Dd[32];
  int kidx[KT], qidx[KT];
};

template <typename T, int D, int SB>
__global__ void __launch_bounds__(64 * (SB < 32 ? 1 : SB / 32))
    sparse_bwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                      const T* __restrict__ dO, const float* __restrict__ lse,
                      const float* __restrict__ rc, const float* __restrict__ rD,
                      const int32_t* __restrict__ qperm, const int32_t* __restrict__ kperm, int N,
                      int causal, int levels, float scale, T* __restrict__ dQp,
                      T* __restrict__ dKp, T* __restrict__ dVp) {
  typedef MF<T> M;
  constexpr int KT = SB < 32 ? 32 : SB, NW = KT / 32;
  __shared__ SbwdSmem<T, D, SB> sm;
  const int bh = blockIdx.y, item = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const size_t P = perm_stride(N, levels, causal);
  const size_t slots = partial_slots(N, levels, causal);

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
  for (int t = tid; t < KT; t += blockDim.x) {
    sm.kidx[t] = t < SB ? (leaf ? tok0 + t : ksrc[t]) : -1;
    sm.qidx[t] = t < SB ? (leaf ? tok0 + t : qsrc[t]) : -1;
  }
  __syncthreads();
  for (int idx = tid; idx < KT * (D / 8); idx += blockDim.x) {
    const int t = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    const int j = sm.kidx[t];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sm.Kt[c8 + e][t] = j >= 0 ? K[((size_t)bh * N + j) * D + c8 + e] : from_f<T>(0.0f);
  }
  const int key = 32 * w + col;
  const int jk = sm.kidx[key];
  const bool kvalid = jk >= 0;
  typename M::frag kf[D / M::KSTEP], vf[D / M::KSTEP];
#pragma unroll
  for (int ks = 0; ks < D / M::KSTEP; ++ks) {
    const size_t o = ((size_t)bh * N + (kvalid ? jk : 0)) * D + ks * M::KSTEP + M::KPL * h;
    kf[ks] = kvalid ? M::load(K + o) : M::zero();
    vf[ks] = kvalid ? M::load(V + o) : M::zero();
  }
  floatx16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) { dk[dt] = zero16(); dv[dt] = zero16(); }

  for (int qt = 0; qt < KT / 32; ++qt) {
    __syncthreads();
    for (int idx = tid; idx < 32 * (D / 8); idx += blockDim.x) {
      const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
      const int i = sm.qidx[32 * qt + r];
      float qv[8], ov[8];
      if (i >= 0) {
        const size_t o = ((size_t)bh * N + i) * D + c8;
        const float c = rc[(size_t)bh * N + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) { qv[e] = to_f(Q[o + e]); ov[e] = c * to_f(dO[o + e]); }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { qv[e] = 0.0f; ov[e] = 0.0f; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const T a = from_f<T>(qv[e]), b = from_f<T>(ov[e]);
        sm.Qs[r][c8 + e] = a;
        sm.QsT[c8 + e][r] = a;
        sm.dOs[r][c8 + e] = b;
        sm.dOsT[c8 + e][r] = b;
      }
    }
    if (tid < 32) {
      const int i = sm.qidx[32 * qt + tid];
      sm.lse[tid] = i >= 0 ? lse[(size_t)bh * N + i] : 0.0f;
      sm.Dd[tid] = i >= 0 ? rD[(size_t)bh * N + i] : 0.0f;
    }
    __syncthreads();
    if (!(leaf && qt < w)) {
      floatx16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks) {
        const int k0 = ks * M::KSTEP + M::KPL * h;
        s = M::mma(M::load(&sm.Qs[col][k0]), kf[ks], s);
        dp = M::mma(M::load(&sm.dOs[col][k0]), vf[ks], dp);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int qr = acc_row(v, h), qloc = 32 * qt + qr;
        const bool ok = kvalid && sm.qidx[qloc] >= 0 && !(leaf && key > qloc);
        const float p = ok ? fast_exp(s[v] * scale - sm.lse[qr]) : 0.0f;
        s[v] = p;
        dp[v] = p * (dp[v] - sm.Dd[qr]);
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
        const typename M::frag pf = M::from_acc(s, ks2), sf = M::from_acc(dp, ks2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          dv[dt] = M::mma(M::load_accperm(&sm.dOsT[32 * dt + col][0], ks2, h), pf, dv[dt]);
          dk[dt] = M::mma(M::load_accperm(&sm.QsT[32 * dt + col][0], ks2, h), sf, dk[dt]);
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) sm.dSs[acc_row(v, h)][key] = from_f<T>(dp[v]);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) sm.dSs[acc_row(v, h)][key] = from_f<T>(0.0f);
    }
    __syncthreads();
    for (int dt = w; dt < D / 32; dt += NW) {
      floatx16 acc = zero16();
      for (int ks = 0; ks < KT / M::KSTEP; ++ks) {
        const int k0 = ks * M::KSTEP + M::KPL * h;
        acc = M::mma(M::load(&sm.dSs[col][k0]), M::load(&sm.Kt[32 * dt + col][k0]), acc);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = sm.qidx[32 * qt + acc_row(v, h)];
        if (i >= 0) {
          const size_t sl = lev >= 0 ? (size_t)N + (size_t)lev * (N / 2) + compact_future_b(i, N, lev)
                                     : (size_t)i;
          dQp[((size_t)bh * slots + sl) * D + 32 * dt + col] = from_f<T>(acc[v] * scale);
        }
      }
    }
  }
  if (kvalid) {
    const size_t sl = lev >= 0 ? (size_t)N + (size_t)lev * (N / 2) + compact_past(jk, N, lev)
                               : (size_t)jk;
    T* kd = dKp + ((size_t)bh * slots + sl) * D;
    T* vd = dVp + ((size_t)bh * slots + sl) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int d = 32 * dt + acc_row(v, h);
        kd[d] = from_f<T>(dk[dt][v] * scale);
        vd[d] = from_f<T>(dv[dt][v]);
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
                    int H, int N, int L, int span, int levels, int causal, float scale, float tau,
                    int grp, int first, int last) {
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
    const int f = idx / D, d = idx % D;
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
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sm.VS[t][c8 + e] = tk < t_end ? V[((size_t)bh * N + tk) * D + c8 + e] : from_f<T>(0.0f);
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
#pragma unroll
        for (int k = 0; k < M::KPL; ++k) x[k] = e * to_f(orow[ks * M::KSTEP + M::KPL * h + k]);
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
      features_dx<T, D, LPG>(da, pl, Lg, c2, lane, dx);
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
                    float* __restrict__ scrV, T* __restrict__ dK, T* __restrict__ dV, int H, int N,
                    int L, int span, int levels, int causal, float scale, float tau, int grp,
                    int first, int last) {
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
      for (int jp = 0; jp < LPG / 2; ++jp)
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const int f = Feat::feat(jp, b, h);
          const T x = from_f<T>(valid ? Fq.phi[jp][b] : 0.0f);
          sm.QFT[f][32 * w + col] = x;
          sm.QF[32 * w + col][f] = x;
        }
    } else {
      for (int idx = tid - 128; idx < STEP * (D / 8); idx += 128) {
        const int t = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
        const int tk = s0 + t;
        const float e = tk < t_end ? re[(size_t)bh * N + tk] : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const T x = from_f<T>(tk < t_end ? e * to_f(dO[((size_t)bh * N + tk) * D + c8 + k]) : 0.0f);
          sm.dnS[t][c8 + k] = x;
          sm.dnT[c8 + k][t] = x;
        }
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
      features_dx<T, D, LPG>(da, pl, Lg, c2, lane, dx);
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

struct BwdLayout {
  size_t rows, dlam, parts, gsum, gstate, scratch, total;
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
  const int groups = padded_tables(pb.L) > 8 ? 2 : 1;
  l.scratch = off; off += groups > 1 ? al(sizeof(float) * 3 * BH * N * D) : 0;
  l.total = off;
  return l;
}

template <typename T, int D, int SB>
constexpr size_t sbwd_lds() { return sizeof(SbwdSmem<T, D, SB>); }

}  // namespace

size_t bwd_ws_bytes(const Problem& pb) { return bwd_layout(pb).total; }

size_t bwd_lds_need(const Problem& pb) {
  const size_t e = pb.elem, d = pb.d, kt = pb.s < 32 ? 32 : pb.s;
  const size_t rpg = 16 * (size_t)(padded_tables(pb.L) > 8 ? 8 : padded_tables(pb.L));
  const size_t sb = e * (d * (kt + 8) + 2 * 32 * (d + 8) + 2 * d * 40 + 32 * (kt + 8)) + 8 * 32 + 8 * kt;
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
      ELSAA_LAUNCH("bwd_rows", (bwd_rows_kernel<T, D>), dim3(lay.nblk, BH), dim3(256), 0, st,
                         (const T*)dO, (const T*)O_s, (const T*)O_lr, lse, d_lr, lambda, g_s,
                         g_lr, pb.eps, pb.H, pb.N, rc, rD, re, rdd, dg_s, dg_lr, dlam_part);
      if (dlambda)
        ELSAA_LAUNCH("dlam_reduce", dlam_reduce_kernel, dim3((pb.H + 63) / 64), dim3(64), 0, st, dlam_part,
                           pb.B, pb.H, lay.nblk, dlambda);
      run_lr_sums(pb, Q, dO, re, rdd, planes_lr, S, Z, st);
      run_lr_scan(pb, S, Z, pb.causal ? 2 : 0, Gs, gzs, st);
      auto run_sparse = [&](auto sc) {
        constexpr int SB = ELSAA_C(sc);
        if constexpr (sbwd_lds<T, D, SB>() <= kLdsBytes)
          ELSAA_LAUNCH("sparse_bwd", (sparse_bwd_kernel<T, D, SB>), dim3(items, BH),
                             dim3(64 * (SB < 32 ? 1 : SB / 32)), 0, st, (const T*)Q,
                             (const T*)K, (const T*)V, (const T*)dO, lse, rc, rD, qperm, kperm,
                             pb.N, (int)pb.causal, pb.levels, pb.scale, (T*)dQp, (T*)dKp,
                             (T*)dVp);
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
                               (const T*)dQp, scrQ, (T*)dQ, pb.H, pb.N, pb.L, span, pb.levels,
                               (int)pb.causal, pb.scale, pb.tau, g, first, last);
          if constexpr (sizeof(LbkSmem<T, D, LPG>) <= kLdsBytes)
            ELSAA_LAUNCH("lr_bwd_k", (lr_bwd_k_kernel<T, D, LPG>),
                               dim3((pb.N + span_k - 1) / span_k, BH), dim3(256), 0, st,
                               (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, planes_lr, Gs,
                               gzs, re, rdd, (const T*)dKp, (const T*)dVp, scrK, scrV, (T*)dK,
                               (T*)dV, pb.H, pb.N, pb.L, span_k, pb.levels, (int)pb.causal,
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
