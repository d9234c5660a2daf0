// fwd.hip -- forward of the ELSAA operator on gfx950.
//
// sparse_fwd_kernel (ELSAA paper, Section 3.2): one workgroup per selected block.
// The block's s keys are gathered by the sorted order into LDS (K row-major, V
// transposed); each wave owns 32 of the block's queries and streams the keys in
// tiles of 32 with an online softmax. Scores are formed as S^T = K Q^T so that a
// lane owns one query (column statistics stay in-lane) and the probabilities P^T
// are directly the B operand of O^T += V^T P^T. The normalized block output and
// its log-sum-exp go to a partial slot of the query:
//   causal: leaf blocks (dense causal segments of s tokens) -> slot i,
//           level l block   -> slot N + l N/2 + compact_l(i);
//   non-causal: the single block of query i -> slot i.
//
// fwd_epilogue_kernel: per head and chunk of tokens, 64 tokens per step:
//   - sparse branch: log-sum-exp merge of the query's partials (Section 3.2's
//     merge that keeps exact softmax normalization over the union support);
//   - low-rank branch (Section 3.1): normalized ratio readout of the running
//     bucket statistics (inter-chunk part, exclusive of the step) plus the causally
//     masked intra-step part, then the statistics are advanced by the step's keys
//     on chip;
//   - fusion: Eq. 5 m_i = d_s / (d_s + lambda d_lr + eps) evaluated as
//     1 / (1 + exp(log(lambda d_lr + eps) - lse)), then Eq. 4.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

// Compact index of query i within level l's future halves (i must be in one).
__device__ __forceinline__ int compact_future(int i, int N, int l) {
  const int n = N >> l, half = n >> 1;
  return (i / n) * half + (i % n) - half;
}

template <typename T, int D, int SB>
constexpr size_t sparse_fwd_lds() {
  constexpr int KT = SB < 32 ? 32 : SB;
  return sizeof(T) * 2 * (size_t)KT * tile_ld<T>(D) + sizeof(int) * KT;
}

template <typename T, int D, int SB>
__global__ void __launch_bounds__(64 * (SB < 32 ? 1 : SB / 32))
    sparse_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                      const int32_t* __restrict__ qperm, const int32_t* __restrict__ kperm, int N,
                      int causal, int levels, float scale, T* __restrict__ Opart,
                      float* __restrict__ Lpart) {
  typedef MF<T> M;
  constexpr int KT = SB < 32 ? 32 : SB;  // key rows held in LDS
  constexpr int LD = tile_ld<T>(D);        // row stride (elements) of the LDS tiles
  __shared__ T Ks[KT][LD];
  __shared__ T Vs[KT][LD];
  __shared__ int kidx[KT];

  const int bh = blockIdx.y, item = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const size_t P = perm_stride(N, levels, causal);
  const size_t slots = partial_slots(N, levels, causal);

  // Decode the work item.
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

  for (int t = tid; t < KT; t += blockDim.x)
    kidx[t] = t < SB ? (leaf ? tok0 + t : ksrc[t]) : -1;
  __syncthreads();
  // Gather the block's K and V rows into LDS (row-major, 16-byte row-contiguous
  // copies, all loads in flight together); rows past the block are zero.
  {
    T* const dst[2] = {&Ks[0][0], &Vs[0][0]};
    const T* const src[2] = {K, V};
    const float* const sc[2] = {nullptr, nullptr};
    gather_rows<T, D, KT, 64 * (SB < 32 ? 1 : SB / 32), 2>(dst, LD, src, sc, kidx, (size_t)bh * N, tid);
  }

  // This wave's queries (one per lane column).
  const int qloc = 32 * w + col;
  const bool qvalid = qloc < SB;
  const int qi = qvalid ? (leaf ? tok0 + qloc : qsrc[qloc]) : 0;
  typename M::frag qf[D / M::KSTEP];
  {
    const T* qr = Q + ((size_t)bh * N + qi) * D;
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks)
      qf[ks] = qvalid ? M::load(qr + ks * M::KSTEP + M::KPL * h) : M::zero();
  }
  __syncthreads();

  floatx16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
  float mrun = -INFINITY, lrun = 0.0f;
  const int nkt = leaf ? (w + 1) : KT / 32;  // causal leaf: key tiles up to the diagonal
  for (int kt = 0; kt < nkt; ++kt) {
    floatx16 sacc = zero16();
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks)
      sacc = M::mma(row_frag<T>(&Ks[0][0], LD, 32 * kt, 0, ks, lane), qf[ks], sacc);
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kr = 32 * kt + acc_row(v, h);
      const bool masked = kr >= SB || (leaf && kr > qloc);
      sacc[v] = masked ? -INFINITY : sacc[v] * scale;
      mx = fmaxf(mx, sacc[v]);
    }
    mx = fmaxf(mx, swap_half(mx));
    const float mnew = fmaxf(mrun, mx);
    const float msub = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = fast_exp(mrun - msub);
    float ps = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sacc[v] = fast_exp(sacc[v] - msub);
      ps += sacc[v];
    }
    ps += swap_half(ps);
    lrun = lrun * alpha + ps;
    mrun = mnew;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
#pragma unroll
    for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
      const typename M::frag pf = M::from_acc(sacc, ks2);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = M::mma(tr_frag<T>(&Vs[0][0], LD, 32 * kt, 32 * dt, ks2, lane, true), pf, o[dt]);
    }
  }

  if (qvalid) {
    const float inv = 1.0f / lrun;
    const size_t slot = lev >= 0 ? (size_t)N + (size_t)lev * (N / 2) + compact_future(qi, N, lev)
                                 : (size_t)qi;
    T* dst = Opart + ((size_t)bh * slots + slot) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = o[dt][4 * g + e] * inv;
        store4(dst + 32 * dt + 8 * g + 4 * h, x);
      }
    if (h == 0) Lpart[(size_t)bh * slots + slot] = mrun + __logf(lrun);
  }
}

// ---------------------------------------------------------------------------

template <typename T, int D, int LP>
struct EpiSmem {
  static constexpr int RP = 16 * LP, STEP = 64;
  T VT[D][STEP + 8];     // V^T of the step's keys
  T KF[STEP][RP + 8];    // phi(K) of the step's keys, [key][feature]
  T AT[D][RP + 8];       // running statistics (value channel x feature) as MFMA operand
  float zr[RP];          // running sum of phi(K)
};

template <typename T, int D, int LP>
__global__ void __launch_bounds__(256)
    fwd_epilogue_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                        const float* __restrict__ planes, const float* __restrict__ A,
                        const float* __restrict__ z, const T* __restrict__ Opart,
                        const float* __restrict__ Lpart, const float* __restrict__ lambda,
                        const float* __restrict__ gs, const float* __restrict__ glr,
                        T* __restrict__ O, T* __restrict__ Os, T* __restrict__ Olr,
                        float* __restrict__ lse_out, float* __restrict__ dlr_out, int H, int N,
                        int L, int span, int levels, int causal, int s, float scale, float tau,
                        float eps) {
  typedef MF<T> M;
  typedef Features<T, D, LP> Feat;
  constexpr int RP = 16 * LP, STEP = 64;
  constexpr int NT_N = RP / 32, NST = (D / 32) * NT_N, SPW = (NST + 3) / 4;
  constexpr int DH = D / 2;                     // output rows per wave
  constexpr int NDT = DH >= 32 ? DH / 32 : 1;   // 32-row output tiles per wave
  __shared__ EpiSmem<T, D, LP> sm;

  const int bh = blockIdx.y, c = blockIdx.x, head = bh % H;
  const int r = 16 * L;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int qt = w >> 1, dh = w & 1;
  // D = 32: one 32-row tile; both waves of a query tile compute it, only dh == 0 writes.
  const int dbase = D >= 64 ? dh * DH : 0;
  const bool writer = D >= 64 || dh == 0;
  const float* pl = planes + (size_t)head * L * 4 * D;
  const int t_beg = c * span, t_end = min(N, t_beg + span);
  const size_t slots = partial_slots(N, levels, causal);
  const float lam = lambda[head];
  const int logN = 31 - __clz(N);

  // Load the statistics at the start of this span.
  const float* Ac = A + (size_t)(causal ? (size_t)bh * (N / span) + c : bh) * D * r;
  const float* zc = z + (size_t)(causal ? (size_t)bh * (N / span) + c : bh) * r;
  floatx16 st[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    st[i] = zero16();
    const int tix = w + 4 * i;
    if (causal && tix < NST) {
      const int mt = tix / NT_N, nt = tix % NT_N, f = 32 * nt + col;
      if (f < r)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[i][v] = Ac[(size_t)(32 * mt + acc_row(v, h)) * r + f];
    }
  }
  for (int idx = tid; idx < D * RP; idx += blockDim.x) {
    const int e = idx / RP, f = idx % RP;
    sm.AT[e][f] = from_f<T>(f < r ? Ac[(size_t)e * r + f] : 0.0f);
  }
  for (int f = tid; f < RP; f += blockDim.x) sm.zr[f] = f < r ? zc[f] : 0.0f;

  for (int s0 = t_beg; s0 < t_end; s0 += STEP) {
    // phase A: phi(K) of the step's keys and V^T into LDS (causal only); phi(Q) in
    // registers for this wave's query tile.
    if (causal) {
      if (dh == 0) {
        const int tok = s0 + 32 * qt + col;
        const bool valid = tok < t_end;
        Feat Fk;
        Fk.compute(K + ((size_t)bh * N + (valid ? tok : t_beg)) * D, valid, pl, L, scale, tau, lane);
#pragma unroll
        for (int jp = 0; jp < LP / 2; ++jp)
#pragma unroll
          for (int b = 0; b < 16; ++b)
            sm.KF[32 * qt + col][Feat::feat(jp, b, h)] = from_f<T>(valid ? Fk.phi[jp][b] : 0.0f);
      } else {
        for (int idx = lane + 64 * qt; idx < STEP * (D / 8); idx += 128) {
          const int tk = idx % STEP, c8 = (idx / STEP) * 8;  // token-fastest V^T stores
          const int tok = s0 + tk;
          float x[8];
          if (tok < t_end) {
            load8(V + ((size_t)bh * N + tok) * D + c8, x);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.0f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.VT[c8 + e][tk] = from_f<T>(x[e]);
        }
      }
    }
    const int qtok = s0 + 32 * qt + col;
    const bool qvalid = qtok < t_end;
    Feat Fq;
    Fq.compute(Q + ((size_t)bh * N + (qvalid ? qtok : t_beg)) * D, qvalid, pl, L, scale, tau, lane);
    __syncthreads();

    // phase B: readout. num^T rows [dbase, dbase + 32 NDT) x this wave's 32 queries.
    floatx16 num[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) num[dt] = zero16();
    float den = 0.0f;
#pragma unroll
    for (int jp = 0; jp < LP / 2; ++jp)
#pragma unroll
      for (int b = 0; b < 16; ++b) den += Fq.phi[jp][b] * sm.zr[Feat::feat(jp, b, h)];
    den += swap_half(den);
#pragma unroll
    for (int ks = 0; ks < RP / M::KSTEP; ++ks) {
      const typename M::frag fb = Fq.frag(ks);
      const int f0 = Feat::frag_feat(ks, 0, h);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        num[dt] = M::mma(M::load(&sm.AT[dbase + 32 * dt + col][f0]), fb, num[dt]);
    }
    if (causal) {
      float dintra = 0.0f;
      for (int kt = 0; kt <= qt; ++kt) {
        floatx16 wt = zero16();
#pragma unroll
        for (int ks = 0; ks < RP / M::KSTEP; ++ks)
          wt = M::mma(M::load(&sm.KF[32 * kt + col][Feat::frag_feat(ks, 0, h)]), Fq.frag(ks), wt);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (kt == qt && acc_row(v, h) > col) wt[v] = 0.0f;
          dintra += wt[v];
        }
#pragma unroll
        for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
          const typename M::frag wf = M::from_acc(wt, ks2);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            num[dt] = M::mma(M::load_accperm(&sm.VT[dbase + 32 * dt + col][32 * kt], ks2, h), wf, num[dt]);
        }
      }
      den += dintra + swap_half(dintra);
    }
    __syncthreads();

    // phase C: advance the running statistics by the step's keys.
    if (causal) {
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int tix = w + 4 * i;
        if (tix < NST) {
          const int mt = tix / NT_N, nt = tix % NT_N;
#pragma unroll
          for (int ks = 0; ks < STEP / M::KSTEP; ++ks) {
            const int k0 = ks * M::KSTEP + M::KPL * h;
            float kb[M::KPL];
#pragma unroll
            for (int e = 0; e < M::KPL; ++e) kb[e] = to_f(sm.KF[k0 + e][32 * nt + col]);
            st[i] = M::mma(M::load(&sm.VT[32 * mt + col][k0]), M::from_floats(kb), st[i]);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) sm.AT[32 * mt + acc_row(v, h)][32 * nt + col] = from_f<T>(st[i][v]);
        }
      }
      for (int f = tid; f < RP; f += blockDim.x) {
        float zs = 0.0f;
        for (int t = 0; t < STEP; ++t) zs += to_f(sm.KF[t][f]);
        sm.zr[f] += zs;
      }
    }

    // phase D: sparse merge, fusion, outputs for this wave's queries and rows.
    if (qvalid) {
      const int i = qtok;
      const float* lp = Lpart + (size_t)bh * slots;
      auto slot_of = [&](int l) -> size_t {
        return (size_t)N + (size_t)l * (N / 2) + compact_future(i, N, l);
      };
      auto in_level = [&](int l) -> bool { return causal && ((i >> (logN - 1 - l)) & 1); };
      float lmax = lp[i];
      for (int l = 0; l < levels; ++l)
        if (in_level(l)) lmax = fmaxf(lmax, lp[slot_of(l)]);
      float wsum = fast_exp(lp[i] - lmax);
      for (int l = 0; l < levels; ++l)
        if (in_level(l)) wsum += fast_exp(lp[slot_of(l)] - lmax);
      const float lse = lmax + __logf(wsum);
      const float winv = 1.0f / wsum;
      float os[NDT][4][4];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) os[dt][g][e] = 0.0f;
      for (int l = -1; l < levels; ++l) {
        if (l >= 0 && !in_level(l)) continue;
        const size_t sl = l < 0 ? (size_t)i : slot_of(l);
        const float wk = fast_exp(lp[sl] - lmax) * winv;
        const T* src = Opart + ((size_t)bh * slots + sl) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float x[4];
            load4(src + dbase + 32 * dt + 8 * g + 4 * h, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) os[dt][g][e] += wk * x[e];
          }
      }
      const float m = 1.0f / (1.0f + fast_exp(__logf(lam * den + eps) - lse));
      const float g1 = gs ? gs[(size_t)bh * N + i] : 1.0f;
      const float g2 = glr ? glr[(size_t)bh * N + i] : 1.0f;
      const float dinv = 1.0f / den;
      const size_t row = ((size_t)bh * N + i) * D;
      if (writer) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dd = dbase + 32 * dt + 8 * g + 4 * h;
            float xo[4], xl[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              xl[e] = num[dt][4 * g + e] * dinv;
              xo[e] = g1 * m * os[dt][g][e] + g2 * xl[e];
            }
            store4(O + row + dd, xo);
            store4(Os + row + dd, os[dt][g]);
            store4(Olr + row + dd, xl);
          }
        if (h == 0 && dh == 0) {
          lse_out[(size_t)bh * N + i] = lse;
          dlr_out[(size_t)bh * N + i] = den;
        }
      }
    }
    __syncthreads();
  }
}

size_t fwd_ws_bytes(const Problem& pb) {
  const size_t slots = partial_slots(pb.N, pb.levels, pb.causal);
  return (size_t)pb.B * pb.H * slots * ((size_t)pb.d * pb.elem + sizeof(float)) + 256;
}

void launch_fwd(const Problem& pb, const void* Q, const void* K, const void* V,
                const float* planes_lr, const int32_t* qperm, const int32_t* kperm,
                const float* A, const float* z, const float* lambda, const float* g_s,
                const float* g_lr, void* O, void* O_s, void* O_lr, float* lse, float* d_lr,
                void* ws, hipStream_t st) {
  const int BH = pb.B * pb.H;
  const size_t slots = partial_slots(pb.N, pb.levels, pb.causal);
  float* Lpart = (float*)ws;
  void* Opart = (char*)ws + (((size_t)BH * slots * sizeof(float) + 255) & ~(size_t)255);
  const int items = pb.causal ? pb.levels * (pb.N / 2) / pb.s + pb.N / pb.s : pb.N / pb.s;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      auto run = [&](auto sc) {
        constexpr int SB = ELSAA_C(sc);
        if constexpr (sparse_fwd_lds<T, D, SB>() <= kLdsBytes)
        ELSAA_LAUNCH("sparse_fwd", (sparse_fwd_kernel<T, D, SB>), dim3(items, BH),
                           dim3(64 * (SB < 32 ? 1 : SB / 32)), 0, st, (const T*)Q, (const T*)K,
                           (const T*)V, qperm, kperm, pb.N, (int)pb.causal, pb.levels, pb.scale,
                           (T*)Opart, Lpart);
      };
      switch (pb.s) {
        case 16: run(std::integral_constant<int, 16>{}); break;
        case 32: run(std::integral_constant<int, 32>{}); break;
        case 64: run(std::integral_constant<int, 64>{}); break;
        case 128: run(std::integral_constant<int, 128>{}); break;
        default: run(std::integral_constant<int, 256>{}); break;
      }
      with_LP(pb.L, [&](auto lc) {
        constexpr int LP = ELSAA_C(lc);
        const int span = pb.causal ? pb.chunk : 64;
        const int nspan = (pb.N + span - 1) / span;
        if constexpr (sizeof(EpiSmem<T, D, LP>) <= kLdsBytes)
        ELSAA_LAUNCH("fwd_epilogue", (fwd_epilogue_kernel<T, D, LP>), dim3(nspan, BH), dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, planes_lr, A, z,
                           (const T*)Opart, Lpart, lambda, g_s, g_lr, (T*)O, (T*)O_s, (T*)O_lr,
                           lse, d_lr, pb.H, pb.N, pb.L, span, pb.levels, (int)pb.causal, pb.s,
                           pb.scale, pb.tau, pb.eps);
      });
    });
  });
}

}  // namespace elsaa
