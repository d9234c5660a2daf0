// fused.hip -- the whole non-causal forward of the ELSAA operator in one launch
// (the paper's Section 8 names fused GPU kernels as the next step; this is that
// fusion for the non-causal operator, where a head's work has no dependency on
// any other head's).
//
// One workgroup of 4 waves per (batch, head) runs, with workgroup barriers
// between them:
//   1. sortLSH codes of the head's queries and keys (Section 3.2): the sign of
//      the fp64 fused-multiply-add chain of each row against each hyperplane, in
//      index order from +0.0, as the two-launch selection forms them;
//   2. stable counting sort of each side by the Gray rank of its code (ties to the
//      lower token index), two waves, one per side;
//   3. the RACE summary (Section 3.1): A = sum_j phi(K_j) V_j^T and z = sum_j
//      phi(K_j) over the head's keys, 128 keys per step on MFMA; the statistics
//      stay in LDS as the readout's operand;
//   4. the selected blocks (Section 3.2): each block's keys and values gathered by
//      the sorted order into LDS, exact softmax block attention with an online
//      softmax, and, from the same query rows already in registers, the query's
//      RACE features and the normalized ratio readout phi(Q) A / phi(Q) z; then
//      Eq. 5's mass ratio m = 1 / (1 + (lambda d_lr + eps) / exp(lse)) and Eq. 4,
//      O = g_s m O_s + g_lr O_lr, written with the saved statistics.
// Both branches read each query row once (step 4); the keys are read three times
// (hash, summary, block), from the last-level cache after the first.
//
// The outputs are those of elsaa_select + elsaa_lowrank_summary + elsaa_fwd for a
// single hash round and no extra edges: codes, orders, A and z, O, O_s, O_lr, the
// sparse log-sum-exp and d_lr.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

constexpr int kFusedBits = 10;   // sortLSH bits the fused forward takes (1024 bins)
constexpr int kFusedStep = 128;  // keys per summary step (4 waves x 32)

template <typename T, int D, int LP>
struct FusedSmem {
  static constexpr int LD = tile_ld<T>(D), RP = 16 * LP, LDR = tile_ld<T>(RP);
  union U {
    struct {
      T XS[kFusedStep][LD];  // V rows of a summary step
      T FS[kFusedStep][LDR];  // phi(K) rows of the step
    } sum;
    struct {
      T Ks[128][LD];  // K and V rows of the blocks of one round
      T Vs[128][LD];
    } blk;
    int bins[2][1 << kFusedBits];   // counting sort, one array per side
  } u;
  T SF[RP][LD];            // the statistics as the readout's operand, [feature][channel]
  PlanesLds<T, D, LP> PL;  // the RACE hyperplanes as MFMA operands
  alignas(16) float zr[RP];
};

// Static LDS of one workgroup; the codes and orders of the head (4 x N uint16)
// come on top as dynamic LDS.
template <typename T, int D, int LP>
constexpr size_t fused_static_lds() {
  return sizeof(FusedSmem<T, D, LP>);
}

// Code of one row (its NP 16-byte pieces in registers) against `bits` hyperplanes
// ps ([bits][D] fp32; the same for every lane, so read with scalar loads and
// widened exactly to fp64 where used): bit b is the sign of the fp64 chain
// acc = fma(x[j], (double)ps[b][j], acc), j = 0 .. D-1, from +0.0. Two bits at a
// time, so that two independent chains are in flight.
template <typename T, int D>
__device__ __forceinline__ unsigned hash_row(const uint4 (&cur)[D * (int)sizeof(T) / 16],
                                             const float* ps, int bits) {
  constexpr int NP = D * (int)sizeof(T) / 16, EPP = 16 / (int)sizeof(T);
  unsigned cd = 0;
  for (int b = 0; b < bits; b += 2) {
    const float* p0 = ps + b * D;
    const float* p1 = ps + (b + 1 < bits ? b + 1 : b) * D;
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      const uint4 v = cur[c];
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
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const double xd = (double)xv[e];
        a0 = __builtin_fma(xd, (double)p0[c * EPP + e], a0);
        a1 = __builtin_fma(xd, (double)p1[c * EPP + e], a1);
      }
    }
    if (a0 > 0.0) cd |= 1u << b;
    if (b + 1 < bits && a1 > 0.0) cd |= 1u << (b + 1);
  }
  return cd;
}

template <typename T, int D, int LP>
__global__ void __launch_bounds__(256)
    fused_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                     const float* __restrict__ planes_s, const float* __restrict__ planes_lr,
                     const float* __restrict__ lambda, const float* __restrict__ gs,
                     const float* __restrict__ glr, uint16_t* __restrict__ qc,
                     uint16_t* __restrict__ kc, int32_t* __restrict__ qperm,
                     int32_t* __restrict__ kperm, float* __restrict__ A, float* __restrict__ z,
                     T* __restrict__ O, float* __restrict__ Os, T* __restrict__ Olr,
                     float* __restrict__ lse_out, float* __restrict__ dlr_out, int H, int N,
                     int sb, int bits, int L, float scale, float tau, float eps) {
  typedef MF<T> M;
  typedef Features<T, D, LP> Feat;
  typedef FusedSmem<T, D, LP> Sm;
  constexpr int LD = Sm::LD, RP = Sm::RP, LDR = Sm::LDR;
  constexpr int NW = 4, NJP = LP / 2, NFT = RP / 32, NST = (D / 32) * NFT;
  constexpr int SPW = (NST + NW - 1) / NW;
  constexpr int CH = D / 8;  // 8-element pieces of a row
  __shared__ Sm sm;
  extern __shared__ uint16_t dyn[];  // code[2][N], order[2][N]
  uint16_t* const code[2] = {dyn, dyn + N};
  uint16_t* const ord[2] = {dyn + 2 * N, dyn + 3 * N};

  const int bh = blockIdx.x, head = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = wave_id();
  const int r = 16 * L;
  const size_t rb = (size_t)bh * N;
  const T* Qh = Q + rb * D;
  const T* Kh = K + rb * D;
  const T* Vh = V + rb * D;
  const float* pl = planes_lr + (size_t)head * L * 4 * D;
  stage_planes<T, D, LP, 256>(pl, L, sm.PL, tid);  // (read after the first barrier)
  const T* PH = &sm.PL.p[0][0][0];
  const T* PLo = &sm.PL.p[PlanesLds<T, D, LP>::NPART - 1][0][0];
  constexpr int LDP = PlanesLds<T, D, LP>::LDP;

  // ---- 1. codes ----------------------------------------------------------------
  {
    // The hyperplanes are the same for every lane: read with scalar loads (fp32,
    // widened exactly to fp64 where used), not from LDS, whose bandwidth a
    // per-operation broadcast of them would take.
    const float* ps = planes_s + (size_t)head * bits * D;
    // Each thread hashes rows tid, tid + 256, ...; the next row's pieces are loaded
    // while the current row's chains run.
    constexpr int NP = D * (int)sizeof(T) / 16, EPP = 16 / (int)sizeof(T);
    auto row_ptr = [&](int row) __attribute__((always_inline)) {
      const int rr = row < 2 * N ? row : 2 * N - 1;
      return reinterpret_cast<const uint4*>((rr >= N ? Kh : Qh) + (size_t)(rr >= N ? rr - N : rr) * D);
    };
    uint4 cur[NP], nxt[NP];
    {
      const uint4* x = row_ptr(tid);
#pragma unroll
      for (int c = 0; c < NP; ++c) cur[c] = x[c];
    }
    for (int row = tid; row < 2 * N; row += 256) {
      {
        const uint4* x = row_ptr(row + 256);
#pragma unroll
        for (int c = 0; c < NP; ++c) nxt[c] = x[c];
      }
      const unsigned cd = hash_row<T, D>(cur, ps, bits);
      const int isk = row >= N, t = isk ? row - N : row;
      code[isk][t] = (uint16_t)cd;
      (isk ? kc : qc)[rb + t] = (uint16_t)cd;
#pragma unroll
      for (int c = 0; c < NP; ++c) cur[c] = nxt[c];
    }
  }
  __syncthreads();

  // ---- 2. orders: stable counting sort by Gray rank, wave 0 queries, wave 1 keys --
  if (w < 2) {
    int* cnt = sm.u.bins[w];
    const uint16_t* cd = code[w];
    uint16_t* od = ord[w];
    int32_t* gp = (w ? kperm : qperm) + rb;
    const int nbins = 1 << bits;
    for (int i = lane; i < nbins; i += 64) cnt[i] = 0;
    for (int t = lane; t < N; t += 64) atomicAdd(&cnt[gray_rank(cd[t])], 1);
    // Exclusive prefix over the bins: lane l takes a contiguous run of them.
    const int per = (nbins + 63) / 64;
    int run = 0;
    for (int j = 0; j < per; ++j) {
      const int i = lane * per + j;
      if (i < nbins) run += cnt[i];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int base = incl - run;
    for (int j = 0; j < per; ++j) {
      const int i = lane * per + j;
      if (i < nbins) {
        const int c = cnt[i];
        cnt[i] = base;
        base += c;
      }
    }
    // Placement, 64 tokens at a time in token order: a lane goes after the lanes
    // below it with the same rank, and the highest of them advances the bin.
    for (int t0 = 0; t0 < N; t0 += 64) {
      const int t = t0 + lane;
      const bool valid = t < N;
      const unsigned rk = valid ? gray_rank(cd[t]) : (unsigned)nbins;
      unsigned long long same = ~0ull;
      for (int bb = 0; bb <= bits; ++bb) {
        const unsigned long long bal = __ballot((rk >> bb) & 1u);
        same &= ((rk >> bb) & 1u) ? bal : ~bal;
      }
      const int before = __popcll(same & ((1ull << lane) - 1ull));
      const int off = valid ? cnt[rk] : 0;
      const int pos = off + before;
      if (valid && (same >> lane) == 1ull) cnt[rk] = pos + 1;
      if (valid) {
        od[pos] = (uint16_t)t;
        gp[pos] = t;
      }
    }
  }
  __syncthreads();

  // ---- 3. RACE summary: S^T = V^T phi(K) and z = sum phi(K) -------------------------
  floatx16 st[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) st[i] = zero16();
  for (int f = tid; f < RP; f += 256) sm.zr[f] = 0.0f;
  // The next step's K row fragments and V pieces are loaded during this step's
  // products.
  constexpr int VIT = kFusedStep * CH / 256;
  typename M::frag kx[D / M::KSTEP];
  Vec8<T> sv[VIT];
  auto load_step = [&](int s0) __attribute__((always_inline)) {
    const int tok = s0 + 32 * w + col;
    load_row_frags<T, D>(Kh + (size_t)(tok < N ? tok : 0) * D, tok < N, kx, h);
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int p = tid + 256 * i, tk = s0 + p / CH;
      if (tk < N) sv[i].load(Vh + (size_t)tk * D + (p % CH) * 8);
      else sv[i].zero();
    }
  };
  load_step(0);
  for (int s0 = 0; s0 < N; s0 += kFusedStep) {
    Feat::template compute_to_row<0, NJP>(kx, PH, PLo, LDP, L, scale, tau, lane, s0 + 32 * w + col < N,
                                          &sm.u.sum.FS[32 * w + col][0]);
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int p = tid + 256 * i;
      sv[i].store(&sm.u.sum.XS[p / CH][(p % CH) * 8]);
    }
    __syncthreads();
    if (s0 + kFusedStep < N) load_step(s0 + kFusedStep);
    advance_stats<T, D, LP, SPW, kFusedStep, true, NW>(&sm.u.sum.XS[0][0], LD, &sm.u.sum.FS[0][0],
                                                       LDR, nullptr, w, lane, st, &sm.SF[0][0],
                                                       sm.zr);
    __syncthreads();
  }
  // A [d][r] and z [r] of the head (fp32, as elsaa_lowrank_summary writes them).
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int tix = w + NW * i;
    if (tix < NST) {
      const int mt = tix / NFT, f = 32 * (tix % NFT) + col;
      if (f < r)
#pragma unroll
        for (int v = 0; v < 16; ++v) A[(bh * (size_t)D + 32 * mt + acc_row(v, h)) * r + f] = st[i][v];
    }
  }
  for (int f = tid; f < r; f += 256) z[(size_t)bh * r + f] = sm.zr[f];

  // ---- 4. blocks, readout and fusion -----------------------------------------------
  const int KT = sb < 32 ? 32 : sb;  // key rows of a block in LDS
  const int WPB = KT / 32, CB = NW / WPB;  // waves per block, blocks per round
  const int nb = N / sb;
  const float lam = lambda[head];
  const float c2 = scale * kLog2e;
  // The K and V rows of a round's blocks (block c at rows c KT ..), 16-byte row
  // pieces; rows past a block are zero. With D <= 64 the next round's rows are in
  // flight during this round's products (with D = 128 the registers do not allow).
  constexpr int PIT = 128 * CH / 256;
  constexpr bool KV_AHEAD = D <= 64;
  Vec8<T> kb[PIT], vb[PIT];
  auto load_round = [&](int b0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PIT; ++i) {
      const int p = tid + 256 * i, row = p / CH, c8 = (p % CH) * 8;
      const int c = row / KT, t = row % KT, b = b0 + c;
      if (b < nb && t < sb) {
        const int j = ord[1][b * sb + t];
        kb[i].load(Kh + (size_t)j * D + c8);
        vb[i].load(Vh + (size_t)j * D + c8);
      } else {
        kb[i].zero();
        vb[i].zero();
      }
    }
  };
  // This lane's query of round b0 (its block b0 + w / WPB, row 32 (w % WPB) + col).
  const int cb = w / WPB, qloc = 32 * (w % WPB) + col;
  auto query_of = [&](int b0) __attribute__((always_inline)) {
    const int b = b0 + cb;
    return b < nb && qloc < sb ? (int)ord[0][b * sb + qloc] : 0;
  };
  // With D <= 64 the next round's query rows are in flight during this round too.
  typename M::frag qf[D / M::KSTEP], qn[D / M::KSTEP];
  if constexpr (KV_AHEAD) {
    load_round(0);
    prefetch_row_frags<T, D>(Qh + (size_t)query_of(0) * D, qn, h);
  }
  for (int b0 = 0; b0 < nb; b0 += CB) {
    if constexpr (!KV_AHEAD) load_round(b0);
#pragma unroll
    for (int i = 0; i < PIT; ++i) {
      const int p = tid + 256 * i, row = p / CH, c8 = (p % CH) * 8;
      kb[i].store(&sm.u.blk.Ks[row][c8]);
      vb[i].store(&sm.u.blk.Vs[row][c8]);
    }
    const int b = b0 + cb;
    const bool qvalid = b < nb && qloc < sb;
    const int qi = query_of(b0);
    if constexpr (KV_AHEAD) {
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks) qf[ks] = qn[ks];
    } else {
      prefetch_row_frags<T, D>(Qh + (size_t)qi * D, qf, h);
    }
    __syncthreads();
    if constexpr (KV_AHEAD)
      if (b0 + CB < nb) {
        load_round(b0 + CB);
        prefetch_row_frags<T, D>(Qh + (size_t)query_of(b0 + CB) * D, qn, h);
      }
    if (b < nb) {
      const T* Kb = &sm.u.blk.Ks[cb * KT][0];
      const T* Vb = &sm.u.blk.Vs[cb * KT][0];
      // Sparse branch: S^T = K Q^T per key tile (a lane owns a query), online
      // softmax in base 2, O^T += V^T P^T.
      floatx16 o[D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
      float mrun = -INFINITY, lrun = 0.0f;
      for (int kt = 0; kt < KT / 32; ++kt) {
        floatx16 sacc = zero16();
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks)
          sacc = M::mma(row_frag<T>(Kb, LD, 32 * kt, 0, ks, lane), qf[ks], sacc);
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const bool masked = 32 * kt + acc_row(v, h) >= sb;
          sacc[v] = masked ? -INFINITY : sacc[v] * c2;
          mx = fmaxf(mx, sacc[v]);
        }
        const float mnew = fmaxf(mrun, max_halves(mx));
        const float msub = mnew == -INFINITY ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrun - msub);
        float ps = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          sacc[v] = __builtin_amdgcn_exp2f(sacc[v] - msub);
          ps += sacc[v];
        }
        lrun = lrun * alpha + sum_halves(ps);
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
            o[dt] = M::mma(tr_frag<T>(Vb, LD, 32 * kt, 32 * dt, ks2, lane, true), pf, o[dt]);
        }
      }
      // Low-rank branch from the same query rows: num^T = S^T phi(Q)^T, den = phi(Q) . z.
      Feat Fq;
      Fq.compute(qf, PH, PLo, LDP, L, scale, tau, lane);
      float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int jp = 0; jp < NJP; ++jp)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const floatx4 zz = *reinterpret_cast<const floatx4*>(&sm.zr[Feat::feat(jp, 4 * q4, h)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) d4[e] += Fq.phi[jp][4 * q4 + e] * zz[e];
        }
      const float den = sum_halves((d4[0] + d4[1]) + (d4[2] + d4[3]));
      floatx16 num[D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) num[dt] = zero16();
#pragma unroll
      for (int ks = 0; ks < RP / M::KSTEP; ++ks) {
        const typename M::frag fb = Fq.frag(ks);
        const int f0 = Feat::frag_feat(ks, 0, h);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          num[dt] = M::mma(tr_rows(&sm.SF[0][0], LD, f0, f0 + 4, 32 * dt, lane), fb, num[dt]);
      }
      if (qvalid) {
        // Eq. 5 and Eq. 4 (the hardware reciprocal is within 1 ulp: its argument
        // is at least 1).
        const size_t k = rb + qi;
        const float lse = (mrun + __log2f(lrun)) * kLn2;
        const float m = __builtin_amdgcn_rcpf(1.0f + fast_exp(__logf(lam * den + eps) - lse));
        const float g1 = gs ? gs[k] : 1.0f;
        const float g2 = glr ? glr[k] : 1.0f;
        const float inv = 1.0f / lrun, dinv = 1.0f / den;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          float xs[16], xl[16], xo[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            xs[v] = o[dt][v] * inv;
            xl[v] = num[dt][v] * dinv;
            xo[v] = g1 * m * xs[v] + g2 * xl[v];
          }
          // (qvalid is the same for the two lanes of a query)
          store_tile_row(Os + k * D + 32 * dt, xs, h);
          store_tile_row(Olr + k * D + 32 * dt, xl, h);
          store_tile_row(O + k * D + 32 * dt, xo, h);
        }
        if (h == 0) {
          lse_out[k] = lse;
          dlr_out[k] = den;
        }
      }
    }
    __syncthreads();  // the round's rows are no longer read
  }
}

}  // namespace

size_t fused_fwd_lds(const Problem& pb) {
  size_t n = 0;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      with_LP(pb.L, [&](auto lc) {
        constexpr int LP = ELSAA_C(lc);
        if constexpr (LP <= 8) n = fused_static_lds<T, D, LP>() + 8 * (size_t)pb.N;
        else n = ~(size_t)0;
      });
    });
  });
  return n;
}

bool fused_fwd_supported(const Problem& pb) {
  return !pb.causal && pb.rounds == 1 && pb.E == 0 && pb.hash_bits <= kFusedBits &&
         pb.s <= 128 && pb.N <= 65536 && fused_fwd_lds(pb) <= kLdsBytes;
}

void launch_fused_fwd(const Problem& pb, const void* Q, const void* K, const void* V,
                      const float* planes_s, const float* planes_lr, const float* lambda,
                      const float* g_s, const float* g_lr, uint16_t* qc, uint16_t* kc,
                      int32_t* qperm, int32_t* kperm, float* A, float* z, void* O, float* O_s,
                      void* O_lr, float* lse, float* d_lr, hipStream_t st) {
  const int BH = pb.B * pb.H;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      with_LP(pb.L, [&](auto lc) {
        constexpr int LP = ELSAA_C(lc);
        if constexpr (LP <= 8 && fused_static_lds<T, D, LP>() <= kLdsBytes) {
          ELSAA_LAUNCH("fused_fwd", (fused_fwd_kernel<T, D, LP>), dim3(BH), dim3(256),
                       8 * (size_t)pb.N, st, (const T*)Q, (const T*)K, (const T*)V, planes_s,
                       planes_lr, lambda, g_s, g_lr, qc, kc, qperm, kperm, A, z, (T*)O, O_s,
                       (T*)O_lr, lse, d_lr, pb.H, pb.N, pb.s, pb.hash_bits, pb.L, pb.scale,
                       pb.tau, pb.eps);
        }
      });
    });
  });
}

}  // namespace elsaa
