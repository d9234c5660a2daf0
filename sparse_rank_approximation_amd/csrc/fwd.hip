// fwd.hip -- forward of the ELSAA operator on gfx950.
//
// sparse_fwd_kernel (ELSAA paper, Section 3.2): persistent workgroups walk the
// selected blocks. A block's s keys are gathered by the sorted order into LDS (K
// and V row-major, V read transposed); each wave owns 32 of the block's queries
// and streams the keys in tiles of 32 with an online softmax. Scores are formed as S^T = K Q^T so that a
// lane owns one query (column statistics stay in-lane) and the probabilities P^T
// are directly the B operand of O^T += V^T P^T. The normalized block output and
// its log-sum-exp go to a partial slot of the query:
//   causal: leaf blocks (dense causal segments of s tokens) -> slot i,
//           level l block   -> slot N + l N/2 + compact_l(i);
//   non-causal: the single block of query i -> slot i.
//
// fwd_epilogue_kernel: per head and chunk of tokens, in steps of 64 or 128 tokens:
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

// Compact index of query i within level l's future halves (i must be in one). N is
// a power of two whenever there are levels, so the segment length n is one and
// masks and shifts replace divisions.
__device__ __forceinline__ int compact_future(int i, int N, int l) {
  const int n = N >> l;
  return ((i & -n) >> 1) + (i & (n - 1)) - (n >> 1);
}

template <typename T, int D, int SB, bool MR = false>
constexpr size_t sparse_fwd_lds() {
  constexpr int KT = SB < 32 ? 32 : SB;
  return sizeof(T) * 2 * (size_t)KT * tile_ld<T>(D) +
         sizeof(int) * (5 + (MR ? kMaxRounds - 1 : 0)) * KT;
}

// Persistent workgroups take the selected blocks g, g + G, g + 2G, ... (G = grid
// size, a multiple of 8, so that all of a workgroup's blocks are its XCD's share
// in the XCD-aware order). The order entries of the next block are loaded with
// this block's rows and kept in LDS, so that a block's row gathers start at once.
// bf16: two workgroups per CU (two waves per SIMD) is what the LDS allows; the
// register budget is held to it.
// MR: several hash rounds (the pair test against the earlier rounds' blocks and
// its LDS are compiled only then; a lane keeps its query's block indices in
// registers and only the keys' go to LDS, so that two workgroups still fit).
template <typename T, int D, int SB, bool MR>
__global__ void __launch_bounds__(64 * (SB < 32 ? 1 : SB / 32), sizeof(T) == 2 ? 2 : 1)
    sparse_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                      const int32_t* __restrict__ qperm, const int32_t* __restrict__ kperm, int N,
                      int causal, int levels, int rounds, const int32_t* __restrict__ qbid,
                      const int32_t* __restrict__ kbid, float scale, int items, int total,
                      T* __restrict__ Opart, float* __restrict__ Lpart) {
  typedef MF<T> M;
  constexpr int KT = SB < 32 ? 32 : SB;  // key rows held in LDS
  constexpr int LD = tile_ld<T>(D);        // row stride (elements) of the LDS tiles
  constexpr int NT = 64 * (SB < 32 ? 1 : SB / 32);
  __shared__ T Ks[KT][LD];
  __shared__ T Vs[KT][LD];
  __shared__ int kix[2][KT], qix[2][KT];  // key / query token of each row, by block parity
  __shared__ int oslot[KT];               // output slot of each query row
  // Block indices of the key rows in the earlier rounds' orders (several rounds only).
  __shared__ __align__(16) int kbe[MR ? kMaxRounds - 1 : 1][MR ? KT : 1];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = wave_id();  // wave index, uniform (scalar) so that role branches stay uniform
  const size_t P = perm_stride(N, levels, causal, rounds);
  const size_t slots = partial_slots(N, levels, causal, rounds);
  // Orders (round, level) of a head: causal, rounds x levels of N/2 entries each;
  // otherwise one of N per round. Causal items are order-major, then the leaves.
  const int nord = causal ? rounds * levels : rounds;
  const int per_level = causal ? (N / 2) / SB : 0;
  const int nlev_items = causal ? nord * per_level : 0;
  const int G = gridDim.x;

  // Order entries of row t of block g: both are read on every path (a leaf or a
  // row past the block reads the head's first entry and discards it); the choice
  // is made when they are stored, so that nothing waits for them early.
  struct RowIdx {
    int q, k, alt;  // alt: the token itself (causal leaf), -1 past the block, else -2
  };
  auto row_idx = [&](int g, int t) __attribute__((always_inline)) {
    int it;
    const int bh = xcd_item(g, items, per_level, nord, it);
    const bool lf = causal && it >= nlev_items, past = t >= SB;
    const size_t off = (size_t)bh * P + (lf || past ? (size_t)0
                                         : causal ? (size_t)(it / per_level) * (N / 2) +
                                                        (size_t)(it % per_level) * SB + t
                                                  : (size_t)it * SB + t);
    return RowIdx{qperm[off], kperm[off], past ? -1 : lf ? (it - nlev_items) * SB + t : -2};
  };
  auto put_idx = [&](int par, const RowIdx& r) __attribute__((always_inline)) {
    if (tid < KT) {
      qix[par][tid] = r.alt < -1 ? r.q : r.alt;
      kix[par][tid] = r.alt < -1 ? r.k : r.alt;
    }
  };

  int g = blockIdx.x;
  if (g >= total) return;
  put_idx(0, row_idx(g, tid % KT));
  __syncthreads();
  const int qloc = 32 * w + col;  // this lane's query row
  const bool qvalid = qloc < SB;
  for (int par = 0; g < total; g += G, par ^= 1) {
    int item;
    const int bh = xcd_item(g, items, per_level, nord, item);
    const bool leaf = causal && item >= nlev_items;
    // The block's order (-1: a leaf), its level (the segment geometry) and round.
    const int ord = leaf ? -1 : causal ? item / per_level : item / (N / SB);
    const int lev = causal && ord >= 0 ? ord % levels : 0;
    const int rnd = ord < 0 ? 0 : causal ? ord / levels : ord;
    // The next block's order entries, then this block's query rows as MFMA
    // operands (queries past the block read row 0, unused) and its K and V rows
    // gathered into LDS (row-major, 16-byte row-contiguous copies; rows past the
    // block are zero), all loads in flight together.
    const RowIdx nx = row_idx(min(g + G, total - 1), tid % KT);
    const int qi = qvalid ? qix[par][qloc] : 0;
    typename M::frag qf[D / M::KSTEP];
    prefetch_row_frags<T, D>(Q + ((size_t)bh * N + qi) * D, qf, h);
    // Several rounds: the rows' block indices in the earlier rounds' orders of the
    // same level (a pair they share a block in is held there, not here): this
    // lane's query's to registers, the keys' to LDS. Their loads go out before
    // the row gathers, and the keys' reach LDS after them, so that no wait for
    // them holds up the gathers.
    int qbr[kMaxRounds - 1], kbv[kMaxRounds - 1];
#pragma unroll
    for (int r = 0; r < kMaxRounds - 1; ++r) qbr[r] = kbv[r] = -2;
    if constexpr (MR) {
      const int rk = tid < KT ? kix[par][tid] : -1;
#pragma unroll
      for (int r = 0; r < kMaxRounds - 1; ++r)
        if (r < rnd) {
          const size_t base = ((size_t)bh * nord + (causal ? r * levels + lev : r)) * N;
          qbr[r] = qbid[base + qi];
          if (rk >= 0) kbv[r] = kbid[base + rk];
        }
    }
    {
      T* const dst[2] = {&Ks[0][0], &Vs[0][0]};
      const T* const src[2] = {K, V};
      const float* const sc[2] = {nullptr, nullptr};
      gather_rows<T, D, KT, NT, 2>(dst, LD, src, sc, kix[par], (size_t)bh * N, tid);
    }
    if constexpr (MR) {
      if (tid < KT)
#pragma unroll
        for (int r = 0; r < kMaxRounds - 1; ++r) kbe[r][tid] = kbv[r];
    }
    __syncthreads();
    put_idx(par ^ 1, nx);

    floatx16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
    // Online softmax in base 2 (scores times scale log2 e). The running maximum
    // moves only when a score exceeds it by more than 8, so the probabilities
    // against it stay below 2^8, and the output tiles are rescaled only when a
    // lane of the wave moved it (the result is the same; most tiles after the
    // first move no maximum).
    float mrun = -INFINITY, lrun = 0.0f;
    const float c2 = scale * kLog2e;
    // Several rounds: bit v of dup[kt] marks the pair (this lane's query, row v of
    // key tile kt) as one an earlier round holds; formed for all tiles at once so
    // that the LDS reads are in flight together, not in the softmax.
    uint32_t dup[KT / 32];
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt) dup[kt] = 0u;
    if constexpr (MR) {
      if (rnd > 0) {
#pragma unroll
        for (int r = 0; r < kMaxRounds - 1; ++r)
          if (r < rnd)
#pragma unroll
            for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
              for (int gg = 0; gg < 4; ++gg) {
                const int4 kb = *reinterpret_cast<const int4*>(&kbe[r][32 * kt + 8 * gg + 4 * h]);
                const int ke[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (ke[e] == qbr[r]) dup[kt] |= 1u << (4 * gg + e);
              }
      }
    }
    auto ktile = [&](int kt, uint32_t dk) __attribute__((always_inline)) {
      floatx16 sacc = zero16();
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks)
        sacc = M::mma(row_frag<T>(&Ks[0][0], LD, 32 * kt, 0, ks, lane), qf[ks], sacc);
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kr = 32 * kt + acc_row(v, h);
        bool masked = kr >= SB || (leaf && kr > qloc);
        if constexpr (MR) masked = masked || ((dk >> v) & 1u);
        sacc[v] = masked ? -INFINITY : sacc[v] * c2;
        mx = fmaxf(mx, sacc[v]);
      }
      mx = max_halves(mx);
      const float mnew = mx > mrun + 8.0f ? mx : mrun;
      const float msub = mnew == -INFINITY ? 0.0f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(mrun - msub);
      float ps = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sacc[v] = __builtin_amdgcn_exp2f(sacc[v] - msub);
        ps += sacc[v];
      }
      ps = sum_halves(ps);
      lrun = lrun * alpha + ps;
      const bool moved = mnew != mrun;
      mrun = mnew;
      // (before the first tile the output tiles are zero; lanes that kept their
      // maximum have alpha = 1 exactly)
      if (kt > 0 && __any(moved)) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
        const typename M::frag pf = M::from_acc(sacc, ks2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          o[dt] = M::mma(tr_frag<T>(&Vs[0][0], LD, 32 * kt, 32 * dt, ks2, lane, true), pf, o[dt]);
      }
    };
    // Causal leaf: key tiles up to the diagonal; otherwise all of them, unrolled so
    // that one tile's scores can be formed while the previous tile's softmax runs.
    if (leaf) {
      for (int kt = 0; kt <= w; ++kt) ktile(kt, 0u);  // (a leaf is in every round)
    } else {
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt) ktile(kt, dup[kt]);
    }

    // The normalized output tile goes to LDS as rows (one per query, over the key
    // tile once every wave is done with it) and leaves with row-contiguous 16-byte
    // stores to the queries' slots.
    const size_t slot = !causal  ? (size_t)rnd * N + qi
                        : leaf ? (size_t)qi
                               : (size_t)N + (size_t)ord * (N / 2) + compact_future(qi, N, lev);
    __syncthreads();
    {
      // (several rounds: every key of the block may already be held by an earlier
      // round; the partial is then empty, weight 0)
      const float inv = lrun > 0.0f ? 1.0f / lrun : 0.0f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = o[dt][4 * gg + e] * inv;
          store4(&Ks[qloc][32 * dt + 8 * gg + 4 * h], x);
        }
      if (h == 0) oslot[qloc] = qvalid ? (int)slot : -1;
    }
    if (qvalid && h == 0)
      Lpart[(size_t)bh * slots + slot] = lrun > 0.0f ? (mrun + __log2f(lrun)) * kLn2 : -INFINITY;
    __syncthreads();
    {
      // All of the thread's LDS reads are issued before its stores (one wait);
      // rows of a block of 32 or more are all valid, so their stores are
      // unconditional.
      constexpr int CH = D / 8, PIT = (KT * CH + NT - 1) / NT;
      Vec8<T> x[PIT];
      int os[PIT];
#pragma unroll
      for (int i = 0; i < PIT; ++i) {
        const int piece = tid + NT * i, r = min(piece / CH, KT - 1), c8 = (piece % CH) * 8;
        x[i].load(&Ks[r][c8]);
        os[i] = piece < KT * CH ? oslot[r] : -1;
      }
#pragma unroll
      for (int i = 0; i < PIT; ++i) {
        const int piece = tid + NT * i, c8 = (piece % CH) * 8;
        if ((SB >= 32 && (KT * CH) % NT == 0) || os[i] >= 0)
          x[i].store_nt(Opart + ((size_t)bh * slots + os[i]) * D + c8);
      }
    }
    __syncthreads();  // Ks and oslot free for the next block
  }
}

// ---------------------------------------------------------------------------

// Epilogue workgroup: one head and one span of tokens (a summary chunk when
// causal), walked in steps of STEP tokens by 8 waves. LDS (WalkSmem) holds the
// step's keys (V in XS, phi(K) in FS, row-major) and the running RACE statistics
// S = sum_j phi(K_j) V_j^T as an MFMA operand (SF, [feature][channel]); the RACE
// hyperplanes too when PLDS (else they are read from memory, which leaves room
// for a longer step).
template <typename T, int D, int LP, int STEP, bool PLDS>
__global__ void __launch_bounds__(512)
    fwd_epilogue_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                        const float* __restrict__ planes, const float* __restrict__ A,
                        const float* __restrict__ z, const float* __restrict__ Os,
                        const float* __restrict__ lse_s, const float* __restrict__ lambda,
                        const float* __restrict__ gs, const float* __restrict__ glr,
                        T* __restrict__ O, T* __restrict__ Olr, float* __restrict__ dlr_out,
                        int H, int N, int L, int span, int causal, float scale, float tau,
                        float eps) {
  typedef MF<T> M;
  typedef Features<T, D, LP> Feat;
  typedef WalkSmem<T, D, LP, STEP> Sm;
  constexpr int NW = 8, RP = 16 * LP, LDD = Sm::LDD, LDR = Sm::LDR;
  constexpr int QT = STEP / 32;                         // query (and key) tiles per step
  constexpr int NDA = D / 32, NDH = NDA > 1 ? NDA / 2 : 1;  // channel tiles per half
  constexpr int NJP = LP / 2, NJH = NJP > 1 ? NJP / 2 : 1;   // table pairs per half
  constexpr int NFT = RP / 32, NST = NDA * NFT, SPW = (NST + NW - 1) / NW;
  constexpr int VCH = D / 8, VIT = (STEP * VCH + 511) / 512;
  __shared__ Sm sm;
  __shared__ PlanesLds<T, D, PLDS ? LP : 2> PLs;

  const int bh = blockIdx.y, c = blockIdx.x, head = bh % H;
  const int r = 16 * L;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = tid >> 6;
  // Waves w and w + 4 share a SIMD; the causal part of a query tile grows with
  // its index, so the second half takes the tiles in reverse order and every SIMD
  // gets the same work (and with two tiles per step, one of each half).
  const int half = w >> 2, qt = half ? 3 - (w & 3) : (w & 3);
  const bool qwave = qt < QT;
  const float* pl = planes + (size_t)head * L * 4 * D;
  const int t_beg = c * span, t_end = min(N, t_beg + span);
  const float lam = lambda[head];
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * D;

  // Statistics at the start of the span: fp32 tiles in registers (D layout, rows =
  // channels, lanes = features) and their operand copy in SF.
  const size_t sidx = causal ? (size_t)bh * (N / span) + c : (size_t)bh;
  const float* Ac = A + sidx * D * r;
  const float* zc = z + sidx * r;
  floatx16 st[SPW];
  load_stats<T, D, LP, SPW, NW>(Ac, r, 0, w, lane, st, &sm.SF[0][0], LDD);
  if constexpr (PLDS) stage_planes<T, D, LP, 512>(pl, L, PLs, tid);
  const T* PH = &PLs.p[0][0][0];
  const T* PLo = &PLs.p[PlanesLds<T, D, PLDS ? LP : 2>::NPART - 1][0][0];
  constexpr int LDP = PlanesLds<T, D, PLDS ? LP : 2>::LDP;
  for (int f = tid; f < RP; f += 512) sm.zr[f] = f < r ? zc[f] : 0.0f;
  __syncthreads();  // hyperplanes and statistics staged

  // The walk, compiled per half (half 0: channel tiles 0 .. NDH-1 and the first
  // half of the tables of phi(K); half 1: the rest), so that each wave keeps only
  // its own registers; both halves pass the same barriers.
  auto walk = [&](auto hc) __attribute__((always_inline)) {
    constexpr int HALF = decltype(hc)::value;
    constexpr int JP0 = HALF * NJH, DT0 = HALF * NDH;
    constexpr bool FEAT_HALF = HALF == 0 || NJP > 1;
    constexpr bool OWNER = HALF == 0 || NDA > 1;
    constexpr bool EARLY = LP <= 8;  // next step's rows issued early (register room)
    // Rows of one step, loaded one step ahead: the wave's query tile, its key
    // tile (for its half of phi(K)) and a share of the V rows. Tokens past the
    // span read a stand-in row: their outputs are not written and their phi(K)
    // rows are stored as zero, which also cancels their V rows in every product.
    typename M::frag qx[D / M::KSTEP], kx[D / M::KSTEP];
    Vec8<T> vb[VIT];
    auto load_q = [&](int s0) __attribute__((always_inline)) {
      prefetch_row_frags<T, D>(Qh + (size_t)min(s0 + 32 * qt + col, N - 1) * D, qx, h);
    };
    auto load_keys = [&](int s0) __attribute__((always_inline)) {
      if (causal) {
        if (FEAT_HALF) prefetch_row_frags<T, D>(Kh + (size_t)min(s0 + 32 * qt + col, N - 1) * D, kx, h);
#pragma unroll
        for (int i = 0; i < VIT; ++i) {
          const int it = tid + 512 * i, tok = s0 + it / VCH;
          if (it < STEP * VCH) vb[i].load(Vh + (size_t)min(tok, N - 1) * D + (it % VCH) * 8);
        }
      }
    };
    load_q(t_beg);
    load_keys(t_beg);

    for (int s0 = t_beg; s0 < t_end; s0 += STEP) {
      const int qtok = s0 + 32 * qt + col;
      const bool qvalid = qwave && qtok < t_end;
      // Stage the step's keys: this half's phi(K) tables and V into LDS (causal).
      if (causal) {
        if (qwave && FEAT_HALF)
          if constexpr (!PLDS)
            Feat::template compute_to_row<JP0, NJH>(kx, pl, L, scale, tau, lane, qvalid,
                                                    &sm.FS[32 * qt + col][0]);
          else
          Feat::template compute_to_row<JP0, NJH>(kx, PH, PLo, LDP, L, scale, tau, lane, qvalid,
                                                  &sm.FS[32 * qt + col][0]);
#pragma unroll
        for (int i = 0; i < VIT; ++i) {
          const int it = tid + 512 * i;
          if (it < STEP * VCH) vb[i].store(&sm.XS[it / VCH][(it % VCH) * 8]);
        }
      }
      Feat Fq;
      if (qwave && OWNER) {
        if constexpr (PLDS) Fq.compute(qx, PH, PLo, LDP, L, scale, tau, lane);
        else Fq.compute(qx, pl, L, scale, tau, lane);
      }
      // The query's merged sparse output and log-sum-exp, in flight during the
      // readout. Without the early key loads they are issued here, ahead of the
      // key loads of the step (so that waiting for them does not wait for those);
      // with them, after the barrier, where the registers are free.
      const size_t k = (size_t)bh * N + min(qtok, N - 1);
      DRow<float, NDH> osr;
      float lse = 0.0f;
      if constexpr (!EARLY) {
        osr.load(Os + k * D, h, DT0);
        lse = lse_s[k];
      }
      // The next step's keys: issued as soon as this step's are consumed, so that
      // their latency hides behind the readout and the statistics update (past the
      // span: loads nothing that matters). With 16 tables the registers do not
      // allow it: they are issued with the queries.
      if constexpr (EARLY) load_keys(s0 + STEP);
      __syncthreads();

      if (qwave && OWNER) {
        if constexpr (EARLY) {
          osr.load(Os + k * D, h, DT0);
          lse = lse_s[k];
        }
        // Low-rank readout: num^T = S^T phi(Q)^T over this half's channel tiles,
        // den = phi(Q) . z; then the causally masked part of the step.
        floatx16 num[NDH];
#pragma unroll
        for (int i = 0; i < NDH; ++i) num[i] = zero16();
        float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int jp = 0; jp < NJP; ++jp)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const floatx4 zz = *reinterpret_cast<const floatx4*>(&sm.zr[Feat::feat(jp, 4 * q4, h)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) d4[e] += Fq.phi[jp][4 * q4 + e] * zz[e];
          }
        float den = (d4[0] + d4[1]) + (d4[2] + d4[3]);
        den = sum_halves(den);
#pragma unroll
        for (int ks = 0; ks < RP / M::KSTEP; ++ks) {
          const typename M::frag fb = Fq.frag(ks);
          const int f0 = Feat::frag_feat(ks, 0, h);
#pragma unroll
          for (int i = 0; i < NDH; ++i)
            num[i] = M::mma(tr_rows(&sm.SF[0][0], LDD, f0, f0 + 4, 32 * (DT0 + i), lane), fb, num[i]);
        }
        if (causal) {
          float dintra = 0.0f;
          for (int kt = 0; kt <= qt; ++kt) {
            floatx16 wt = zero16();
#pragma unroll
            for (int ks = 0; ks < RP / M::KSTEP; ++ks)
              wt = M::mma(M::load(&sm.FS[32 * kt + col][Feat::frag_feat(ks, 0, h)]), Fq.frag(ks), wt);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              if (kt == qt && acc_row(v, h) > col) wt[v] = 0.0f;
              dintra += wt[v];
            }
#pragma unroll
            for (int ks2 = 0; ks2 < 32 / M::KSTEP; ++ks2) {
              const typename M::frag wf = M::from_acc(wt, ks2);
#pragma unroll
              for (int i = 0; i < NDH; ++i)
                num[i] = M::mma(tr_frag<T>(&sm.XS[0][0], LDD, 32 * kt, 32 * (DT0 + i), ks2, lane, true), wf,
                                num[i]);
            }
          }
          den += sum_halves(dintra);
        }

        if (qvalid) {
          // (the hardware reciprocal is within 1 ulp here: its argument is at least 1)
          const float m = __builtin_amdgcn_rcpf(1.0f + fast_exp(__logf(lam * den + eps) - lse));
          const float g1 = gs ? gs[k] : 1.0f;
          const float g2 = glr ? glr[k] : 1.0f;
          const float dinv = 1.0f / den;
          float os[NDH][4][4];
          osr.unpack(os);
#pragma unroll
          for (int i = 0; i < NDH; ++i) {
            float xo[16], xl[16];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                xl[4 * g + e] = num[i][4 * g + e] * dinv;
                xo[4 * g + e] = g1 * m * os[i][g][e] + g2 * xl[4 * g + e];
              }
            // (qvalid is the same for the two lanes of a token)
            store_tile_row(O + k * D + 32 * (DT0 + i), xo, h);
            store_tile_row(Olr + k * D + 32 * (DT0 + i), xl, h);
          }
          if (HALF == 0 && h == 0) dlr_out[k] = den;
        }
      }
      if (!causal) {  // fixed statistics: on to the next step's queries
        load_q(s0 + STEP);
        continue;
      }
      __syncthreads();
      // Advance the statistics by the step's keys: S^T += V^T phi(K), z += sum phi(K).
      if constexpr (EARLY) load_q(s0 + STEP);
      advance_stats<T, D, LP, SPW, STEP, true, NW>(&sm.XS[0][0], LDD, &sm.FS[0][0], LDR, nullptr, w,
                                                   lane, st, &sm.SF[0][0], sm.zr);
      if constexpr (!EARLY) {
        load_q(s0 + STEP);
        load_keys(s0 + STEP);
      }
      __syncthreads();
    }
  };
  if (half == 0) walk(std::integral_constant<int, 0>{});
  else walk(std::integral_constant<int, 1>{});
}

// Workspace: the slots' log-sum-exps and outputs, the block indices (several
// rounds or extra edges), the extra edges' region.
struct FwdLayout {
  size_t lpart, opart, bids, extra, total;
};
FwdLayout fwd_layout(const Problem& pb) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t BH = (size_t)pb.B * pb.H;
  const size_t slots = partial_slots(pb.N, pb.levels, pb.causal, pb.rounds);
  FwdLayout l;
  size_t off = 0;
  l.lpart = off; off += al(BH * slots * sizeof(float));
  l.opart = off; off += al(BH * slots * pb.d * pb.elem);
  l.bids = off; off += al(block_ids_bytes(pb));
  l.extra = off; off += al(extra_layout(pb, false).total);
  l.total = off;
  return l;
}

size_t fwd_ws_bytes(const Problem& pb) { return fwd_layout(pb).total; }

// The epilogue keeps the RACE hyperplanes in LDS unless that would cut its step
// to 32 tokens where reading them from memory allows a longer one.
template <typename T, int D, int LP>
constexpr bool epilogue_planes_in_lds() {
  constexpr int with = walk_step<T, D, LP, 128, sizeof(PlanesLds<T, D, LP>)>();
  constexpr int without = walk_step<T, D, LP, 128, 0>();
  return with >= 64 || without <= with;
}
template <typename T, int D, int LP>
constexpr int epilogue_step() {
  return epilogue_planes_in_lds<T, D, LP>() ? walk_step<T, D, LP, 128, sizeof(PlanesLds<T, D, LP>)>()
                                            : walk_step<T, D, LP, 128, 0>();
}

size_t fwd_lds_need(const Problem& pb) {
  size_t need = 0;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      with_LP(pb.L, [&](auto lc) {
        constexpr int LP = ELSAA_C(lc);
        constexpr bool PLDS = epilogue_planes_in_lds<T, D, LP>();
        constexpr int STEP = epilogue_step<T, D, LP>();
        need = (PLDS ? sizeof(PlanesLds<T, D, LP>) : 0) +
               (STEP > 0 ? sizeof(WalkSmem<T, D, LP, STEP>) : sizeof(WalkSmem<T, D, LP, 32>));
      });
    });
  });
  const size_t kt = pb.s < 32 ? 32 : pb.s;
  const size_t sparse = (size_t)pb.elem * 2 * kt * (pb.d + (pb.bf16 ? 24 : 8)) +
                        4 * (5 + (pb.rounds > 1 ? 2 * (kMaxRounds - 1) : 0)) * kt;
  return need > sparse ? need : sparse;
}

bool launch_fwd(const Problem& pb, const void* Q, const void* K, const void* V,
                const float* planes_lr, const int32_t* qperm, const int32_t* kperm,
                const float* A, const float* z, const float* lambda, const float* g_s,
                const float* g_lr, const int32_t* extra, void* O, float* O_s, void* O_lr,
                float* lse, float* d_lr, void* ws, hipStream_t st, bool dry) {
  bool ok = true;
  const int BH = pb.B * pb.H;
  const FwdLayout lay = fwd_layout(pb);
  char* base = (char*)ws;
  float* Lpart = (float*)(base + lay.lpart);
  void* Opart = base + lay.opart;
  int32_t* qbid = (int32_t*)(base + lay.bids);
  int32_t* kbid = qbid + block_ids_bytes(pb) / (2 * sizeof(int32_t));
  const ExtraLayout xl = extra_layout(pb, false);
  int32_t* jq = (int32_t*)(base + lay.extra + xl.jq);
  void* Ox = pb.E ? base + lay.extra + xl.rows : nullptr;
  float* Lx = pb.E ? (float*)(base + lay.extra + xl.lse) : nullptr;
  const int nord = pb.causal ? pb.rounds * pb.levels : pb.rounds;
  const int items = pb.causal ? nord * (pb.N / 2) / pb.s + pb.N / pb.s : nord * (pb.N / pb.s);
  if (!dry && (pb.rounds > 1 || pb.E > 0)) launch_block_ids(pb, qperm, kperm, qbid, kbid, st);
  if (!dry && pb.E > 0) {
    launch_extra_prep(pb, extra, qbid, kbid, jq, nullptr, nullptr, st);
    launch_extra_fwd(pb, Q, K, V, jq, Ox, Lx, st);
  }
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      auto run = [&](auto sc) {
        constexpr int SB = ELSAA_C(sc);
        auto go = [&](auto mc) {
          constexpr bool MR = decltype(mc)::value;
          if constexpr (sparse_fwd_lds<T, D, SB, MR>() > kLdsBytes) {
            ok = false;
          } else if (!dry) {
            constexpr int NT = 64 * (SB < 32 ? 1 : SB / 32);
            const int total = items * BH;
            const int G = persistent_grid((const void*)sparse_fwd_kernel<T, D, SB, MR>, NT, total);
            // The kernel reads an order entry for every row, leaves included; with no
            // level (causal, N = s) the orders are empty and may be null, and the
            // entry it reads (and discards) is then the first word of the workspace.
            const int32_t* qp = qperm ? qperm : (const int32_t*)Lpart;
            const int32_t* kp = kperm ? kperm : (const int32_t*)Lpart;
            ELSAA_LAUNCH("sparse_fwd", (sparse_fwd_kernel<T, D, SB, MR>), dim3(G), dim3(NT), 0, st,
                         (const T*)Q, (const T*)K, (const T*)V, qp, kp, pb.N, (int)pb.causal,
                         pb.levels, pb.rounds, qbid, kbid, pb.scale, items, total, (T*)Opart,
                         Lpart);
          }
        };
        if (pb.rounds > 1) go(std::true_type{});
        else go(std::false_type{});
      };
      switch (pb.s) {
        case 16: run(std::integral_constant<int, 16>{}); break;
        case 32: run(std::integral_constant<int, 32>{}); break;
        case 64: run(std::integral_constant<int, 64>{}); break;
        case 128: run(std::integral_constant<int, 128>{}); break;
        default: run(std::integral_constant<int, 256>{}); break;
      }
      if (!dry) launch_merge(pb, Opart, Lpart, Ox, Lx, O_s, lse, st);
      with_LP(pb.L, [&](auto lc) {
        constexpr int LP = ELSAA_C(lc);
        constexpr bool PLDS = epilogue_planes_in_lds<T, D, LP>();
        constexpr int STEP = epilogue_step<T, D, LP>();
        if constexpr (STEP == 0) {
          ok = false;
        } else if (!dry) {
          const int span = pb.causal ? pb.chunk : noncausal_span(pb.N, BH, STEP);
          const int nspan = (pb.N + span - 1) / span;
          ELSAA_LAUNCH("fwd_epilogue", (fwd_epilogue_kernel<T, D, LP, STEP, PLDS>), dim3(nspan, BH),
                       dim3(512), 0, st, (const T*)Q, (const T*)K, (const T*)V, planes_lr, A, z,
                       O_s, lse, lambda, g_s, g_lr, (T*)O, (T*)O_lr, d_lr, pb.H, pb.N,
                       pb.L, span, (int)pb.causal, pb.scale, pb.tau, pb.eps);
        }
      });
    });
  });
  return ok;
}

}  // namespace elsaa
