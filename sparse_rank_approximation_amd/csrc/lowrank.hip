// lowrank.hip -- RACE bucket statistics (ELSAA paper, Section 3.1: keys are
// softly assigned to hypercube buckets of every table and key/value statistics
// are accumulated per bucket; causally, the statistics of strictly earlier
// chunks are combined by prefix sums).
//
// lr_sums_kernel: per (head, tile of TT tokens) the sums
//     S^T[e][f] = sum_t phi_f(X_t) alpha_t Y_t[e],   z[f] = sum_t phi_f(X_t) beta_t
// (forward: X = K, Y = V, alpha = beta = 1), as a bf16/fp32 MFMA contraction over
// the tokens with fp32 accumulation.
// lr_scan_kernel: combines the tile sums into the summaries: the total
// (non-causal), the exclusive prefix (causal forward) or the exclusive suffix
// (causal backward) over tiles.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

template <typename T, int D, int LP, int SUB>
struct SumsSmem {
  static constexpr int LDD = tile_ld<T>(D), LDR = tile_ld<T>(16 * LP);
  T YS[SUB][LDD];        // alpha_t Y_t of the step, [token][channel]
  T FS[SUB][LDR];        // phi(X_t) of the step, [token][feature]
  alignas(16) float zr[16 * LP];
  alignas(16) float bet[SUB];
};

// Largest step (128, 64 or 32 tokens) whose LDS (with the staged hyperplanes) fits.
template <typename T, int D, int LP>
constexpr int sums_step() {
  constexpr size_t P = sizeof(PlanesLds<T, D, LP>);
  return sizeof(SumsSmem<T, D, LP, 128>) + P <= kLdsBytes  ? 128
         : sizeof(SumsSmem<T, D, LP, 64>) + P <= kLdsBytes ? 64
                                                            : 32;
}

// One workgroup per (head, tile of TT tokens), 8 waves, SUB tokens per step: wave
// w < SUB / 32 featurizes token tile w of the step (hyperplanes in LDS), waves
// 4..7 stage the step's alpha-scaled Y rows; then st += Y^T phi(X) and
// z += phi(X)^T beta on MFMA (advance_stats, tiles spread over the 8 waves) with
// the next step's rows already in flight. Eight waves keep each wave's registers
// within half the file, so two waves share each SIMD.
// WEIGHTED: alpha and beta are given (else both are 1), a compile-time choice so
// that the weight loads are unconditional and never make the row loads wait.
template <typename T, int D, int LP, int SUB, bool WEIGHTED>
__global__ void __launch_bounds__(512) lr_sums_kernel(const T* __restrict__ X, const T* __restrict__ Y,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta,
                                                      const float* __restrict__ planes, int H, int N,
                                                      int L, int TT, float scale, float tau,
                                                      float* __restrict__ S, float* __restrict__ Z) {
  typedef MF<T> M;
  typedef Features<T, D, LP> Feat;
  typedef SumsSmem<T, D, LP, SUB> Sm;
  constexpr int NW = 8, RP = 16 * LP, NFT = RP / 32, NST = (D / 32) * NFT;
  constexpr int SPW = (NST + NW - 1) / NW;
  constexpr int QT = SUB / 32, LDD = Sm::LDD, LDR = Sm::LDR;
  constexpr int VCH = D / 8, VIT = (SUB * VCH + 255) / 256;  // per staging thread (waves 4..7)
  __shared__ Sm sm;
  __shared__ PlanesLds<T, D, LP> PLs;
  const int bh = blockIdx.y, tile = blockIdx.x, ntile = gridDim.x;
  const int r = 16 * L;
  const int t0 = tile * TT, t1 = min(N, t0 + TT);
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = wave_id();  // wave index, uniform (scalar) so that role branches stay uniform
  const T* Xh = X + (size_t)bh * N * D;
  const T* Yh = Y + (size_t)bh * N * D;
  stage_planes<T, D, LP, 512>(planes + (size_t)(bh % H) * L * 4 * D, L, PLs, tid);
  const T* PH = &PLs.p[0][0][0];
  const T* PLo = &PLs.p[PlanesLds<T, D, LP>::NPART - 1][0][0];
  constexpr int LDP = PlanesLds<T, D, LP>::LDP;
  for (int f = tid; f < RP; f += 512) sm.zr[f] = 0.0f;
  const int ts = tid - 256;  // staging thread index (waves 4..7)

  floatx16 st[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) st[i] = zero16();

  // Rows of one step (tokens past the tile read a stand-in row and get zero
  // weight: their phi rows are stored as zero).
  typename M::frag xr[D / M::KSTEP];
  Vec8<T> yb[VIT];
  float ya[VIT], bt = 1.0f;
#pragma unroll
  for (int i = 0; i < VIT; ++i) ya[i] = 1.0f;
  auto load_rows = [&](int s0) __attribute__((always_inline)) {
    if (w < QT) prefetch_row_frags<T, D>(Xh + (size_t)min(s0 + 32 * w + col, N - 1) * D, xr, h);
    if (ts >= 0) {
#pragma unroll
      for (int i = 0; i < VIT; ++i) {
        const int it = ts + 256 * i, tc = min(s0 + it / VCH, N - 1);
        if ((SUB * VCH) % 256 == 0 || it < SUB * VCH) yb[i].load(Yh + (size_t)tc * D + (it % VCH) * 8);
        if constexpr (WEIGHTED) ya[i] = alpha[(size_t)bh * N + tc];
      }
      if constexpr (WEIGHTED) bt = beta[(size_t)bh * N + min(s0 + ts % SUB, N - 1)];
    }
  };
  __syncthreads();  // hyperplanes staged
  load_rows(t0);
  for (int s0 = t0; s0 < t1; s0 += SUB) {
    if (w < QT)
      Feat::compute_to_row(xr, PH, PLo, LDP, L, scale, tau, lane, s0 + 32 * w + col < t1,
                           &sm.FS[32 * w + col][0]);
    if (ts >= 0) {
#pragma unroll
      for (int i = 0; i < VIT; ++i) {
        const int it = ts + 256 * i;
        if (it < SUB * VCH) {
          yb[i].scale(s0 + it / VCH < t1 ? ya[i] : 0.0f);
          yb[i].store(&sm.YS[it / VCH][(it % VCH) * 8]);
        }
      }
      if (ts < SUB) sm.bet[ts] = s0 + ts < t1 ? bt : 0.0f;
    }
    __syncthreads();
    load_rows(s0 + SUB);
    advance_stats<T, D, LP, SPW, SUB, false, NW>(&sm.YS[0][0], LDD, &sm.FS[0][0], LDR, sm.bet, w,
                                                 lane, st, nullptr, sm.zr);
    __syncthreads();
  }

  const size_t base = (size_t)bh * ntile + tile;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int tix = w + NW * i;
    if (tix < NST) {
      const int mt = tix / NFT, f = 32 * (tix % NFT) + col;
      if (f < r)
#pragma unroll
        for (int v = 0; v < 16; ++v) S[(base * D + 32 * mt + acc_row(v, h)) * r + f] = st[i][v];
    }
  }
  for (int f = tid; f < r; f += 512) Z[base * r + f] = sm.zr[f];
}

// mode 0: total over tiles (one output); 1: exclusive prefix; 2: exclusive suffix.
__global__ void __launch_bounds__(256) lr_scan_kernel(const float* __restrict__ S,
                                                      const float* __restrict__ Z, float* __restrict__ A,
                                                      float* __restrict__ zo, int ntile, int per,
                                                      int r, int mode) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= per + r) return;
  const bool isz = e >= per;
  const int idx = isz ? e - per : e, stride = isz ? r : per;
  const float* src = (isz ? Z : S) + (size_t)bh * ntile * stride + idx;
  const int nout = mode == 0 ? 1 : ntile;
  float* dst = (isz ? zo : A) + (size_t)bh * nout * stride + idx;
  float run = 0.0f;
  if (mode == 0) {
    for (int c = 0; c < ntile; ++c) run += src[(size_t)c * stride];
    dst[0] = run;
  } else if (mode == 1) {
    for (int c = 0; c < ntile; ++c) {
      const float v = src[(size_t)c * stride];
      dst[(size_t)c * stride] = run;
      run += v;
    }
  } else {
    for (int c = ntile - 1; c >= 0; --c) {
      const float v = src[(size_t)c * stride];
      dst[(size_t)c * stride] = run;
      run += v;
    }
  }
}

int lr_tiles(const Problem& pb) {
  const int TT = lr_tile_tokens(pb);
  return (pb.N + TT - 1) / TT;
}

int lr_tile_tokens(const Problem& pb) { return pb.causal ? pb.chunk : (pb.N < 512 ? pb.N : 512); }

void run_lr_sums(const Problem& pb, const void* X, const void* Y, const float* alpha,
                 const float* beta, const float* planes, float* S, float* Z, hipStream_t st) {
  const int BH = pb.B * pb.H, TT = lr_tile_tokens(pb), nt = lr_tiles(pb);
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      with_LP(pb.L, [&](auto lc) {
        constexpr int LP = ELSAA_C(lc);
        constexpr int SUB = sums_step<T, D, LP>();
        auto go = [&](auto wc) {
          constexpr bool W = decltype(wc)::value;
          ELSAA_LAUNCH("lr_sums", (lr_sums_kernel<T, D, LP, SUB, W>), dim3(nt, BH), dim3(512), 0, st,
                       (const T*)X, (const T*)Y, alpha, beta, planes, pb.H, pb.N, pb.L, TT,
                       pb.scale, pb.tau, S, Z);
        };
        if (alpha) go(std::true_type{});
        else go(std::false_type{});
      });
    });
  });
}

void run_lr_scan(const Problem& pb, const float* S, const float* Z, int mode, float* A, float* z,
                 hipStream_t st) {
  const int BH = pb.B * pb.H, nt = lr_tiles(pb), per = pb.d * pb.r;
  ELSAA_LAUNCH("lr_scan", lr_scan_kernel, dim3((per + pb.r + 255) / 256, BH), dim3(256), 0, st, S, Z, A,
                     z, nt, per, pb.r, mode);
}

size_t summary_lds_need(const Problem& pb) {
  size_t need = 0;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      with_LP(pb.L, [&](auto lc) {
        constexpr int LP = ELSAA_C(lc);
        need = sizeof(SumsSmem<T, D, LP, sums_step<T, D, LP>()>) + sizeof(PlanesLds<T, D, LP>);
      });
    });
  });
  return need;
}

size_t summary_ws_bytes(const Problem& pb) {
  return sizeof(float) * (size_t)pb.B * pb.H * lr_tiles(pb) * ((size_t)pb.d * pb.r + pb.r);
}

void launch_summary(const Problem& pb, const void* K, const void* V, const float* planes_lr,
                    float* A, float* z, void* ws, hipStream_t st) {
  float* S = (float*)ws;
  float* Z = S + (size_t)pb.B * pb.H * lr_tiles(pb) * pb.d * pb.r;
  run_lr_sums(pb, K, V, nullptr, nullptr, planes_lr, S, Z, st);
  run_lr_scan(pb, S, Z, pb.causal ? 1 : 0, A, z, st);
}

}  // namespace elsaa
