// lowrank.hip -- RACE bucket statistics (ELSAA paper, Section 3.1: keys are
// softly assigned to hypercube buckets of every table and key/value statistics
// are accumulated per bucket; causally, the statistics of strictly earlier
// chunks are combined by prefix sums).
//
// lr_sums_kernel: per (head, tile of TT tokens) the sums
//     S^T[e][f] = sum_t phi_f(X_t) alpha_t Y_t[e],   z[f] = sum_t phi_f(X_t) beta_t
// (forward: X = K, Y = V, alpha = beta = 1), as a bf16/fp32 MFMA contraction over
// the tokens with fp32 accumulation, 64 tokens per step.
// lr_scan_kernel: combines the tile sums into the summaries: the total
// (non-causal), the exclusive prefix (causal forward) or the exclusive suffix
// (causal backward) over tiles.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

template <typename T, int D, int LP>
__global__ void __launch_bounds__(256) lr_sums_kernel(const T* __restrict__ X, const T* __restrict__ Y,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta,
                                                      const float* __restrict__ planes, int H, int N,
                                                      int L, int TT, float scale, float tau,
                                                      float* __restrict__ S, float* __restrict__ Z) {
  typedef MF<T> M;
  constexpr int RP = 16 * LP, SUB = 64, PAD = 8;
  constexpr int NT_N = RP / 32, NTILES = (D / 32) * NT_N, TPW = (NTILES + 3) / 4;
  __shared__ T KfT[RP][SUB + PAD];
  __shared__ T YT[D][SUB + PAD];
  __shared__ float bet[SUB];
  const int bh = blockIdx.y, tile = blockIdx.x, ntile = gridDim.x;
  const int r = 16 * L;
  const int t0 = tile * TT, t1 = min(N, t0 + TT);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const float* pl = planes + (size_t)(bh % H) * L * 4 * D;

  floatx16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero16();
  float zacc = 0.0f;

  for (int s0 = t0; s0 < t1; s0 += SUB) {
    if (w < 2) {
      const int tok = s0 + 32 * w + col;
      const bool valid = tok < t1;
      Features<T, D, LP> F;
      F.compute(X + ((size_t)bh * N + (valid ? tok : t0)) * D, valid, pl, L, scale, tau, lane);
#pragma unroll
      for (int jp = 0; jp < LP / 2; ++jp)
#pragma unroll
        for (int b = 0; b < 16; ++b)
          KfT[Features<T, D, LP>::feat(jp, b, h)][32 * w + col] = from_f<T>(valid ? F.phi[jp][b] : 0.0f);
      if (h == 0) bet[32 * w + col] = valid ? (beta ? beta[(size_t)bh * N + tok] : 1.0f) : 0.0f;
    } else {
      for (int idx = tid - 128; idx < SUB * (D / 8); idx += 128) {
        const int tk = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
        const int tok = s0 + tk;
        float y[8];
        if (tok < t1) {
          const float a = alpha ? alpha[(size_t)bh * N + tok] : 1.0f;
          const T* yr = Y + ((size_t)bh * N + tok) * D + c8;
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = to_f(yr[e]) * a;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) YT[c8 + e][tk] = from_f<T>(y[e]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tix = w + 4 * i;
      if (tix < NTILES) {
        const int mt = tix / NT_N, nt = tix % NT_N;
#pragma unroll
        for (int ks = 0; ks < SUB / M::KSTEP; ++ks) {
          const int k0 = ks * M::KSTEP + M::KPL * h;
          acc[i] = M::mma(M::load(&YT[32 * mt + col][k0]), M::load(&KfT[32 * nt + col][k0]), acc[i]);
        }
      }
    }
    if (tid < RP) {
#pragma unroll 8
      for (int t = 0; t < SUB; ++t) zacc += to_f(KfT[tid][t]) * bet[t];
    }
    __syncthreads();
  }

  const size_t base = (size_t)bh * ntile + tile;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tix = w + 4 * i;
    if (tix < NTILES) {
      const int mt = tix / NT_N, nt = tix % NT_N;
      const int f = 32 * nt + col;
      if (f < r) {
#pragma unroll
        for (int v = 0; v < 16; ++v) S[(base * D + 32 * mt + acc_row(v, h)) * r + f] = acc[i][v];
      }
    }
  }
  if (tid < r) Z[base * r + tid] = zacc;
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
        ELSAA_LAUNCH("lr_sums", (lr_sums_kernel<T, D, LP>), dim3(nt, BH), dim3(256), 0, st,
                           (const T*)X, (const T*)Y, alpha, beta, planes, pb.H, pb.N, pb.L, TT,
                           pb.scale, pb.tau, S, Z);
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
