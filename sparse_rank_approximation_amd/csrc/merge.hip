// merge.hip -- per-token reductions over the sparse branch's partial slots (every
// level and every hash round of a token), as
// streaming kernels (each lane owns a 16-byte piece of a row, D / 8 lanes per row,
// and every slot of a batch is loaded before any is used):
//   merge_kernel    forward: the log-sum-exp merge of a query's partial block
//                   outputs (Section 3.2's recursive merge, which keeps the softmax
//                   normalised over the union of the blocks) -> O_s and lse;
//   combine_kernel  backward: out = out + sum of the token's partial gradient rows,
//                   where out holds the low-rank branch's part on entry.
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

// Slots in flight per lane (MB): measured per kernel at the headline workload
// (merge 4, dQ combine 2, dK/dV combine 4; 8 cost each of them 8-12 %, 16 nearly
// doubled them: more rows in flight per lane hold more registers, and fewer
// workgroups stay resident).
constexpr int kMergeBatch = 4, kCombineQBatch = 2, kCombineKVBatch = 4;

template <typename T, int D, int MB>
__global__ void __launch_bounds__(256)
    merge_kernel(const T* __restrict__ Opart, const float* __restrict__ Lpart,
                 const T* __restrict__ Ox, const float* __restrict__ Lx, int N, int levels,
                 int causal, int rounds, float* __restrict__ Os, float* __restrict__ lse) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int tok = blockIdx.x * RPB + tid / LPR, c8 = (tid % LPR) * 8;
  const bool valid = tok < N;
  const size_t slots = partial_slots(N, levels, causal, rounds);
  const T* Op = Opart + (size_t)bh * slots * D + c8;
  const float* Lp = Lpart + (size_t)bh * slots;
  SlotWalk<true> sw(valid ? tok : 0, N, levels, causal != 0, rounds);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.0f;
  for (;;) {
    size_t sl[MB];
    const int n = valid ? sw.template next<MB>(sl) : 0;
    if (!__any(n > 0)) break;
    Vec8<T> raw[MB];
    float lw[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j)
      if (j < n) {
        raw[j].load(Op + sl[j] * D);
        lw[j] = Lp[sl[j]];
      }
    if (n > 0) {
      float bm = -INFINITY;
#pragma unroll
      for (int j = 0; j < MB; ++j)
        if (j < n) bm = fmaxf(bm, lw[j]);
      const float mnew = fmaxf(mrun, bm);
      const float a = fast_exp(mrun - mnew);  // 0 on the first batch (mrun = -inf)
      lrun *= a;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= a;
#pragma unroll
      for (int j = 0; j < MB; ++j)
        if (j < n) {
          const float wj = fast_exp(lw[j] - mnew);
          lrun += wj;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += wj * raw[j].get(e);
        }
      mrun = mnew;
    }
  }
  // The extra edges' partial (every token has a sortLSH partial, so mrun is
  // finite here; an empty extra partial has weight 0).
  if (Ox && valid) {
    Vec8<T> raw;
    raw.load(Ox + ((size_t)bh * N + tok) * D + c8);
    const float lw = Lx[(size_t)bh * N + tok], mnew = fmaxf(mrun, lw);
    const float a = fast_exp(mrun - mnew), wj = fast_exp(lw - mnew);
    lrun = lrun * a + wj;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + wj * raw.get(e);
    mrun = mnew;
  }
  if (valid) {
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    store8(Os + ((size_t)bh * N + tok) * D + c8, acc);
    if (c8 == 0) lse[(size_t)bh * N + tok] = mrun + __logf(lrun);
  }
}

template <typename T, int D, bool QUERY, int NX, int MB>
__global__ void __launch_bounds__(256)
    combine_kernel(const T* __restrict__ p0, const T* __restrict__ p1, const T* __restrict__ x0,
                   const T* __restrict__ x1, T* __restrict__ o0, T* __restrict__ o1, int N,
                   int levels, int causal, int rounds) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int tok = blockIdx.x * RPB + tid / LPR, c8 = (tid % LPR) * 8;
  const bool valid = tok < N;
  const size_t slots = partial_slots(N, levels, causal, rounds);
  const T* const part[2] = {p0 + (size_t)bh * slots * D + c8, p1 ? p1 + (size_t)bh * slots * D + c8 : nullptr};
  T* const out[2] = {o0, o1};
  const size_t row = ((size_t)bh * N + (valid ? tok : 0)) * D + c8;
  float acc[NX][8];
#pragma unroll
  for (int x = 0; x < NX; ++x) load8(out[x] + row, acc[x]);
  SlotWalk<QUERY> sw(valid ? tok : 0, N, levels, causal != 0, rounds);
  for (;;) {
    size_t sl[MB];
    const int n = valid ? sw.template next<MB>(sl) : 0;
    if (!__any(n > 0)) break;
    Vec8<T> raw[NX][MB];
#pragma unroll
    for (int j = 0; j < MB; ++j)
      if (j < n)
#pragma unroll
        for (int x = 0; x < NX; ++x) raw[x][j].load(part[x] + sl[j] * D);
#pragma unroll
    for (int j = 0; j < MB; ++j)
      if (j < n)
#pragma unroll
        for (int x = 0; x < NX; ++x)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[x][e] += raw[x][j].get(e);
  }
  if (x0 && valid) {  // the extra edges' part (one row per token)
    const T* const xs[2] = {x0, x1};
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      Vec8<T> raw;
      raw.load(xs[x] + row);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[x][e] += raw.get(e);
    }
  }
  if (valid)
#pragma unroll
    for (int x = 0; x < NX; ++x) store8(out[x] + row, acc[x]);
}

}  // namespace

void launch_merge(const Problem& pb, const void* Opart, const float* Lpart, const void* Ox,
                  const float* Lx, float* O_s, float* lse, hipStream_t st) {
  const int BH = pb.B * pb.H;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      constexpr int RPB = 256 / (D / 8);
      ELSAA_LAUNCH("merge", (merge_kernel<T, D, kMergeBatch>), dim3((pb.N + RPB - 1) / RPB, BH), dim3(256), 0,
                   st, (const T*)Opart, Lpart, (const T*)Ox, Lx, pb.N, pb.levels, (int)pb.causal,
                   pb.rounds, O_s, lse);
    });
  });
}

void launch_combine(const Problem& pb, const void* dQp, const void* dKp, const void* dVp,
                    const void* dQx, const void* dKx, const void* dVx, void* dQ, void* dK,
                    void* dV, hipStream_t st) {
  const int BH = pb.B * pb.H;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      constexpr int RPB = 256 / (D / 8);
      const dim3 grid((pb.N + RPB - 1) / RPB, BH);
      ELSAA_LAUNCH("combine_q", (combine_kernel<T, D, true, 1, kCombineQBatch>), grid, dim3(256), 0, st,
                   (const T*)dQp, (const T*)nullptr, (const T*)dQx, (const T*)nullptr, (T*)dQ,
                   (T*)nullptr, pb.N, pb.levels,
                   (int)pb.causal, pb.rounds);
      ELSAA_LAUNCH("combine_kv", (combine_kernel<T, D, false, 2, kCombineKVBatch>), grid, dim3(256), 0, st,
                   (const T*)dKp, (const T*)dVp, (const T*)dKx, (const T*)dVx, (T*)dK, (T*)dV,
                   pb.N, pb.levels,
                   (int)pb.causal, pb.rounds);
    });
  });
}

}  // namespace elsaa
