// gates.hip -- learnable gates of Eq. 4 (g_sparse,i and g_lr,i, learned with the
// model: ELSAA paper, Sections 7 and 8) as the logistic function of a per-head
// affine projection of the query, g_k,i = sigmoid(<W_k, Q_i> + b_k), and their
// backward:
//   gates_fwd_kernel     g_s, g_lr from Q (streaming, D/8 lanes per row);
//   gates_bwd_kernel     dt_k = dL/dg_k g_k (1 - g_k); dQ_i += dt_s W_s + dt_lr W_lr
//                        (in place); per-workgroup sums of dt_k Q_i and dt_k;
//   gates_reduce_kernel  dW, db per head from those sums in a fixed order
//                        (deterministic).
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

namespace {

constexpr int kGateRows = 128;  // rows per workgroup

template <typename T, int D>
__global__ void __launch_bounds__(256)
    gates_fwd_kernel(const T* __restrict__ Q, const float* __restrict__ W,
                     const float* __restrict__ b, int H, int N, float* __restrict__ gs,
                     float* __restrict__ glr) {
  constexpr int TPR = D / 8, RPI = 256 / TPR;
  const int bh = blockIdx.y, head = bh % H, tid = threadIdx.x;
  const int part = tid % TPR, c8 = part * 8;
  float w0[8], w1[8];
  load8(W + (size_t)head * 2 * D + c8, w0);
  load8(W + ((size_t)head * 2 + 1) * D + c8, w1);
  const float b0 = b[2 * head], b1 = b[2 * head + 1];
  const int r0 = blockIdx.x * kGateRows;
#pragma unroll 2
  for (int rr = tid / TPR; rr < kGateRows; rr += RPI) {
    const int i = r0 + rr;
    const bool valid = i < N;
    float x[8];
    load8(Q + ((size_t)bh * N + (valid ? i : 0)) * D + c8, x);
    float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      t0 = fmaf(w0[e], x[e], t0);
      t1 = fmaf(w1[e], x[e], t1);
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) {
      t0 += __shfl_xor(t0, off, 64);
      t1 += __shfl_xor(t1, off, 64);
    }
    if (valid && part == 0) {
      gs[(size_t)bh * N + i] = 1.0f / (1.0f + __expf(-(t0 + b0)));
      glr[(size_t)bh * N + i] = 1.0f / (1.0f + __expf(-(t1 + b1)));
    }
  }
}

// Workgroup (row tile, head): thread (row slot, part) owns channels 8 part .. + 8
// of rows rr, rr + RPI, ...; its sums of dt_k Q over those rows meet in LDS, added
// in a fixed order.
template <typename T, int D>
__global__ void __launch_bounds__(256)
    gates_bwd_kernel(const T* __restrict__ Q, const float* __restrict__ W,
                     const float* __restrict__ gs, const float* __restrict__ glr,
                     const float* __restrict__ dgs, const float* __restrict__ dglr, int H, int N,
                     T* __restrict__ dQ, float* __restrict__ part_w) {
  constexpr int TPR = D / 8, RPI = 256 / TPR;
  __shared__ float red[RPI][2][D + 1];
  __shared__ float redb[RPI][2];
  const int bh = blockIdx.y, head = bh % H, tid = threadIdx.x;
  const int slot = tid / TPR, part = tid % TPR, c8 = part * 8;
  float w0[8], w1[8];
  load8(W + (size_t)head * 2 * D + c8, w0);
  load8(W + ((size_t)head * 2 + 1) * D + c8, w1);
  float aw0[8] = {0, 0, 0, 0, 0, 0, 0, 0}, aw1[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float ab0 = 0.0f, ab1 = 0.0f;
  const int r0 = blockIdx.x * kGateRows;
  for (int rr = slot; rr < kGateRows; rr += RPI) {
    const int i = r0 + rr;
    if (i >= N) break;
    const size_t k = (size_t)bh * N + i;
    const float g0 = gs[k], g1 = glr[k];
    const float t0 = dgs[k] * g0 * (1.0f - g0), t1 = dglr[k] * g1 * (1.0f - g1);
    const size_t row = k * D + c8;
    float x[8], dq[8];
    load8(Q + row, x);
    load8(dQ + row, dq);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      aw0[e] = fmaf(t0, x[e], aw0[e]);
      aw1[e] = fmaf(t1, x[e], aw1[e]);
      dq[e] = fmaf(t0, w0[e], fmaf(t1, w1[e], dq[e]));
    }
    store8(dQ + row, dq);
    ab0 += t0;
    ab1 += t1;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[slot][0][c8 + e] = aw0[e];
    red[slot][1][c8 + e] = aw1[e];
  }
  if (part == 0) {
    redb[slot][0] = ab0;
    redb[slot][1] = ab1;
  }
  __syncthreads();
  // Workgroup sums: 2 D weight sums and 2 bias sums, over the row slots in order.
  float* out = part_w + ((size_t)bh * gridDim.x + blockIdx.x) * (2 * D + 2);
  for (int j = tid; j < 2 * D + 2; j += 256) {
    float s = 0.0f;
    if (j < 2 * D)
      for (int r = 0; r < RPI; ++r) s += red[r][j / D][j % D];
    else
      for (int r = 0; r < RPI; ++r) s += redb[r][j - 2 * D];
    out[j] = s;
  }
}

// dW [H][2][D] and db [H][2]: for head h, the workgroup sums of every batch entry
// and row tile, in order.
__global__ void __launch_bounds__(256)
    gates_reduce_kernel(const float* __restrict__ part_w, int B, int H, int nblk, int D,
                        float* __restrict__ dW, float* __restrict__ db) {
  const int h = blockIdx.x;
  for (int j = threadIdx.x; j < 2 * D + 2; j += 256) {
    float s = 0.0f;
    for (int bb = 0; bb < B; ++bb)
      for (int k = 0; k < nblk; ++k)
        s += part_w[(((size_t)bb * H + h) * nblk + k) * (2 * D + 2) + j];
    if (j < 2 * D) dW[(size_t)h * 2 * D + j] = s;
    else db[2 * h + (j - 2 * D)] = s;
  }
}

int gate_tiles(const Problem& pb) { return (pb.N + kGateRows - 1) / kGateRows; }

}  // namespace

size_t gates_bwd_ws_bytes(const Problem& pb) {
  return sizeof(float) * (size_t)pb.B * pb.H * gate_tiles(pb) * (2 * (size_t)pb.d + 2);
}

void launch_gates_fwd(const Problem& pb, const void* Q, const float* W, const float* b, float* gs,
                      float* glr, hipStream_t st) {
  const dim3 grid(gate_tiles(pb), pb.B * pb.H);
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      ELSAA_LAUNCH("gates_fwd", (gates_fwd_kernel<T, D>), grid, dim3(256), 0, st, (const T*)Q, W,
                   b, pb.H, pb.N, gs, glr);
    });
  });
}

void launch_gates_bwd(const Problem& pb, const void* Q, const float* W, const float* gs,
                      const float* glr, const float* dgs, const float* dglr, void* dQ, float* dW,
                      float* db, void* ws, hipStream_t st) {
  const int nblk = gate_tiles(pb);
  const dim3 grid(nblk, pb.B * pb.H);
  float* part = (float*)ws;
  with_T(pb.bf16, [&](auto tp) {
    using T = ELSAA_T(tp);
    with_D(pb.d, [&](auto dc) {
      constexpr int D = ELSAA_C(dc);
      ELSAA_LAUNCH("gates_bwd", (gates_bwd_kernel<T, D>), grid, dim3(256), 0, st, (const T*)Q, W,
                   gs, glr, dgs, dglr, pb.H, pb.N, (T*)dQ, part);
    });
  });
  ELSAA_LAUNCH("gates_reduce", gates_reduce_kernel, dim3(pb.H), dim3(256), 0, st, part, pb.B,
               pb.H, nblk, pb.d, dW, db);
}

}  // namespace elsaa
