// common.hpp -- device helpers shared by the libelsaa kernels (gfx950 / CDNA4).
//
// Matrix products use the 32x32 MFMA tiles of one 64-lane wavefront:
//   bf16 : v_mfma_f32_32x32x16_bf16 (K step 16, 8 elements per lane)
//   fp32 : v_mfma_f32_32x32x2_f32   (K step 2,  1 element  per lane)
// Operand layout (both types, KPL = elements per lane, h = lane / 32):
//   A[m][k] : lane (m = lane % 32) holds k = KPL*h + e, e < KPL
//   B[k][n] : lane (n = lane % 32) holds k = KPL*h + e
//   D[m][n] : lane (n = lane % 32) holds m = acc_row(v, h), v < 16
// A K step may visit the K index in any order as long as A and B agree; the
// "accperm" helpers below use the order in which D rows sit in a lane, so that a
// D tile (e.g. attention probabilities P^T with keys as rows) can feed the next
// product as its B operand without leaving registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace elsaa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

template <typename T>
struct MF;

template <>
struct MF<__bf16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef bf16x8 frag;
  static __device__ __forceinline__ floatx16 mma(const frag& a, const frag& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const __bf16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (__bf16)0.0f;
    return f;
  }
  // B (or A) fragment from accumulators acc[ks*8 .. ks*8+7].
  static __device__ __forceinline__ frag from_acc(const floatx16& a, int ks) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (__bf16)a[ks * 8 + e];
    return f;
  }
  // Fragment of row[] at the K indices acc_row(ks*8+e, h), e < 8, i.e. the two
  // runs row[16ks + 4h .. +4) and row[16ks + 8 + 4h .. +4).
  static __device__ __forceinline__ frag load_accperm(const __bf16* row, int ks, int h) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 16 * ks + 4 * h);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 * ks + 8 + 4 * h);
    frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[e] = lo[e]; f[4 + e] = hi[e]; }
    return f;
  }
  // Fragment from KPL floats, rounded to bf16.
  static __device__ __forceinline__ frag from_floats(const float* x) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (__bf16)x[e];
    return f;
  }
};

template <>
struct MF<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  static __device__ __forceinline__ floatx16 mma(const frag& a, const frag& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ frag zero() { return 0.0f; }
  static __device__ __forceinline__ frag from_acc(const floatx16& a, int ks) { return a[ks]; }
  static __device__ __forceinline__ frag load_accperm(const float* row, int ks, int h) {
    return row[acc_row(ks, h)];
  }
  static __device__ __forceinline__ frag from_floats(const float* x) { return x[0]; }
};

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

template <typename T>
__device__ __forceinline__ float to_f(T x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f(float x) { return (T)x; }

// Value of the other lane half (lane ^ 32).
__device__ __forceinline__ float swap_half(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Inverse of the reflected binary Gray code (position along the Gray sequence).
__device__ __forceinline__ unsigned gray_rank(unsigned c) {
  c ^= c >> 1;
  c ^= c >> 2;
  c ^= c >> 4;
  c ^= c >> 8;
  return c;
}

// ---------------------------------------------------------------------------
// RACE features of the 32 tokens of one wave (lane % 32 = token, h = lane / 32).
//
// Projections u_p = scale <R_p, x> for p = 4 l + t are evaluated as the D tile
// U^T = R X^T (rows = projections, columns = tokens): a lane then holds, for its
// token, the four projections of tables l = 8 mt + 2 g + h (g < 4) of every
// 32-row projection tile mt. phi_{l,b} = prod_t sigmoid(+-2 u_lt / tau) is formed
// in registers as phi[jp][b] with jp = 4 mt + g, so that table(jp, h) = 2 jp + h.
// Tables >= L are zero. Fragments of X come from `xrow` (the token's row).
// For bf16 the fp32 hyperplanes are split into hi + lo bf16 parts (two products)
// so that u carries about 16 significant bits.
// ---------------------------------------------------------------------------
template <typename T, int D, int LP>  // LP = number of tables rounded up to even
struct Features {
  static constexpr int NPT = (4 * LP + 31) / 32;  // 32-row projection tiles
  static constexpr int NJP = LP / 2;               // table pairs
  float phi[NJP][16];
  float sp[NJP][4], sq[NJP][4];  // sigmoid(+a_t), sigmoid(-a_t), a_t = 2 u_t / tau

  __device__ __forceinline__ void compute(const T* xrow, bool valid, const float* planes,
                                          int L, float scale, float tau, int lane) {
    typedef MF<T> M;
    const int h = lane >> 5, col = lane & 31;
    floatx16 u[NPT];
#pragma unroll
    for (int mt = 0; mt < NPT; ++mt) u[mt] = zero16();
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks) {
      const int k0 = ks * M::KSTEP + M::KPL * h;
      typename M::frag xb = valid ? M::load(xrow + k0) : M::zero();
#pragma unroll
      for (int mt = 0; mt < NPT; ++mt) {
        const int prow = 32 * mt + col;  // projection index of this lane's A row
        float r[M::KPL];
        if (prow < 4 * L) {
#pragma unroll
          for (int e = 0; e < M::KPL; ++e) r[e] = planes[(size_t)prow * D + k0 + e];
        } else {
#pragma unroll
          for (int e = 0; e < M::KPL; ++e) r[e] = 0.0f;
        }
        if constexpr (M::KPL == 1) {
          u[mt] = M::mma(r[0], xb, u[mt]);
        } else {
          float lo[M::KPL];
          typename M::frag hi = M::from_floats(r);
#pragma unroll
          for (int e = 0; e < M::KPL; ++e) lo[e] = r[e] - (float)hi[e];
          u[mt] = M::mma(hi, xb, u[mt]);
          u[mt] = M::mma(M::from_floats(lo), xb, u[mt]);
        }
      }
    }
    const float c2 = 2.0f * scale / tau;
#pragma unroll
    for (int mt = 0; mt < NPT; ++mt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jp = 4 * mt + g;
        if (jp >= NJP) continue;
        const int table = 2 * jp + h;
        float p[4], q[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a = c2 * u[mt][4 * g + t];
          p[t] = sigmoid(a);
          q[t] = sigmoid(-a);
          sp[jp][t] = p[t];
          sq[jp][t] = q[t];
        }
        float lo4[4], hi4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          lo4[b] = ((b & 1) ? p[0] : q[0]) * ((b & 2) ? p[1] : q[1]);
          hi4[b] = ((b & 1) ? p[2] : q[2]) * ((b & 2) ? p[3] : q[3]);
        }
        const bool live = table < L;
#pragma unroll
        for (int b = 0; b < 16; ++b) phi[jp][b] = live ? lo4[b & 3] * hi4[b >> 2] : 0.0f;
      }
    }
  }

  // Feature index of phi[jp][b] for this lane half.
  static __device__ __forceinline__ int feat(int jp, int b, int h) { return 16 * (2 * jp + h) + b; }

  // Fragment of the features for K step ks of a product over the feature axis
  // (KPL features per lane half): half h supplies features 16 (2 jp + h) + b0 + e.
  __device__ __forceinline__ typename MF<T>::frag frag(int ks) const {
    typedef MF<T> M;
    constexpr int SPJ = 16 / M::KPL;  // K steps per table pair
    const int jp = ks / SPJ, b0 = (ks % SPJ) * M::KPL;
    float x[M::KPL];
#pragma unroll
    for (int e = 0; e < M::KPL; ++e) x[e] = phi[jp][b0 + e];
    return M::from_floats(x);
  }
  // Backward of phi through a_t = (2 scale / tau) <R_t, x>: given dphi in this
  // lane's layout, da_t = sum_b dphi_b phi_b (bit t of b ? sigmoid(-a_t) : -sigmoid(a_t)).
  __device__ __forceinline__ void backward(const float (&dphi)[NJP][16], float (&da)[NJP][4]) const {
#pragma unroll
    for (int jp = 0; jp < NJP; ++jp)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const float w = dphi[jp][b] * phi[jp][b];
          acc += ((b >> t) & 1) ? w * sq[jp][t] : -w * sp[jp][t];
        }
        da[jp][t] = acc;
      }
  }

  // Feature index that K step ks, element e uses for lane half h.
  static __device__ __forceinline__ int frag_feat(int ks, int e, int h) {
    constexpr int SPJ = 16 / MF<T>::KPL;
    return 16 * (2 * (ks / SPJ) + h) + (ks % SPJ) * MF<T>::KPL + e;
  }
};

// A D tile whose rows are the 32 features of tables (2 jp, 2 jp + 1) and whose
// columns are tokens (lane % 32) holds, in lane half h, rows 8 g + 4 h + t. One
// exchange with the other half leaves lane half h with all 16 buckets of table
// 2 jp + h, the layout of Features::phi[jp].
__device__ __forceinline__ void tile_to_table(const floatx16& acc, int h, float (&out)[16]) {
#pragma unroll
  for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float keep = h ? acc[8 + 4 * g2 + t] : acc[4 * g2 + t];
      const float send = h ? acc[4 * g2 + t] : acc[8 + 4 * g2 + t];
      const float recv = swap_half(send);
      // own rows: b = 8 g2 + 4 h + t; partner rows: b = 8 g2 + 4 (1 - h) + t
      out[8 * g2 + t] = h ? recv : keep;
      out[8 * g2 + 4 + t] = h ? keep : recv;
    }
}

// dX^T (D x 32 tokens, D/32 tiles, columns = lane % 32) = c2 * R^T dA^T, where lane
// half h holds da[jp][t] for table 2 jp + h of its token and R = planes [L][4][D].
// This is the last step of the backward through the RACE features:
// dx = sum_{l,t} da_lt (2 scale / tau) R_lt.
template <typename T, int D, int LP>
__device__ __forceinline__ void features_dx(const float (&da)[LP / 2][4], const float* planes, int L,
                                            float c2, int lane, floatx16 (&dx)[D / 32]) {
  typedef MF<T> M;
  constexpr int NQ = 2 * LP;  // (table, hyperplane) pairs per lane half
  constexpr int NKS = (NQ + M::KPL - 1) / M::KPL;
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dx[dt] = zero16();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    float a[M::KPL], b[M::KPL];
#pragma unroll
    for (int e = 0; e < M::KPL; ++e) {
      const int q = ks * M::KPL + e, jp = q >> 2, t = q & 3;
      b[e] = (q < NQ) ? da[jp < LP / 2 ? jp : 0][t] : 0.0f;
    }
    const typename M::frag bf = M::from_floats(b);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int e = 0; e < M::KPL; ++e) {
        const int q = ks * M::KPL + e, jp = q >> 2, t = q & 3, table = 2 * jp + h;
        a[e] = (q < NQ && table < L) ? planes[(size_t)(4 * table + t) * D + 32 * dt + col] : 0.0f;
      }
      dx[dt] = M::mma(M::from_floats(a), bf, dx[dt]);
    }
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dx[dt][v] *= c2;
}

}  // namespace elsaa
