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

// Index of this wave in its workgroup, as a wave-uniform (scalar register) value:
// branches and loop bounds that depend only on it are then known to be uniform.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
}

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

typedef __bf16 bf16x4_tr __attribute__((ext_vector_type(4)));

// Leading dimension (elements) of row-major LDS tiles with D columns. For bf16 a
// row stride of 12 (mod 64) dwords makes both 16-lane row-fragment reads (lane ->
// row, 16 bytes each) and transposed reads (4 rows x 32 bytes per 16 lanes) free
// of bank conflicts, for D = 32, 64 and 128.
template <typename T>
__host__ __device__ constexpr int tile_ld(int D) { return sizeof(T) == 2 ? D + 24 : D + 8; }

// Fragment whose lanes run over the COLUMNS of a row-major LDS matrix X (leading
// dimension ld, in elements) and whose K elements run over its ROWS: lane
// (n = n0 + lane % 32, half h) receives X[k0 + kofs(e)][n] for e < KPL, with the
// K order of the accumulator rows (accperm: kofs = acc_row(ks * KPL + e, h)) or the
// plain order (kofs = ks * KSTEP + KPL h + e). This is the operand of a product
// that contracts over the rows of X, read without a transposed copy.
//
// bf16 uses ds_read_b64_tr_b16: within each 16-lane group, lane s supplies the
// address of 4 consecutive elements and output lane i, element e receives element
// i % 4 of lane 4 e + (i % 16) / 4's address; pointing lane s at
// X[kb + s / 4][nb + 4 (s % 4)] therefore returns X[kb + e][nb + i % 16] in lane i.
// Two such reads (rows kb .. kb+3 and kb2 .. kb2+3) make the 8 elements.
template <typename T>
__device__ __forceinline__ typename MF<T>::frag tr_frag(const T* X, int ld, int k0, int n0, int ks,
                                                        int lane, bool accperm);

// The bf16 primitive: elements 0..3 from rows kb1 .. kb1 + 3, elements 4..7 from
// rows kb2 .. kb2 + 3 (kb1, kb2 may differ between lane halves).
__device__ __forceinline__ bf16x8 tr_rows(const __bf16* X, int ld, int kb1, int kb2, int n0,
                                          int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int nb = n0 + 16 * (g & 1) + 4 * (s & 3);
  typedef __attribute__((address_space(3))) bf16x4_tr* lds_ptr;
  const bf16x4_tr a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_ptr)(X + (size_t)(kb1 + (s >> 2)) * ld + nb));
  const bf16x4_tr b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_ptr)(X + (size_t)(kb2 + (s >> 2)) * ld + nb));
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[e] = a[e]; f[4 + e] = b[e]; }
  return f;
}
__device__ __forceinline__ float tr_rows(const float* X, int ld, int kb1, int, int n0, int lane) {
  return X[(size_t)kb1 * ld + n0 + (lane & 31)];
}

template <>
__device__ __forceinline__ bf16x8 tr_frag<__bf16>(const __bf16* X, int ld, int k0, int n0, int ks,
                                                  int lane, bool accperm) {
  const int h = lane >> 5;
  const int kb1 = k0 + (accperm ? 16 * ks + 4 * h : 16 * ks + 8 * h);
  return tr_rows(X, ld, kb1, kb1 + (accperm ? 8 : 4), n0, lane);
}

template <>
__device__ __forceinline__ float tr_frag<float>(const float* X, int ld, int k0, int n0, int ks,
                                                int lane, bool accperm) {
  const int h = lane >> 5;
  const int k = k0 + (accperm ? acc_row(ks, h) : 2 * ks + h);
  return X[(size_t)k * ld + n0 + (lane & 31)];
}

// Row fragment from LDS: lane (row r0 + lane % 32, half h) receives
// X[r0 + lane % 32][k0 + ks * KSTEP + KPL h + e], e < KPL.
template <typename T>
__device__ __forceinline__ typename MF<T>::frag row_frag(const T* X, int ld, int r0, int k0, int ks,
                                                         int lane) {
  typedef MF<T> M;
  return M::load(X + (size_t)(r0 + (lane & 31)) * ld + k0 + ks * M::KSTEP + M::KPL * (lane >> 5));
}

// acc + the sum of a fragment's elements, as the product sees them (bf16: four
// v_dot2_f32_bf16 against ones).
template <typename T>
__device__ __forceinline__ float frag_sum(const typename MF<T>::frag& f, float acc);
template <>
__device__ __forceinline__ float frag_sum<__bf16>(const bf16x8& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[2 * e], f[2 * e + 1]}, one, acc, false);
  return acc;
}
template <>
__device__ __forceinline__ float frag_sum<float>(const float& f, float acc) { return acc + f; }

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

// Vector loads / stores of 4 and 8 consecutive elements (8/16 B for bf16,
// 16/32 B for fp32), converted to / from fp32. Pointers must be aligned to the
// access size.
__device__ __forceinline__ void load4(const __bf16* p, float (&x)[4]) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load4(const float* p, float (&x)[4]) {
  const floatx4 v = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = v[e];
}
__device__ __forceinline__ void store4(__bf16* p, const float (&x)[4]) {
  bf16x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (__bf16)x[e];
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, const float (&x)[4]) {
  floatx4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = x[e];
  *reinterpret_cast<floatx4*>(p) = v;
}
// Stores one 32-channel tile of a row held in the MFMA accumulator layout (lane
// half h holds channels 8 g + 4 h .. 8 g + 4 h + 3 of group g = 0..3 as x[4 g ..
// 4 g + 3]) to dst (the tile's first channel). bf16: the lane halves trade 8-byte
// pieces (one v_permlane32_swap per dword) so that each lane stores 16 contiguous
// bytes, half 0 the channels 16 m .. 16 m + 7 and half 1 the next eight (m = 0, 1);
// the two lanes of a pair must be active together. fp32: four 16-byte stores.
template <typename X>
__device__ __forceinline__ void store_tile_row(__bf16* dst, const X& x, int h) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bf16x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = (__bf16)x[8 * m + e];
      b[e] = (__bf16)x[8 * m + 4 + e];
    }
    const uint2 au = *reinterpret_cast<const uint2*>(&a);
    const uint2 bu = *reinterpret_cast<const uint2*>(&b);
    const auto s0 = __builtin_amdgcn_permlane32_swap(au.x, bu.x, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(au.y, bu.y, false, false);
    *reinterpret_cast<uint4*>(dst + 16 * m + 8 * h) = uint4{s0[0], s1[0], s0[1], s1[1]};
  }
}
template <typename X>
__device__ __forceinline__ void store_tile_row(float* dst, const X& x, int h) {
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<floatx4*>(dst + 8 * g + 4 * h) =
        floatx4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
}
__device__ __forceinline__ void load8(const __bf16* p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}
__device__ __forceinline__ void store8(__bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  floatx4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = x[e]; b[e] = x[4 + e]; }
  *reinterpret_cast<floatx4*>(p) = a;
  *reinterpret_cast<floatx4*>(p + 4) = b;
}
// Copy of 8 consecutive elements.
__device__ __forceinline__ void copy8(__bf16* d, const __bf16* s) {
  *reinterpret_cast<bf16x8*>(d) = *reinterpret_cast<const bf16x8*>(s);
}
__device__ __forceinline__ void copy8(float* d, const float* s) {
  *reinterpret_cast<floatx4*>(d) = *reinterpret_cast<const floatx4*>(s);
  *reinterpret_cast<floatx4*>(d + 4) = *reinterpret_cast<const floatx4*>(s + 4);
}

// 8 consecutive elements held in registers (16 B for bf16, 32 B for fp32).
template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
  }
  __device__ __forceinline__ void scale(float c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] * c);
  }
  __device__ __forceinline__ void store(__bf16* p) const { *reinterpret_cast<bf16x8*>(p) = v; }
  // A store of data no kernel reads soon (partial slots, read back by a later
  // pass): marked non-temporal so that it does not displace reused rows in L2.
  __device__ __forceinline__ void store_nt(__bf16* p) const {
    __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
  }
  __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};
template <>
struct Vec8<float> {
  floatx4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const floatx4*>(p);
    b = *reinterpret_cast<const floatx4*>(p + 4);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 4; ++e) { a[e] = 0.0f; b[e] = 0.0f; }
  }
  __device__ __forceinline__ void scale(float c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { a[e] *= c; b[e] *= c; }
  }
  __device__ __forceinline__ void store(float* p) const {
    *reinterpret_cast<floatx4*>(p) = a;
    *reinterpret_cast<floatx4*>(p + 4) = b;
  }
  __device__ __forceinline__ void store_nt(float* p) const {
    __builtin_nontemporal_store(a, reinterpret_cast<floatx4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<floatx4*>(p + 4));
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Gathers ROWS rows of D elements (row r of tensor t taken from
// X[t] + (base + idx[r]) * D, zero when idx[r] < 0, optionally multiplied by
// scale[t][r]) into row-major LDS tiles dst[t] (leading dimension ld) with NT
// threads. Consecutive threads copy consecutive 16-byte pieces of a row, and
// every load of a thread is issued before its first store so that the gather
// costs one memory latency rather than one per row.
template <typename T, int D, int ROWS, int NT, int NX>
__device__ __forceinline__ void gather_rows(T* const (&dst)[NX], int ld, const T* const (&X)[NX],
                                            const float* const (&scale)[NX], const int* idx,
                                            size_t base, int tid) {
  constexpr int CH = D / 8, TOT = ROWS * CH, IT = (TOT + NT - 1) / NT;
  Vec8<T> buf[NX][IT];
  bool ok[IT];
  // Every load is issued unconditionally (a missing row reads row 0 of the
  // block's tensor in its place and is zeroed when stored), so that no load has
  // to complete before the next one is issued.
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int it = tid + i * NT;
    const int r = it / CH, c8 = (it % CH) * 8;
    const int j = idx[r < ROWS ? r : ROWS - 1];
    ok[i] = it < TOT && j >= 0;
#pragma unroll
    for (int x = 0; x < NX; ++x) buf[x][i].load(X[x] + (base + (j > 0 ? j : 0)) * D + c8);
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int it = tid + i * NT;
    if (it < TOT) {
      const int r = it / CH, c8 = (it % CH) * 8;
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        if (!ok[i]) buf[x][i].zero();
        if (scale[x]) buf[x][i].scale(scale[x][r]);
        buf[x][i].store(dst[x] + (size_t)r * ld + c8);
      }
    }
  }
}

// x of lane l % 32 (lo) and of lane l % 32 + 32 (hi), for every lane l, with one
// v_permlane32_swap (a VALU operation: no LDS round trip).
struct HalfPair {
  float lo, hi;
};
__device__ __forceinline__ HalfPair half_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Value of the other lane half (lane ^ 32).
__device__ __forceinline__ float swap_half(float x) {
  const HalfPair p = half_pair(x);
  return (threadIdx.x & 32) ? p.lo : p.hi;
}
// x + swap_half(x) and max(x, swap_half(x)), the same in both halves.
__device__ __forceinline__ float sum_halves(float x) {
  const HalfPair p = half_pair(x);
  return p.lo + p.hi;
}
__device__ __forceinline__ float max_halves(float x) {
  const HalfPair p = half_pair(x);
  return fmaxf(p.lo, p.hi);
}

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// sigmoid(a) and sigmoid(-a) from one exponential and one reciprocal: with
// t = exp(-|a|) in (0, 1], sigmoid(|a|) = 1 / (1 + t) and sigmoid(-|a|) =
// t / (1 + t) (no cancellation for either, no overflow); v_rcp_f32 is within
// 1 ulp of 1 / (1 + t) on (1, 2].
__device__ __forceinline__ void sigmoid_pair(float a, float& p, float& q) {
  const float t = __expf(-fabsf(a));
  const float s = __builtin_amdgcn_rcpf(1.0f + t);
  const float r = t * s;
  p = a >= 0.0f ? s : r;
  q = a >= 0.0f ? r : s;
}

// Inverse of the reflected binary Gray code (position along the Gray sequence).
__device__ __forceinline__ unsigned gray_rank(unsigned c) {
  c ^= c >> 1;
  c ^= c >> 2;
  c ^= c >> 4;
  c ^= c >> 8;
  return c;
}

// Row fragments of one token row in global memory (B operand of a product over
// the row's D elements; lane half h holds elements ks * KSTEP + KPL h + e).
// Invalid rows give zero fragments (x is not read for them).
template <typename T, int D>
__device__ __forceinline__ void load_row_frags(const T* x, bool valid,
                                               typename MF<T>::frag (&f)[D / MF<T>::KSTEP], int h) {
  typedef MF<T> M;
#pragma unroll
  for (int ks = 0; ks < D / M::KSTEP; ++ks)
    f[ks] = valid ? M::load(x + ks * M::KSTEP + M::KPL * h) : M::zero();
}

// The same row fragments, always read (x must point to a readable row). Nothing
// here depends on the loaded values, so the loads stay in flight until the
// fragments are used; a caller that loads a stand-in row for a token that does not
// exist must keep it from mattering where it is used.
template <typename T, int D>
__device__ __forceinline__ void prefetch_row_frags(const T* x,
                                                   typename MF<T>::frag (&f)[D / MF<T>::KSTEP],
                                                   int h) {
  typedef MF<T> M;
#pragma unroll
  for (int ks = 0; ks < D / M::KSTEP; ++ks) f[ks] = M::load(x + ks * M::KSTEP + M::KPL * h);
}

// The part of one token row that a lane holds in the accumulator layout of
// D x 32 tiles whose columns are tokens: channels 32 dt + 8 g + 4 h + e for the
// NDT tiles dt0 .. dt0 + NDT - 1 (dt0 = 0 unless given). load() issues the loads;
// unpack() (once they are needed) gives the values as x[dt][g][e]. bf16: each lane
// loads 16 contiguous bytes (half 0 the channels 16 m .. 16 m + 7 of a tile, half
// 1 the next eight, m = 0, 1) and unpack() trades 8-byte pieces between the lane
// halves (v_permlane32_swap), so the two lanes of a token must unpack together.
template <typename T, int NDT>
struct DRow;
template <int NDT>
struct DRow<__bf16, NDT> {
  uint4 raw[NDT][2];
  __device__ __forceinline__ void load(const __bf16* row, int h, int dt0 = 0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        raw[dt][m] = *reinterpret_cast<const uint4*>(row + 32 * (dt0 + dt) + 16 * m + 8 * h);
  }
  __device__ __forceinline__ void unpack(float (&x)[NDT][4][4]) const {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // half 0 holds (A0, A1), half 1 (B0, B1); groups 2 m and 2 m + 1 want
        // (A0 | A1) and (B0 | B1) split by half.
        const uint4 u = raw[dt][m];
        const auto s0 = __builtin_amdgcn_permlane32_swap(u.x, u.z, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(u.y, u.w, false, false);
        const uint32_t g0[2] = {s0[0], s1[0]}, g1[2] = {s0[1], s1[1]};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          x[dt][2 * m][2 * e] = __uint_as_float(g0[e] << 16);
          x[dt][2 * m][2 * e + 1] = __uint_as_float(g0[e] & 0xffff0000u);
          x[dt][2 * m + 1][2 * e] = __uint_as_float(g1[e] << 16);
          x[dt][2 * m + 1][2 * e + 1] = __uint_as_float(g1[e] & 0xffff0000u);
        }
      }
  }
};
template <int NDT>
struct DRow<float, NDT> {
  floatx4 raw[NDT][4];
  __device__ __forceinline__ void load(const float* row, int h, int dt0 = 0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        raw[dt][g] = *reinterpret_cast<const floatx4*>(row + 32 * (dt0 + dt) + 8 * g + 4 * h);
  }
  __device__ __forceinline__ void unpack(float (&x)[NDT][4][4]) const {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[dt][g][e] = raw[dt][g][e];
  }
};

// Partial-result slots of one token (see partial_slots): its own slot (the causal
// leaf block, or its first round's block) and then, causal, the slot of round r's
// level l for every round and every level at which the token lies in a future
// half of a segment (QUERY) or in a past half (!QUERY); non-causal, its block of
// every further round. next() hands them out in batches so that a batch of row
// loads can be in flight together.
template <bool QUERY>
struct SlotWalk {
  int tok, N, levels, total, logN, c;  // total: rounds x levels (causal), rounds - 1
  bool own, causal;
  __device__ __forceinline__ SlotWalk(int tok_, int N_, int levels_, bool causal_, int rounds = 1)
      : tok(tok_), N(N_), levels(levels_),
        total(causal_ ? rounds * levels_ : rounds - 1), logN(31 - __clz(N_)), c(0), own(true),
        causal(causal_) {}
  __device__ __forceinline__ bool member(int lv) const {
    return (((tok >> (logN - 1 - lv)) & 1) != 0) == QUERY;
  }
  // (N is a power of two whenever there are levels: masks instead of divisions.)
  __device__ __forceinline__ size_t slot(int cc, int lv) const {
    if (!causal) return (size_t)(cc + 1) * N + tok;
    const int n = N >> lv;
    const int s = ((tok & -n) >> 1) + (tok & (n - 1)) - (QUERY ? n >> 1 : 0);
    return (size_t)N + (size_t)cc * (N / 2) + s;
  }
  // Fills sl[0 .. n) with the next n <= KB slots; returns n (0 when done).
  template <int KB>
  __device__ __forceinline__ int next(size_t (&sl)[KB]) {
    int n = 0;
    if (own) {
      sl[0] = (size_t)tok;
      n = 1;
      own = false;
    }
    for (; c < total && n < KB; ++c) {
      const int lv = causal ? c % levels : 0;
      if (!causal || member(lv)) {
        const size_t x = slot(c, lv);
#pragma unroll
        for (int j = 0; j < KB; ++j)
          if (j == n) sl[j] = x;
        ++n;
      }
    }
    return n;
  }
};

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
  float sp[NJP][4];  // sigmoid(a_t), a_t = 2 u_t / tau

  __device__ __forceinline__ void compute(const T* xrow, bool valid, const float* planes,
                                          int L, float scale, float tau, int lane) {
    typename MF<T>::frag xb[D / MF<T>::KSTEP];
    load_row_frags<T, D>(xrow, valid, xb, lane >> 5);
    compute(xb, planes, L, scale, tau, lane);
  }
  // Projection tiles U^T = R X^T of this lane's token, from fp32 hyperplanes in
  // memory (bf16: split into hi + lo parts on the fly).
  static __device__ __forceinline__ void project(const typename MF<T>::frag (&xf)[D / MF<T>::KSTEP],
                                                 const float* planes, int L, int lane,
                                                 floatx16 (&u)[NPT]) {
    typedef MF<T> M;
    const int h = lane >> 5, col = lane & 31;
#pragma unroll
    for (int mt = 0; mt < NPT; ++mt) u[mt] = zero16();
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks) {
      const int k0 = ks * M::KSTEP + M::KPL * h;
      const typename M::frag xb = xf[ks];
#pragma unroll
      for (int mt = 0; mt < NPT; ++mt) {
        const int prow = 32 * mt + col;  // projection index of this lane's A row
        float r[M::KPL];
        if (prow < 4 * L) {
          if constexpr (M::KPL == 8) {
            load8(planes + (size_t)prow * D + k0, r);
          } else {
#pragma unroll
            for (int e = 0; e < M::KPL; ++e) r[e] = planes[(size_t)prow * D + k0 + e];
          }
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
  }
  // The same from the hyperplanes staged in LDS by stage_planes (PL unused for fp32).
  static __device__ __forceinline__ void project(const typename MF<T>::frag (&xf)[D / MF<T>::KSTEP],
                                                 const T* PH, const T* PL, int ldp, int lane,
                                                 floatx16 (&u)[NPT]) {
    typedef MF<T> M;
#pragma unroll
    for (int mt = 0; mt < NPT; ++mt) u[mt] = zero16();
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks)
#pragma unroll
      for (int mt = 0; mt < NPT; ++mt) {
        u[mt] = M::mma(row_frag<T>(PH, ldp, 32 * mt, 0, ks, lane), xf[ks], u[mt]);
        if constexpr (M::KPL > 1) u[mt] = M::mma(row_frag<T>(PL, ldp, 32 * mt, 0, ks, lane), xf[ks], u[mt]);
      }
  }

  // Same, from the token's row fragments (zero fragments give zero projections).
  __device__ __forceinline__ void compute(const typename MF<T>::frag (&xf)[D / MF<T>::KSTEP],
                                          const float* planes, int L, float scale, float tau,
                                          int lane) {
    floatx16 u[NPT];
    project(xf, planes, L, lane, u);
    activate(u, L, scale, tau, lane);
  }
  // Same, with the hyperplanes staged in LDS by stage_planes (PL unused for fp32);
  // phi and sp of the table pairs JP0 .. JP0 + NJ - 1 only (the rest are left
  // unset).
  template <int JP0 = 0, int NJ = NJP>
  __device__ __forceinline__ void compute(const typename MF<T>::frag (&xf)[D / MF<T>::KSTEP],
                                          const T* PH, const T* PL, int ldp, int L, float scale,
                                          float tau, int lane) {
    floatx16 u[NPT];
    project(xf, PH, PL, ldp, lane, u);
    activate<JP0, NJ>(u, L, scale, tau, lane);
  }
  // phi of every table for this lane's token (zero when !valid) stored straight
  // into the LDS row dst (features 16 table + b), one table pair at a time so that
  // only 16 feature values are live at once.
  template <int JP0 = 0, int NJ = NJP>
  static __device__ __forceinline__ void compute_to_row(
      const typename MF<T>::frag (&xf)[D / MF<T>::KSTEP], const T* PH, const T* PL, int ldp, int L,
      float scale, float tau, int lane, bool valid, T* dst) {
    floatx16 u[NPT];
    project(xf, PH, PL, ldp, lane, u);
    store_row<JP0, NJ>(u, L, scale, tau, lane, valid, dst);
  }
  // The same with the hyperplanes read from memory.
  template <int JP0 = 0, int NJ = NJP>
  static __device__ __forceinline__ void compute_to_row(
      const typename MF<T>::frag (&xf)[D / MF<T>::KSTEP], const float* planes, int L, float scale,
      float tau, int lane, bool valid, T* dst) {
    floatx16 u[NPT];
    project(xf, planes, L, lane, u);
    store_row<JP0, NJ>(u, L, scale, tau, lane, valid, dst);
  }
  template <int JP0, int NJ>
  static __device__ __forceinline__ void store_row(const floatx16 (&u)[NPT], int L, float scale,
                                                   float tau, int lane, bool valid, T* dst) {
    const int h = lane >> 5;
    const float c2 = 2.0f * scale / tau;
#pragma unroll
    for (int mt = 0; mt < NPT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jp = 4 * mt + g;
        if (jp >= NJP || jp < JP0 || jp >= JP0 + NJ) continue;
        const bool live = valid && 2 * jp + h < L;
        float p[4], q[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a = c2 * u[mt][4 * g + t];
          sigmoid_pair(a, p[t], q[t]);
        }
        // (every product takes p[0] or q[0]: zeroing those zeroes a dead row)
        p[0] = live ? p[0] : 0.0f;
        q[0] = live ? q[0] : 0.0f;
        float lo4[4], hi4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          lo4[b] = ((b & 1) ? p[0] : q[0]) * ((b & 2) ? p[1] : q[1]);
          hi4[b] = ((b & 1) ? p[2] : q[2]) * ((b & 2) ? p[3] : q[3]);
        }
        float x0[8], x1[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          x0[b] = lo4[b & 3] * hi4[b >> 2];
          x1[b] = lo4[(8 + b) & 3] * hi4[(8 + b) >> 2];
        }
        store8(dst + feat(jp, 0, h), x0);
        store8(dst + feat(jp, 8, h), x1);
      }
  }

  // phi from the projection tiles u (rows = projections, columns = tokens), for
  // the table pairs JP0 .. JP0 + NJ - 1.
  template <int JP0 = 0, int NJ = NJP>
  __device__ __forceinline__ void activate(const floatx16 (&u)[NPT], int L, float scale, float tau,
                                           int lane) {
    const int h = lane >> 5;
    const float c2 = 2.0f * scale / tau;
#pragma unroll
    for (int mt = 0; mt < NPT; ++mt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jp = 4 * mt + g;
        if (jp >= NJP || jp < JP0 || jp >= JP0 + NJ) continue;
        const int table = 2 * jp + h;
        float p[4], q[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a = c2 * u[mt][4 * g + t];
          sigmoid_pair(a, p[t], q[t]);
          sp[jp][t] = p[t];
        }
        // (every product takes p[0] or q[0]: zeroing those zeroes a dead table)
        const bool live = table < L;
        p[0] = live ? p[0] : 0.0f;
        q[0] = live ? q[0] : 0.0f;
        float lo4[4], hi4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          lo4[b] = ((b & 1) ? p[0] : q[0]) * ((b & 2) ? p[1] : q[1]);
          hi4[b] = ((b & 1) ? p[2] : q[2]) * ((b & 2) ? p[3] : q[3]);
        }
#pragma unroll
        for (int b = 0; b < 16; ++b) phi[jp][b] = lo4[b & 3] * hi4[b >> 2];
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
  // Backward of phi through a_t = (2 scale / tau) <R_t, x> for table pair jp:
  // with w_b = dphi_b phi_b, d phi_b / d a_t = phi_b ([bit t of b] - sigmoid(a_t)),
  // so da_t = sum_{b with bit t} w_b - sigmoid(a_t) sum_b w_b.
  __device__ __forceinline__ void backward_table(int jp, const float (&dphi)[16],
                                                 float (&da)[4]) const {
    float wsum = 0.0f, s1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const float w = dphi[b] * phi[jp][b];
      wsum += w;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if ((b >> t) & 1) s1[t] += w;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) da[t] = s1[t] - sp[jp][t] * wsum;
  }
  __device__ __forceinline__ void backward(const float (&dphi)[NJP][16], float (&da)[NJP][4]) const {
#pragma unroll
    for (int jp = 0; jp < NJP; ++jp) backward_table(jp, dphi[jp], da[jp]);
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
  (void)h;
  // v_permlane32_swap(x = acc[i], y = acc[8 + i]) trades the upper lanes of x for
  // the lower lanes of y. Lane half 0 then holds its own acc[i] (bucket 8 g2 + t of
  // table 2 jp) and the partner's acc[i] (bucket 8 g2 + 4 + t); lane half 1 holds
  // the partner's acc[8 + i] (bucket 8 g2 + t of table 2 jp + 1) and its own
  // acc[8 + i] (bucket 8 g2 + 4 + t). The same two outputs for both halves, no
  // selects.
#pragma unroll
  for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 4 * g2 + t;
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i]),
                                                      __float_as_uint(acc[8 + i]), false, false);
      out[8 * g2 + t] = __uint_as_float(r[0]);
      out[8 * g2 + 4 + t] = __uint_as_float(r[1]);
    }
}

// dX^T (D x 32 tokens, D/32 tiles, columns = lane % 32) = c2 * R^T dA^T, where lane
// half h holds da[jp][t] for table 2 jp + h of its token. This is the last step of
// the backward through the RACE features: dx = sum_{l,t} da_lt (2 scale / tau) R_lt.
// The K order of the product (projection p = 4 (2 jp + h) + t for element q of
// the lane half, jp = q / 4, t = q % 4) is the accumulator-row order, so the
// hyperplanes are read from RT = R^T ([D][row stride pw] fp32, zero past 4 L) with
// the same two-run pattern as load_accperm.
template <typename T, int D, int LP, typename R, int NDT = D / 32>
__device__ __forceinline__ void features_dx(const float (&da)[LP / 2][4], const R* RT, int pw,
                                            float c2, int lane, floatx16 (&dx)[NDT], int dt0 = 0) {
  typedef MF<T> M;
  constexpr int NQ = 2 * LP;  // (table, hyperplane) pairs per lane half
  constexpr int NKS = (NQ + M::KPL - 1) / M::KPL;
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dx[dt] = zero16();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    float b[M::KPL];
#pragma unroll
    for (int e = 0; e < M::KPL; ++e) {
      const int q = ks * M::KPL + e, jp = q >> 2, t = q & 3;
      b[e] = (q < NQ) ? da[jp < LP / 2 ? jp : 0][t] : 0.0f;
    }
    const typename M::frag bf = M::from_floats(b);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const R* row = RT + (size_t)(32 * (dt0 + dt) + col) * pw;
      float a[M::KPL];
      if constexpr (M::KPL == 8) {
        float lo[4], hi[4];
        load4(row + 16 * ks + 4 * h, lo);
        load4(row + 16 * ks + 8 + 4 * h, hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) { a[e] = lo[e]; a[4 + e] = hi[e]; }
      } else {
        a[0] = (float)row[acc_row(ks, h)];
      }
      dx[dt] = M::mma(M::from_floats(a), bf, dx[dt]);
    }
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dx[dt][v] *= c2;
}

// Row stride of the transposed hyperplanes staged in LDS for features_dx (which
// reads columns up to max(16, 4 LP)); 2 (mod 4) dwords keeps its row reads apart.
template <int LP>
constexpr int rt_lds_width() { return (4 * LP > 16 ? 4 * LP : 16) + 4; }

// RTs[d][p] = RT[d * pw + p] for p < 4 LP, zero beyond (NT threads).
template <typename T, int D, int LP, int NT>
__device__ __forceinline__ void stage_rt(const float* RT, int pw, T* RTs, int tid) {
  constexpr int W = rt_lds_width<LP>();
  for (int i = tid; i < D * W; i += NT) {
    const int d = i / W, p = i % W;
    RTs[i] = from_f<T>(p < 4 * LP ? RT[(size_t)d * pw + p] : 0.0f);
  }
}

// The hyperplanes of LP tables as MFMA A operands in LDS: [projection][channel]
// (row stride tile_ld), bf16 hi and lo parts (hi + lo carries about 16 bits of the
// fp32 value), or fp32 once. Projections past 4 L are zero.
template <typename T, int D, int LP>
struct PlanesLds {
  static constexpr int NP = 32 * ((4 * LP + 31) / 32), LDP = tile_ld<T>(D);
  static constexpr int NPART = sizeof(T) == 2 ? 2 : 1;
  T p[NPART][NP][LDP];
};
template <typename T, int D, int LP, int NT>
__device__ __forceinline__ void stage_planes(const float* planes, int L, PlanesLds<T, D, LP>& P,
                                             int tid) {
  typedef PlanesLds<T, D, LP> PL;
  for (int i = tid; i < PL::NP * D; i += NT) {
    const int p = i / D, d = i % D;
    const float x = p < 4 * L ? planes[(size_t)p * D + d] : 0.0f;
    const T hi = from_f<T>(x);
    P.p[0][p][d] = hi;
    if constexpr (PL::NPART > 1) P.p[1][p][d] = from_f<T>(x - to_f(hi));
  }
}

// Loads the running RACE statistics of a walk (fp32 [channel][feature] rows of
// length r, features f0 .. f0 + RP) into fp32 D tiles st (rows = channels, lanes =
// features; tile w + 4 i of this wave) and their operand copy SF[feature][channel].
template <typename T, int D, int LP, int SPW, int NW = 4>
__device__ __forceinline__ void load_stats(const float* Ac, int r, int f0, int w, int lane,
                                           floatx16 (&st)[SPW], T* SF, int ldd) {
  constexpr int NFT = LP / 2, NST = (D / 32) * NFT;
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int tix = w + NW * i;
    st[i] = zero16();
    if (tix < NST) {
      const int mt = tix / NFT, f = f0 + 32 * (tix % NFT) + col;
      if (f < r)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[i][v] = Ac[(size_t)(32 * mt + acc_row(v, h)) * r + f];
    }
  }
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int tix = w + NW * i;
    if (tix < NST) {
      const int mt = tix / NFT, fl = 32 * (tix % NFT) + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = st[i][4 * g + e];
        store4(SF + (size_t)fl * ldd + 32 * mt + 8 * g + 4 * h, x);
      }
    }
  }
}

// Advances the statistics by one step of STEP tokens: st += X^T F (X: [token]
// [channel], F: [token][feature], both row-major in LDS), rewrites the operand
// copy SF, and adds sum_t wt[t] F[t][f] (wt == nullptr: weights 1) to zr[f]. The
// feature sums are products with a constant-row A operand, formed by the wave that
// owns channel tile 0 of each feature tile; bf16 weights are split into hi + lo
// parts (two products).
template <typename T, int D, int LP, int SPW, int STEP, bool WRITE_SF = true, int NW = 4>
__device__ __forceinline__ void advance_stats(const T* X, int ldd, const T* F, int ldr,
                                              const float* wt, int w, int lane,
                                              floatx16 (&st)[SPW], T* SF, float* zr) {
  typedef MF<T> M;
  constexpr int NFT = LP / 2, NST = (D / 32) * NFT;
  const int h = lane >> 5, col = lane & 31;
  floatx16 zs[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) zs[i] = zero16();
  // K steps outermost (two at a time) with this wave's tiles inside, so that the
  // operand fragments in flight stay few.
#pragma unroll 2
  for (int ks = 0; ks < STEP / M::KSTEP; ++ks) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int tix = w + NW * i;
      if (tix < NST) {
        const int mt = tix / NFT, nt = tix % NFT;
        const typename M::frag fb = tr_frag<T>(F, ldr, 0, 32 * nt, ks, lane, false);
        st[i] = M::mma(tr_frag<T>(X, ldd, 0, 32 * mt, ks, lane, false), fb, st[i]);
        if (mt == 0) {
          float a[M::KPL];
#pragma unroll
          for (int e = 0; e < M::KPL; ++e) a[e] = wt ? wt[ks * M::KSTEP + M::KPL * h + e] : 1.0f;
          const typename M::frag ahi = M::from_floats(a);
          zs[i] = M::mma(ahi, fb, zs[i]);
          if constexpr (M::KPL > 1) {
            if (wt) {
#pragma unroll
              for (int e = 0; e < M::KPL; ++e) a[e] -= (float)ahi[e];
              zs[i] = M::mma(M::from_floats(a), fb, zs[i]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int tix = w + NW * i;
    if (tix < NST) {
      const int mt = tix / NFT, nt = tix % NFT;
      if constexpr (WRITE_SF) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = st[i][4 * g + e];
          store4(SF + (size_t)(32 * nt + col) * ldd + 32 * mt + 8 * g + 4 * h, x);
        }
      }
      if (mt == 0 && h == 0) zr[32 * nt + col] += zs[i][0];
    }
  }
}

}  // namespace elsaa
