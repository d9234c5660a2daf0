// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "common.hpp"

namespace elsaa {

constexpr int kMaxHashBits = 12;
constexpr int kMaxDh = 128;
constexpr int kMaxTables = 16;
constexpr int kLrBits = 4;
constexpr size_t kLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950

constexpr int kMaxLevels = 20;           // log2(N / s) for N <= 2^24, s >= 16
constexpr int kMaxRounds = 4;            // sortLSH hash rounds (tables)
constexpr int kMaxExtra = 64;            // extra edges listed per query

// LDS of the kernels that walk a span of tokens in steps of STEP tokens: one
// step's row-major channel tile (V, or the low-rank output gradient dnum), its
// feature tile (phi of the keys or of the queries), the running RACE statistics
// as an MFMA operand ([feature][channel]), their feature sums and one scalar per
// token of the step.
template <typename T, int D, int LP, int STEP>
struct WalkSmem {
  static constexpr int RP = 16 * LP, LDD = tile_ld<T>(D), LDR = tile_ld<T>(RP);
  T XS[STEP][LDD];
  T FS[STEP][LDR];
  T SF[RP][LDD];
  alignas(16) float zr[RP];
  float dd[STEP];
};

// Largest step (MAXSTEP, halved down to 32) whose LDS, plus EXTRA bytes of the
// kernel's own, fits; 0 if none does.
template <typename T, int D, int LP, int MAXSTEP, size_t EXTRA = 0>
constexpr int walk_step() {
  return (MAXSTEP >= 128 && sizeof(WalkSmem<T, D, LP, 128>) + EXTRA <= kLdsBytes) ? 128
         : (MAXSTEP >= 64 && sizeof(WalkSmem<T, D, LP, 64>) + EXTRA <= kLdsBytes) ? 64
         : sizeof(WalkSmem<T, D, LP, 32>) + EXTRA <= kLdsBytes                    ? 32
                                                                                  : 0;
}

// Validated problem description with derived sizes.
struct Problem {
  int B, H, N, d;
  bool bf16;
  bool causal;
  int s;          // sortLSH block size
  int hash_bits;
  int L;          // RACE tables
  int r;          // features = 16 L
  int chunk;      // causal RACE summary spacing (N when not causal)
  float tau, eps, scale;
  int levels;     // off-diagonal recursion levels (causal), 1 otherwise
  int rounds;     // sortLSH hash rounds (the support is the union of theirs)
  int E;          // extra edges listed per query (0: none)
  int nA;         // summaries per head
  int elem;       // bytes per element of Q/K/V/...
};

// Entries of q_perm / k_perm per head: for every round its orders (causal: one
// per level, N/2 each; otherwise one of N), round-major.
__host__ __device__ inline size_t perm_stride(int N, int levels, bool causal, int rounds = 1) {
  return (size_t)rounds * (causal ? (size_t)levels * (N / 2) : (size_t)N);
}

// Slots of the sparse partial results of one head. Causal: [0, N) the leaf
// blocks, then round r's level l at N + (r levels + l) N/2. Otherwise round r's
// block of each token at r N + token.
__host__ __device__ inline size_t partial_slots(int N, int levels, bool causal, int rounds = 1) {
  return causal ? (size_t)N + (size_t)rounds * levels * (N / 2) : (size_t)rounds * N;
}

// Sparse work items of one head: causal, `levels` off-diagonal levels of
// `per_level` blocks each (level-major), then the N / s leaf blocks; non-causal,
// the N / s blocks of the single sorted order.
//
// Workgroup g of a launch runs on XCD g % 8 (workgroups go round-robin to the
// eight XCDs, each with its own L2). Where every level's block count is a
// multiple of 8, item g is picked so that XCD x takes the x-th eighth of every
// level's blocks and of the leaf blocks: blocks of the levels whose segments are
// at most N / 8 long, and the leaf blocks, then read rows of only the x-th eighth
// of the tokens, which stay in that XCD's L2 from one level to the next.
// Otherwise the order is plain (head-major). Returns the head; `it` is the item.
__host__ __device__ inline int xcd_item(int g, int items, int per_level, int levels, int& it) {
  if (per_level == 0 || (per_level & 7) != 0) {
    it = g % items;
    return g / items;
  }
  const int x = g & 7, k = g >> 3, ipx = items >> 3, lpx = per_level >> 3;
  const int j = k % ipx, nl = levels * lpx;
  it = j < nl ? (j / lpx) * per_level + x * lpx + j % lpx
              : levels * per_level + x * (ipx - nl) + (j - nl);
  return k / ipx;
}

// Tokens per workgroup of the low-rank walks when not causal: the statistics are
// the whole sequence's and stay fixed, so a workgroup walks several steps after
// loading them once; as many steps as keep at least 512 workgroups in the launch.
// Grid of a persistent launch: the workgroups that fit on the device at once
// (at most total), a multiple of 8 when below total so that workgroup g and its
// later items g + G, g + 2G, ... all run on XCD g mod 8.
inline int persistent_grid(const void* kern, int threads, int total) {
  static int cus[64] = {0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  int& n = cus[dev & 63];
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n = 256;
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, 0) != hipSuccess || per < 1)
    per = 1;
  long g = (long)n * per;
  if (g >= total) return total;
  return (int)(g >= 8 ? g & ~7L : g);
}

inline int noncausal_span(int N, int BH, int step) {
  const int steps = (N + step - 1) / step;
  int per = steps * BH / 512;
  per = per < 1 ? 1 : per > steps ? steps : per;
  return per * step;
}

// Compile-time dispatch over the element type, head dimension and padded table
// count (tables are padded to an even power of two; padding tables are zero).
template <typename F>
void with_T(bool bf16, F&& f) {
  if (bf16) f((__bf16*)nullptr);
  else f((float*)nullptr);
}
template <typename F>
void with_D(int d, F&& f) {
  switch (d) {
    case 32: f(std::integral_constant<int, 32>{}); break;
    case 64: f(std::integral_constant<int, 64>{}); break;
    default: f(std::integral_constant<int, 128>{}); break;
  }
}
inline int padded_tables(int L) { return L <= 2 ? 2 : L <= 4 ? 4 : L <= 8 ? 8 : 16; }
template <typename F>
void with_LP(int L, F&& f) {
  switch (padded_tables(L)) {
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    default: f(std::integral_constant<int, 16>{}); break;
  }
}
#define ELSAA_T(tp) std::remove_pointer_t<decltype(tp)>
#define ELSAA_C(c) decltype(c)::value

// Per-kernel timing (prof.cpp): every launch goes through ELSAA_LAUNCH.
// prof_suspend(true) makes this host thread's launches skip it (no events are
// created) until prof_suspend(false).
void prof_begin(hipStream_t st, const char* name);
void prof_end(hipStream_t st);
void prof_suspend(bool on);
#define ELSAA_LAUNCH(name, kern, grid, block, lds, st, ...)        \
  do {                                                             \
    ::elsaa::prof_begin(st, name);                                 \
    hipLaunchKernelGGL(kern, grid, block, lds, st, __VA_ARGS__);   \
    ::elsaa::prof_end(st);                                         \
  } while (0)

size_t select_ws_bytes(const Problem& pb);
// Debug check of the orders (check.hip): per head, the number of entries that
// break the order layout, into bad[B H]; mark: B H N counters of workspace.
size_t check_ws_bytes(const Problem& pb);
void launch_check_orders(const Problem& pb, const int32_t* qperm, const int32_t* kperm,
                         int32_t* bad, int32_t* mark, hipStream_t st);
// The number of NaN and infinite entries of each of nx [B H N d] tensors.
void launch_finite_count(const Problem& pb, const void* const* xs, int nx, int32_t* counts,
                         hipStream_t st);
// Per-token block indices of every (round, level) order (select.hip), used by the
// sparse kernels to count each pair once over several hash rounds, and to keep
// extra edges sortLSH already selects out; bytes of the two arrays (0 with one
// round and no extra edges).
size_t block_ids_bytes(const Problem& pb);
void launch_block_ids(const Problem& pb, const int32_t* qperm, const int32_t* kperm, int32_t* qb,
                      int32_t* kb, hipStream_t st);
// The allocation-free selection's fixed scratch (select.hip): its size, and its
// device address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);
void launch_select(const Problem& pb, const void* Q, const void* K, const float* planes_s,
                   uint16_t* qc, uint16_t* kc, int32_t* qperm, int32_t* kperm, void* ws,
                   hipStream_t st);

// RACE tile sums and their prefix/suffix/total combination (lowrank.hip).
int lr_tile_tokens(const Problem& pb);
int lr_tiles(const Problem& pb);
void run_lr_sums(const Problem& pb, const void* X, const void* Y, const float* alpha,
                 const float* beta, const float* planes, float* S, float* Z, hipStream_t st);
void run_lr_scan(const Problem& pb, const float* S, const float* Z, int mode, float* A, float* z,
                 hipStream_t st);

size_t summary_ws_bytes(const Problem& pb);
size_t summary_lds_need(const Problem& pb);
void launch_summary(const Problem& pb, const void* K, const void* V, const float* planes_lr,
                    float* A, float* z, void* ws, hipStream_t st);

size_t fwd_ws_bytes(const Problem& pb);
size_t fwd_lds_need(const Problem& pb);
// The forward and backward launch sequences. With dry set they launch nothing
// and only report whether every kernel of the sequence has a variant built for
// these sizes (the same compile-time choices as the real launch); they return
// false when one has not.
bool launch_fwd(const Problem& pb, const void* Q, const void* K, const void* V,
                const float* planes_lr, const int32_t* qperm, const int32_t* kperm,
                const float* A, const float* z, const float* lambda, const float* g_s,
                const float* g_lr, const int32_t* extra, void* O, float* O_s, void* O_lr,
                float* lse, float* d_lr, void* ws, hipStream_t st, bool dry);

// Exact per-query top-k selection (topk.hip); dry: report only whether a variant
// is built for k.
size_t topk_ws_bytes(const Problem& pb);
bool launch_topk(const Problem& pb, const void* Q, const void* K, int ktop, int32_t* out,
                 void* ws, hipStream_t st, bool dry);

// Learnable gates of Eq. 4 from a projection of the query (gates.hip).
size_t gates_bwd_ws_bytes(const Problem& pb);
void launch_gates_fwd(const Problem& pb, const void* Q, const float* W, const float* b, float* gs,
                      float* glr, hipStream_t st);
void launch_gates_bwd(const Problem& pb, const void* Q, const float* W, const float* gs,
                      const float* glr, const float* dgs, const float* dglr, void* dQ, float* dW,
                      float* db, void* ws, hipStream_t st);

// Extra edges listed per query (extra.hip). Workspace regions (byte offsets):
// the kept keys per query, the partial rows (forward: output; backward: dQ, dK,
// dV), the forward's log-sum-exps, and the backward's sort buffers and table.
struct ExtraLayout {
  size_t jq, rows, lse, sort[4], table, total;
};
ExtraLayout extra_layout(const Problem& pb, bool bwd);
void launch_extra_prep(const Problem& pb, const int32_t* extra, const int32_t* qbid,
                       const int32_t* kbid, int32_t* jq, int32_t* skey, int32_t* sval,
                       hipStream_t st);
void launch_extra_sort(const Problem& pb, int32_t* const (&buf)[4], int32_t* table,
                       const int32_t** keys, const int32_t** vals, hipStream_t st);
void launch_extra_fwd(const Problem& pb, const void* Q, const void* K, const void* V,
                      const int32_t* jq, void* Ox, float* Lx, hipStream_t st);
void launch_extra_bwd(const Problem& pb, const void* Q, const void* K, const void* V,
                      const void* dO, const float* lse, const float* rc, const float* rD,
                      const int32_t* jq, const int32_t* skey, const int32_t* sval, void* dQx,
                      void* dKx, void* dVx, hipStream_t st);

// Per-token reductions over the sparse partial slots (merge.hip), with the extra
// edges' partial rows (one per token, [B H][N]) when not null.
void launch_merge(const Problem& pb, const void* Opart, const float* Lpart, const void* Ox,
                  const float* Lx, float* O_s, float* lse, hipStream_t st);
void launch_combine(const Problem& pb, const void* dQp, const void* dKp, const void* dVp,
                    const void* dQx, const void* dKx, const void* dVx, void* dQ, void* dK,
                    void* dV, hipStream_t st);

// The non-causal forward in one launch (fused.hip): whether it takes these
// parameters, its LDS per workgroup, and the launch.
size_t fused_fwd_lds(const Problem& pb);
bool fused_fwd_supported(const Problem& pb);
void launch_fused_fwd(const Problem& pb, const void* Q, const void* K, const void* V,
                      const float* planes_s, const float* planes_lr, const float* lambda,
                      const float* g_s, const float* g_lr, uint16_t* qc, uint16_t* kc,
                      int32_t* qperm, int32_t* kperm, float* A, float* z, void* O, float* O_s,
                      void* O_lr, float* lse, float* d_lr, hipStream_t st);

size_t bwd_ws_bytes(const Problem& pb);
size_t bwd_lds_need(const Problem& pb);
bool launch_bwd(const Problem& pb, const void* Q, const void* K, const void* V, const void* dO,
                const float* O_s, const void* O_lr, const float* planes_lr, const int32_t* qperm,
                const int32_t* kperm, const float* A, const float* z, const float* lse,
                const float* d_lr, const float* lambda, const float* g_s, const float* g_lr,
                const int32_t* extra, void* dQ, void* dK, void* dV, float* dlambda, float* dg_s,
                float* dg_lr, void* ws, hipStream_t st, bool dry);

}  // namespace elsaa
