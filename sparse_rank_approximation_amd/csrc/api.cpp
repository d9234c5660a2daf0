// api.cpp -- the C ABI of libelsaa (declared in include/elsaa.h): argument
// validation, workspace sizing and kernel dispatch. Nothing here allocates or
// synchronises device memory; every call only enqueues work on the caller's
// stream after all checks have passed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "elsaa.h"
#include "launch.hpp"

using elsaa::Problem;

namespace {

thread_local std::string g_err;

elsaa_status fail(elsaa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

bool pow2(long x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(long x) {
  int l = 0;
  while ((1L << l) < x) ++l;
  return l;
}

// LDS each kernel family would need for these parameters (bytes).
size_t lds_need(const Problem& pb) {
  const size_t sums = elsaa::summary_lds_need(pb);
  size_t m = elsaa::fwd_lds_need(pb);
  if (sums > m) m = sums;
  const size_t bwd = elsaa::bwd_lds_need(pb);
  return bwd > m ? bwd : m;
}

// Validates *p and fills *pb. `empty` is set when B * H == 0 (nothing to do).
elsaa_status make_problem(const elsaa_params* p, Problem* pb, bool* empty) {
  if (!p) return fail(ELSAA_ERR_INVALID_ARG, "params is NULL");
  *empty = false;
  if (p->B < 0 || p->H < 0) return fail(ELSAA_ERR_INVALID_ARG, "B and H must be >= 0");
  if (p->dtype != ELSAA_F32 && p->dtype != ELSAA_BF16)
    return fail(ELSAA_ERR_INVALID_ARG, "dtype %d is neither ELSAA_F32 nor ELSAA_BF16", p->dtype);
  if (p->d_h != 32 && p->d_h != 64 && p->d_h != 128)
    return fail(ELSAA_ERR_UNSUPPORTED, "d_h = %d: only 32, 64 and 128 are built", p->d_h);
  if (p->N < 32 || p->N % 32 != 0 || p->N > (1 << 24))
    return fail(ELSAA_ERR_INVALID_ARG, "N = %d must be a multiple of 32 in [32, 2^24]", p->N);
  if (p->block != 16 && p->block != 32 && p->block != 64 && p->block != 128 && p->block != 256)
    return fail(ELSAA_ERR_UNSUPPORTED, "block = %d: only 16, 32, 64, 128, 256 are built", p->block);
  if (p->N % p->block != 0)
    return fail(ELSAA_ERR_INVALID_ARG, "N = %d is not a multiple of block = %d", p->N, p->block);
  if (p->causal != 0 && p->causal != 1)
    return fail(ELSAA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->causal && !pow2(p->N / p->block))
    return fail(ELSAA_ERR_INVALID_ARG, "causal: N / block = %d must be a power of two",
                p->N / p->block);
  if (p->hash_bits < 1 || p->hash_bits > 16)
    return fail(ELSAA_ERR_INVALID_ARG, "hash_bits = %d must be in [1, 16]", p->hash_bits);
  if (p->hash_bits > elsaa::kMaxHashBits)
    return fail(ELSAA_ERR_UNSUPPORTED, "hash_bits = %d: at most %d are built", p->hash_bits,
                elsaa::kMaxHashBits);
  if (p->hash_rounds < 0) return fail(ELSAA_ERR_INVALID_ARG, "hash_rounds must be >= 0");
  if (p->hash_rounds > elsaa::kMaxRounds)
    return fail(ELSAA_ERR_UNSUPPORTED, "hash_rounds = %d: at most %d are built", p->hash_rounds,
                elsaa::kMaxRounds);
  if (p->extra_edges < 0) return fail(ELSAA_ERR_INVALID_ARG, "extra_edges must be >= 0");
  if (p->extra_edges > elsaa::kMaxExtra)
    return fail(ELSAA_ERR_UNSUPPORTED, "extra_edges = %d: at most %d are built", p->extra_edges,
                elsaa::kMaxExtra);
  if ((long)p->N * p->extra_edges > 0x7fffffffL)
    return fail(ELSAA_ERR_INVALID_ARG, "N * extra_edges exceeds 2^31 - 1");
  if (p->lr_tables < 1) return fail(ELSAA_ERR_INVALID_ARG, "lr_tables must be >= 1");
  if (p->lr_tables > elsaa::kMaxTables)
    return fail(ELSAA_ERR_UNSUPPORTED, "lr_tables = %d: at most %d are built", p->lr_tables,
                elsaa::kMaxTables);
  if (p->lr_bits != elsaa::kLrBits)
    return fail(ELSAA_ERR_UNSUPPORTED, "lr_bits = %d: only 4 is built", p->lr_bits);
  if (p->causal && (p->chunk < 32 || p->chunk % 32 != 0 || p->N % p->chunk != 0))
    return fail(ELSAA_ERR_INVALID_ARG, "causal: chunk = %d must be a multiple of 32 dividing N",
                p->chunk);
  if (!(p->tau > 0.0f) || !std::isfinite(p->tau))
    return fail(ELSAA_ERR_INVALID_ARG, "tau must be finite and > 0");
  if (!(p->eps >= 0.0f) || !std::isfinite(p->eps))
    return fail(ELSAA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!(p->scale > 0.0f) || !std::isfinite(p->scale))
    return fail(ELSAA_ERR_INVALID_ARG, "scale must be finite and > 0");
  // Heads index the second launch dimension (at most 65535); the sparse work
  // items of all heads are counted in 32-bit integers.
  if ((long)p->B * p->H > 65535)
    return fail(ELSAA_ERR_INVALID_ARG, "B * H = %ld: at most 65535 heads per call",
                (long)p->B * p->H);
  {
    const long nb = p->N / p->block;
    const long R = p->hash_rounds > 1 ? p->hash_rounds : 1;
    const long items = p->causal ? R * ilog2((int)nb) * (nb / 2) + nb : R * nb;
    if (items * p->B * p->H > 0x7fffffffL)
      return fail(ELSAA_ERR_INVALID_ARG,
                  "B * H * %ld sparse blocks exceeds 2^31 - 1: split the heads over calls", items);
  }

  pb->B = p->B; pb->H = p->H; pb->N = p->N; pb->d = p->d_h;
  pb->bf16 = p->dtype == ELSAA_BF16;
  pb->causal = p->causal != 0;
  pb->s = p->block;
  pb->hash_bits = p->hash_bits;
  pb->L = p->lr_tables;
  pb->r = 16 * p->lr_tables;
  pb->chunk = pb->causal ? p->chunk : p->N;
  pb->tau = p->tau; pb->eps = p->eps; pb->scale = p->scale;
  pb->levels = pb->causal ? ilog2(p->N / p->block) : 1;
  pb->rounds = p->hash_rounds > 1 ? p->hash_rounds : 1;
  pb->E = p->extra_edges;
  pb->nA = pb->causal ? p->N / pb->chunk : 1;
  pb->elem = pb->bf16 ? 2 : 4;
  if (lds_need(*pb) > elsaa::kLdsBytes)
    return fail(ELSAA_ERR_UNSUPPORTED,
                "these sizes need %zu bytes of LDS per workgroup in fp32; use bf16 or smaller "
                "block / d_h / lr_tables", lds_need(*pb));
  *empty = (long)p->B * p->H == 0;
  return ELSAA_OK;
}

// A pointer the kernels read or write with 16-byte vector accesses: NULL is an
// error for a required one (optional ones may be NULL), and any that is given
// must be 16-byte aligned.
elsaa_status need(const void* ptr, const char* name, bool required) {
  if (!ptr) return required ? fail(ELSAA_ERR_INVALID_ARG, "%s is NULL", name) : ELSAA_OK;
  if (reinterpret_cast<uintptr_t>(ptr) & 15u)
    return fail(ELSAA_ERR_INVALID_ARG, "%s = %p is not 16-byte aligned", name, ptr);
  return ELSAA_OK;
}

#define NEED(x)                                                \
  do {                                                         \
    elsaa_status s_ = need((const void*)(x), #x, true);        \
    if (s_ != ELSAA_OK) return s_;                             \
  } while (0)
#define OPTIONAL(x)                                            \
  do {                                                         \
    elsaa_status s_ = need((const void*)(x), #x, false);       \
    if (s_ != ELSAA_OK) return s_;                             \
  } while (0)

size_t ws_bytes_for(const Problem& pb, int call) {
  switch (call) {
    case ELSAA_CALL_SELECT: return elsaa::select_ws_bytes(pb);
    case ELSAA_CALL_SUMMARY: return elsaa::summary_ws_bytes(pb);
    case ELSAA_CALL_FWD: return elsaa::fwd_ws_bytes(pb);
    case ELSAA_CALL_BWD: return elsaa::bwd_ws_bytes(pb);
    case ELSAA_CALL_GATES_BWD: return elsaa::gates_bwd_ws_bytes(pb);
    case ELSAA_CALL_CHECK: return elsaa::check_ws_bytes(pb);
    case ELSAA_CALL_TOPK: return elsaa::topk_ws_bytes(pb);
    default: return 0;
  }
}

elsaa_status check_ws(const Problem& pb, int call, const void* ws, size_t ws_bytes) {
  const size_t n = ws_bytes_for(pb, call);
  if (ws_bytes < n)
    return fail(ELSAA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, n);
  if (n > 0 && !ws) return fail(ELSAA_ERR_INVALID_ARG, "ws is NULL but %zu bytes are needed", n);
  return need(ws, "ws", false);
}

elsaa_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ELSAA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err.clear();
  return ELSAA_OK;
}

// Debug mode (ELSAA_CHECK_ORDERS=1): check the orders on the stream, wait, and
// fail the call if any head's are invalid. The workspace of elsaa_fwd / elsaa_bwd
// (at least the partial slots, B H N (d_h e + 4) bytes) holds the counts and the
// per-token counters.
elsaa_status debug_check_orders(const Problem& pb, const int32_t* qperm, const int32_t* kperm,
                                void* ws, hipStream_t st) {
  const char* e = getenv("ELSAA_CHECK_ORDERS");
  if (!e || e[0] != '1' || elsaa::perm_stride(pb.N, pb.levels, pb.causal, pb.rounds) == 0)
    return ELSAA_OK;
  const size_t BH = (size_t)pb.B * pb.H;
  int32_t* bad = (int32_t*)ws;
  int32_t* mark = (int32_t*)((char*)ws + ((BH * sizeof(int32_t) + 255) & ~(size_t)255));
  elsaa::launch_check_orders(pb, qperm, kperm, bad, mark, st);
  std::vector<int32_t> h(BH);
  hipError_t err = hipMemcpyAsync(h.data(), bad, BH * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  if (err != hipSuccess)
    return fail(ELSAA_ERR_HIP, "order check failed: %s", hipGetErrorString(err));
  for (size_t bh = 0; bh < BH; ++bh)
    if (h[bh] != 0)
      return fail(ELSAA_ERR_INVALID_ARG,
                  "q_perm / k_perm of head %zu (b %zu, h %zu) break the order layout: %d "
                  "violations (ELSAA_CHECK_ORDERS)",
                  bh, bh / pb.H, bh % pb.H, h[bh]);
  return ELSAA_OK;
}

// Debug mode (ELSAA_CHECK_FINITE=1): count the NaN / infinite entries of the
// input tensors on the stream, wait, and fail the call if there are any.
elsaa_status debug_check_finite(const Problem& pb, const void* const* xs, const char* const* names,
                                int nx, void* ws, hipStream_t st) {
  const char* e = getenv("ELSAA_CHECK_FINITE");
  if (!e || e[0] != '1') return ELSAA_OK;
  int32_t* counts = (int32_t*)ws;
  elsaa::launch_finite_count(pb, xs, nx, counts, st);
  std::vector<int32_t> h(nx);
  hipError_t err = hipMemcpyAsync(h.data(), counts, nx * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  if (err != hipSuccess)
    return fail(ELSAA_ERR_HIP, "finite check failed: %s", hipGetErrorString(err));
  for (int i = 0; i < nx; ++i)
    if (h[i] != 0)
      return fail(ELSAA_ERR_INVALID_ARG, "%s holds %d NaN or infinite entries (ELSAA_CHECK_FINITE)",
                  names[i], h[i]);
  return ELSAA_OK;
}

#define PROLOGUE(call)                                   \
  Problem pb;                                            \
  bool empty;                                            \
  {                                                      \
    elsaa_status s_ = make_problem(p, &pb, &empty);      \
    if (s_ != ELSAA_OK) return s_;                       \
  }

}  // namespace

extern "C" {

elsaa_status elsaa_workspace_size(const elsaa_params* p, int32_t call, size_t* bytes) {
  if (!bytes) return fail(ELSAA_ERR_INVALID_ARG, "bytes is NULL");
  if (call < ELSAA_CALL_SELECT || call > ELSAA_CALL_TOPK)
    return fail(ELSAA_ERR_INVALID_ARG, "unknown call %d", call);
  PROLOGUE(call);
  *bytes = empty ? 0 : ws_bytes_for(pb, call);
  return ELSAA_OK;
}

elsaa_status elsaa_select(const elsaa_params* p, const void* Q, const void* K,
                          const float* planes_s, uint16_t* q_code, uint16_t* k_code,
                          int32_t* q_perm, int32_t* k_perm, void* ws, size_t ws_bytes,
                          void* stream) {
  PROLOGUE(ELSAA_CALL_SELECT);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(planes_s); NEED(q_code); NEED(k_code);
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal, pb.rounds) > 0) { NEED(q_perm); NEED(k_perm); }
  OPTIONAL(q_perm); OPTIONAL(k_perm);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_SELECT, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_select(pb, Q, K, planes_s, q_code, k_code, q_perm, k_perm, ws,
                       (hipStream_t)stream);
  return launched();
}

elsaa_status elsaa_select_noalloc(const elsaa_params* p, const void* Q, const void* K,
                                  const float* planes_s, uint16_t* q_code, uint16_t* k_code,
                                  int32_t* q_perm, int32_t* k_perm, void* stream) {
  PROLOGUE(ELSAA_CALL_SELECT);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(planes_s); NEED(q_code); NEED(k_code);
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal, pb.rounds) > 0) { NEED(q_perm); NEED(k_perm); }
  OPTIONAL(q_perm); OPTIONAL(k_perm);
  const size_t n = elsaa::select_ws_bytes(pb), cap = elsaa::noalloc_scratch_bytes();
  if (n > cap)
    return fail(ELSAA_ERR_UNSUPPORTED,
                "the allocation-free selection holds at most %zu bytes of scratch; these sizes "
                "need %zu (8 * H * hash_bits * d_h): use elsaa_select with a workspace",
                cap, n);
  void* scr = nullptr;
  const hipError_t e = elsaa::noalloc_scratch(&scr);
  if (e != hipSuccess)
    return fail(ELSAA_ERR_HIP, "device address of the fixed scratch: %s", hipGetErrorString(e));
  elsaa::prof_suspend(true);  // (the diagnostics would create events)
  elsaa::launch_select(pb, Q, K, planes_s, q_code, k_code, q_perm, k_perm, scr,
                       (hipStream_t)stream);
  elsaa::prof_suspend(false);
  return launched();
}

elsaa_status elsaa_lowrank_summary(const elsaa_params* p, const void* K, const void* V,
                                   const float* planes_lr, float* A, float* z, void* ws,
                                   size_t ws_bytes, void* stream) {
  PROLOGUE(ELSAA_CALL_SUMMARY);
  if (empty) return ELSAA_OK;
  NEED(K); NEED(V); NEED(planes_lr); NEED(A); NEED(z);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_SUMMARY, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_summary(pb, K, V, planes_lr, A, z, ws, (hipStream_t)stream);
  return launched();
}

elsaa_status elsaa_fwd(const elsaa_params* p, const void* Q, const void* K, const void* V,
                       const float* planes_lr, const int32_t* q_perm, const int32_t* k_perm,
                       const int32_t* extra_idx, const float* A, const float* z,
                       const float* lambda, const float* g_s, const float* g_lr, void* O,
                       float* O_s, void* O_lr, float* lse_s, float* d_lr, void* ws,
                       size_t ws_bytes, void* stream) {
  PROLOGUE(ELSAA_CALL_FWD);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(V); NEED(planes_lr); NEED(A); NEED(z);
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal, pb.rounds) > 0) { NEED(q_perm); NEED(k_perm); }
  OPTIONAL(q_perm); OPTIONAL(k_perm);
  if (pb.E > 0) NEED(extra_idx);
  OPTIONAL(extra_idx);
  NEED(lambda); OPTIONAL(g_s); OPTIONAL(g_lr);
  NEED(O); NEED(O_s); NEED(O_lr); NEED(lse_s); NEED(d_lr);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_FWD, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  if (!elsaa::launch_fwd(pb, Q, K, V, planes_lr, q_perm, k_perm, A, z, lambda, g_s, g_lr,
                         extra_idx, O, O_s, O_lr, lse_s, d_lr, ws, (hipStream_t)stream, true))
    return fail(ELSAA_ERR_UNSUPPORTED, "no forward kernel variant is built for these sizes");
  {
    elsaa_status s_ = debug_check_orders(pb, q_perm, k_perm, ws, (hipStream_t)stream);
    if (s_ != ELSAA_OK) return s_;
    const void* xs[3] = {Q, K, V};
    const char* names[3] = {"Q", "K", "V"};
    s_ = debug_check_finite(pb, xs, names, 3, ws, (hipStream_t)stream);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_fwd(pb, Q, K, V, planes_lr, q_perm, k_perm, A, z, lambda, g_s, g_lr, extra_idx, O,
                    O_s, O_lr, lse_s, d_lr, ws, (hipStream_t)stream, false);
  return launched();
}

elsaa_status elsaa_fwd_fused(const elsaa_params* p, const void* Q, const void* K, const void* V,
                             const float* planes_s, const float* planes_lr, const float* lambda,
                             const float* g_s, const float* g_lr, uint16_t* q_code,
                             uint16_t* k_code, int32_t* q_perm, int32_t* k_perm, float* A,
                             float* z, void* O, float* O_s, void* O_lr, float* lse_s,
                             float* d_lr, void* stream) {
  PROLOGUE(ELSAA_CALL_FWD);
  if (!elsaa::fused_fwd_supported(pb))
    return fail(ELSAA_ERR_UNSUPPORTED,
                "the fused forward takes non-causal problems with one hash round, no extra "
                "edges, hash_bits <= 10, block <= 128, N <= 65536 and %zu bytes of LDS per "
                "workgroup (these need %zu)",
                (size_t)elsaa::kLdsBytes, elsaa::fused_fwd_lds(pb));
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(V); NEED(planes_s); NEED(planes_lr); NEED(lambda);
  OPTIONAL(g_s); OPTIONAL(g_lr);
  NEED(q_code); NEED(k_code); NEED(q_perm); NEED(k_perm); NEED(A); NEED(z);
  NEED(O); NEED(O_s); NEED(O_lr); NEED(lse_s); NEED(d_lr);
  {
    // (the debug count goes to the first words of O_s, which the kernel overwrites)
    const void* xs[3] = {Q, K, V};
    const char* names[3] = {"Q", "K", "V"};
    elsaa_status s_ = debug_check_finite(pb, xs, names, 3, O_s, (hipStream_t)stream);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_fused_fwd(pb, Q, K, V, planes_s, planes_lr, lambda, g_s, g_lr, q_code, k_code,
                          q_perm, k_perm, A, z, O, O_s, O_lr, lse_s, d_lr, (hipStream_t)stream);
  return launched();
}

elsaa_status elsaa_bwd(const elsaa_params* p, const void* Q, const void* K, const void* V,
                       const void* dO, const float* O_s, const void* O_lr,
                       const float* planes_lr, const int32_t* q_perm, const int32_t* k_perm,
                       const int32_t* extra_idx, const float* A, const float* z,
                       const float* lse_s, const float* d_lr, const float* lambda,
                       const float* g_s, const float* g_lr, void* dQ,
                       void* dK, void* dV, float* dlambda, float* dg_s, float* dg_lr, void* ws,
                       size_t ws_bytes, void* stream) {
  PROLOGUE(ELSAA_CALL_BWD);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(V); NEED(dO); NEED(O_s); NEED(O_lr); NEED(planes_lr);
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal, pb.rounds) > 0) { NEED(q_perm); NEED(k_perm); }
  OPTIONAL(q_perm); OPTIONAL(k_perm);
  if (pb.E > 0) NEED(extra_idx);
  OPTIONAL(extra_idx);
  NEED(A); NEED(z); NEED(lse_s); NEED(d_lr); NEED(lambda); OPTIONAL(g_s); OPTIONAL(g_lr);
  NEED(dQ); NEED(dK); NEED(dV); OPTIONAL(dlambda); OPTIONAL(dg_s); OPTIONAL(dg_lr);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_BWD, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  if (!elsaa::launch_bwd(pb, Q, K, V, dO, O_s, O_lr, planes_lr, q_perm, k_perm, A, z, lse_s, d_lr,
                         lambda, g_s, g_lr, extra_idx, dQ, dK, dV, dlambda, dg_s, dg_lr, ws,
                         (hipStream_t)stream, true))
    return fail(ELSAA_ERR_UNSUPPORTED, "no backward kernel variant is built for these sizes");
  {
    elsaa_status s_ = debug_check_orders(pb, q_perm, k_perm, ws, (hipStream_t)stream);
    if (s_ != ELSAA_OK) return s_;
    const void* xs[4] = {Q, K, V, dO};
    const char* names[4] = {"Q", "K", "V", "dO"};
    s_ = debug_check_finite(pb, xs, names, 4, ws, (hipStream_t)stream);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_bwd(pb, Q, K, V, dO, O_s, O_lr, planes_lr, q_perm, k_perm, A, z, lse_s, d_lr,
                    lambda, g_s, g_lr, extra_idx, dQ, dK, dV, dlambda, dg_s, dg_lr, ws,
                    (hipStream_t)stream, false);
  return launched();
}

elsaa_status elsaa_check_orders(const elsaa_params* p, const int32_t* q_perm,
                                const int32_t* k_perm, int32_t* bad, void* ws, size_t ws_bytes,
                                void* stream) {
  PROLOGUE(ELSAA_CALL_CHECK);
  if (empty) return ELSAA_OK;
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal, pb.rounds) > 0) { NEED(q_perm); NEED(k_perm); }
  OPTIONAL(q_perm); OPTIONAL(k_perm);
  NEED(bad);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_CHECK, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_check_orders(pb, q_perm, k_perm, bad, (int32_t*)ws, (hipStream_t)stream);
  return launched();
}

elsaa_status elsaa_topk(const elsaa_params* p, const void* Q, const void* K, int32_t k,
                        int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  PROLOGUE(ELSAA_CALL_TOPK);
  if (k < 1) return fail(ELSAA_ERR_INVALID_ARG, "k = %d must be >= 1", k);
  if (!elsaa::launch_topk(pb, Q, K, k, idx, nullptr, (hipStream_t)stream, true))
    return fail(ELSAA_ERR_UNSUPPORTED, "k = %d: at most 256 keys per query are built", k);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(idx);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_TOPK, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_topk(pb, Q, K, k, idx, ws, (hipStream_t)stream, false);
  return launched();
}

elsaa_status elsaa_gates_fwd(const elsaa_params* p, const void* Q, const float* W,
                             const float* b, float* g_s, float* g_lr, void* stream) {
  PROLOGUE(ELSAA_CALL_GATES_BWD);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(W); NEED(b); NEED(g_s); NEED(g_lr);
  elsaa::launch_gates_fwd(pb, Q, W, b, g_s, g_lr, (hipStream_t)stream);
  return launched();
}

elsaa_status elsaa_gates_bwd(const elsaa_params* p, const void* Q, const float* W,
                             const float* g_s, const float* g_lr, const float* dg_s,
                             const float* dg_lr, void* dQ, float* dW, float* db, void* ws,
                             size_t ws_bytes, void* stream) {
  PROLOGUE(ELSAA_CALL_GATES_BWD);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(W); NEED(g_s); NEED(g_lr); NEED(dg_s); NEED(dg_lr); NEED(dQ); NEED(dW); NEED(db);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_GATES_BWD, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_gates_bwd(pb, Q, W, g_s, g_lr, dg_s, dg_lr, dQ, dW, db, ws, (hipStream_t)stream);
  return launched();
}

const char* elsaa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
