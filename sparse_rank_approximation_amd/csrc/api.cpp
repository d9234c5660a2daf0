// api.cpp -- the C ABI of libelsaa (declared in include/elsaa.h): argument
// validation, workspace sizing and kernel dispatch. Nothing here allocates or
// synchronises device memory; every call only enqueues work on the caller's
// stream after all checks have passed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

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
    const long items = p->causal ? (long)ilog2((int)nb) * (nb / 2) + nb : nb;
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
  pb->nA = pb->causal ? p->N / pb->chunk : 1;
  pb->elem = pb->bf16 ? 2 : 4;
  if (lds_need(*pb) > elsaa::kLdsBytes)
    return fail(ELSAA_ERR_UNSUPPORTED,
                "these sizes need %zu bytes of LDS per workgroup in fp32; use bf16 or smaller "
                "block / d_h / lr_tables", lds_need(*pb));
  *empty = (long)p->B * p->H == 0;
  return ELSAA_OK;
}

elsaa_status need(const void* ptr, const char* name) {
  return ptr ? ELSAA_OK : fail(ELSAA_ERR_INVALID_ARG, "%s is NULL", name);
}

#define NEED(x)                                          \
  do {                                                   \
    elsaa_status s_ = need((const void*)(x), #x);        \
    if (s_ != ELSAA_OK) return s_;                       \
  } while (0)

size_t ws_bytes_for(const Problem& pb, int call) {
  switch (call) {
    case ELSAA_CALL_SELECT: return elsaa::select_ws_bytes(pb);
    case ELSAA_CALL_SUMMARY: return elsaa::summary_ws_bytes(pb);
    case ELSAA_CALL_FWD: return elsaa::fwd_ws_bytes(pb);
    case ELSAA_CALL_BWD: return elsaa::bwd_ws_bytes(pb);
    default: return 0;
  }
}

elsaa_status check_ws(const Problem& pb, int call, const void* ws, size_t ws_bytes) {
  const size_t n = ws_bytes_for(pb, call);
  if (ws_bytes < n)
    return fail(ELSAA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, n);
  if (n > 0 && !ws) return fail(ELSAA_ERR_INVALID_ARG, "ws is NULL but %zu bytes are needed", n);
  return ELSAA_OK;
}

elsaa_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ELSAA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err.clear();
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
  if (call < ELSAA_CALL_SELECT || call > ELSAA_CALL_BWD)
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
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal) > 0) { NEED(q_perm); NEED(k_perm); }
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_SELECT, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_select(pb, Q, K, planes_s, q_code, k_code, q_perm, k_perm, ws,
                       (hipStream_t)stream);
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
                       const float* A, const float* z, const float* lambda, const float* g_s,
                       const float* g_lr, void* O, void* O_s, void* O_lr, float* lse_s,
                       float* d_lr, void* ws, size_t ws_bytes, void* stream) {
  PROLOGUE(ELSAA_CALL_FWD);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(V); NEED(planes_lr); NEED(A); NEED(z);
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal) > 0) { NEED(q_perm); NEED(k_perm); }
  NEED(lambda); NEED(O); NEED(O_s); NEED(O_lr); NEED(lse_s); NEED(d_lr);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_FWD, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_fwd(pb, Q, K, V, planes_lr, q_perm, k_perm, A, z, lambda, g_s, g_lr, O, O_s, O_lr,
                    lse_s, d_lr, ws, (hipStream_t)stream);
  return launched();
}

elsaa_status elsaa_bwd(const elsaa_params* p, const void* Q, const void* K, const void* V,
                       const void* dO, const void* O_s, const void* O_lr,
                       const float* planes_lr, const int32_t* q_perm, const int32_t* k_perm,
                       const float* A, const float* z, const float* lse_s, const float* d_lr,
                       const float* lambda, const float* g_s, const float* g_lr, void* dQ,
                       void* dK, void* dV, float* dlambda, float* dg_s, float* dg_lr, void* ws,
                       size_t ws_bytes, void* stream) {
  PROLOGUE(ELSAA_CALL_BWD);
  if (empty) return ELSAA_OK;
  NEED(Q); NEED(K); NEED(V); NEED(dO); NEED(O_s); NEED(O_lr); NEED(planes_lr);
  if (elsaa::perm_stride(pb.N, pb.levels, pb.causal) > 0) { NEED(q_perm); NEED(k_perm); }
  NEED(A); NEED(z); NEED(lse_s); NEED(d_lr); NEED(lambda); NEED(dQ); NEED(dK);
  NEED(dV);
  {
    elsaa_status s_ = check_ws(pb, ELSAA_CALL_BWD, ws, ws_bytes);
    if (s_ != ELSAA_OK) return s_;
  }
  elsaa::launch_bwd(pb, Q, K, V, dO, O_s, O_lr, planes_lr, q_perm, k_perm, A, z, lse_s, d_lr,
                    lambda, g_s, g_lr, dQ, dK, dV, dlambda, dg_s, dg_lr, ws, (hipStream_t)stream);
  return launched();
}

const char* elsaa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
