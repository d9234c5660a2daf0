/*
 * elsaa.h -- C ABI of libelsaa, the gfx950 (MI355X) implementation of the ELSAA
 * attention operator of "ELSAA: Efficient Low-Rank and Sparse Attention
 * Approximation for Training Transformers" (Heidari, Rahimi, Moon; arXiv
 * 2607.20214), forward and backward, on one GPU.
 *
 * Section 3 of the paper states the problem: given the per-head query, key and
 * value matrices Q, K, V in R^{N x d_h}, return an approximation of softmax
 * attention without forming the N x N score matrix, as the combination of
 *   - a sparse branch (Section 3.2, sortLSH): exact softmax attention of each query
 *     over the keys of its hash-sorted diagonal block, or, causally, over the union
 *     of the blocks of a past/future divide-and-conquer, merged by log-sum-exp;
 *     it yields O_sparse and d_sparse = exp(lse);
 *   - a low-rank branch (Section 3.1, RACE): keys softly assigned to hypercube
 *     buckets, bucket statistics A = sum_j phi(K_j) V_j^T and z = sum_j phi(K_j)
 *     (causally: prefix sums), read out in normalized ratio form
 *     O_lr,i = phi(Q_i)^T A / phi(Q_i)^T z with d_lr,i = phi(Q_i)^T z;
 *   - the denominator-aware fusion, Eq. 5 and Eq. 4:
 *     m_i = d_sparse,i / (d_sparse,i + lambda d_lr,i + eps),
 *     O_i = g_sparse,i m_i O_sparse,i + g_lr,i O_lr,i.
 *
 * The four calls below are the operator's steps: elsaa_select (hash + sort),
 * elsaa_lowrank_summary (bucket statistics), elsaa_fwd (both branches' outputs
 * and the fusion) and elsaa_bwd (gradients for training).
 *
 * Conventions shared by every call
 *   - Every pointer except `p` and `stream` is a DEVICE pointer, 16-byte aligned,
 *     to a contiguous row-major array owned by the caller. The library allocates,
 *     frees and synchronises nothing; scratch memory comes from `ws`, whose size
 *     elsaa_workspace_size() returns (NULL/0 is fine when that size is 0).
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     kernels on it and return; results are ready when the stream is.
 *   - Tensors shaped [B, H, N, d_h] hold `dtype` elements (fp32 or bf16);
 *     statistics, gates and lambda are fp32.
 *   - Arguments are validated on the host before anything is launched. On any
 *     non-OK status nothing has been enqueued and elsaa_last_error() (per host
 *     thread) describes the problem. A failed launch returns ELSAA_ERR_HIP.
 *   - Results are bitwise reproducible run to run (no floating-point atomics).
 *   - Selections (codes and permutations) are exact: they reproduce, bit for bit,
 *     the fp64 fused-multiply-add sign tests described at elsaa_select.
 */
#ifndef ELSAA_H
#define ELSAA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ELSAA_OK = 0,
  ELSAA_ERR_INVALID_ARG = 1, /* null pointer, inconsistent or out-of-range size   */
  ELSAA_ERR_UNSUPPORTED = 2, /* valid for the method, not built here (e.g. d_h)   */
  ELSAA_ERR_WORKSPACE = 3,   /* ws_bytes smaller than elsaa_workspace_size()      */
  ELSAA_ERR_HIP = 4          /* a kernel launch failed                             */
} elsaa_status;

typedef enum { ELSAA_F32 = 0, ELSAA_BF16 = 1 } elsaa_dtype;

typedef enum {
  ELSAA_CALL_SELECT = 0,
  ELSAA_CALL_SUMMARY = 1,
  ELSAA_CALL_FWD = 2,
  ELSAA_CALL_BWD = 3
} elsaa_call;

/* Problem description.
 *   B, H, N, d_h : batch, heads, tokens, head dimension; d_h in {32, 64, 128};
 *                  N a multiple of 32 up to 2^24; B * H == 0 is a valid empty
 *                  problem; B * H <= 65535, and B * H times the number of sparse
 *                  blocks per head (causal: log2(N/s) * N/(2s) + N/s; otherwise
 *                  N/s) below 2^31 (larger batches are split over calls).
 *   dtype        : element type of Q, K, V, O, dO, dQ, dK, dV (elsaa_dtype).
 *   causal       : 0 = every query may see every key; 1 = key j only for j <= i.
 *   block        : sortLSH block size s in {16, 32, 64, 128, 256}; N % s == 0; when
 *                  causal, N / s must be a power of two. Non-causal, each query
 *                  attends to exactly s keys; causal, query i to
 *                  (i mod s) + 1 + s * popcount(i / s) keys.
 *   hash_bits    : sortLSH hyperplanes per head, 1..12 (2^hash_bits buckets).
 *   lr_tables    : RACE tables L, 1..16; lr_bits: hyperplanes per table, must be 4
 *                  (16 buckets per table, as in the paper's worked example in
 *                  Appendix C.5). The feature count is r = L * 16.
 *   chunk        : causal RACE summary spacing C: a multiple of 32 dividing N.
 *                  elsaa_lowrank_summary stores one summary per
 *                  chunk; elsaa_fwd/elsaa_bwd carry the running statistics inside a
 *                  chunk on chip. Only changes rounding. Ignored when not causal.
 *   tau          : temperature of the soft bucket assignment (> 0).
 *   eps          : the epsilon of Eq. 5 (>= 0).
 *   scale        : score scale, normally 1/sqrt(d_h) (Section 3) (> 0).
 * Derived: levels Lv = log2(N / s) when causal (off-diagonal recursion levels), 1
 * when not; the permutation length P = Lv * N / 2 when causal, N when not; the
 * number of summaries nA = N / C when causal, 1 when not.
 */
typedef struct {
  int32_t B, H, N, d_h;
  int32_t dtype;
  int32_t causal;
  int32_t block;
  int32_t hash_bits;
  int32_t lr_tables, lr_bits;
  int32_t chunk;
  float tau, eps, scale;
} elsaa_params;

/* Bytes of workspace the given call needs for these parameters (written to
 * *bytes). Returns ELSAA_ERR_INVALID_ARG/UNSUPPORTED for parameters the call
 * would reject. */
elsaa_status elsaa_workspace_size(const elsaa_params* p, int32_t call, size_t* bytes);

/* sortLSH selection (Section 3.2: queries and keys are hashed, sorted by hash and
 * grouped into equal-size blocks; query block b pairs with key block b).
 *   Q, K      : [B, H, N, d_h] dtype.
 *   planes_s  : fp32 [H, hash_bits, d_h], the hyperplanes of each head.
 *   q_code, k_code (out): uint16 [B, H, N]. Bit b of a token's code is set iff the
 *               projection of its row x on hyperplane b is > 0, the projection being
 *               the fp64 fused-multiply-add chain acc = fma(x[j], R[b][j], acc) for
 *               j = 0..d_h-1 from acc = +0.0.
 *   q_perm, k_perm (out): int32 [B, H, P]. Tokens are ordered by the position of
 *               their code along the reflected Gray sequence, ties by ascending
 *               token index. Non-causal: one order of all N tokens. Causal: for
 *               level l in [0, Lv) and segment g of n = N >> l tokens starting at
 *               a = g n, entries [l N/2 + g n/2, l N/2 + (g+1) n/2) hold the sorted
 *               future half [a + n/2, a + n) (q_perm) and past half [a, a + n/2)
 *               (k_perm).
 *   ws        : device workspace of elsaa_workspace_size(p, ELSAA_CALL_SELECT) bytes
 *               (the hyperplanes widened to fp64).
 */
elsaa_status elsaa_select(const elsaa_params* p, const void* Q, const void* K,
                          const float* planes_s, uint16_t* q_code, uint16_t* k_code,
                          int32_t* q_perm, int32_t* k_perm, void* ws, size_t ws_bytes,
                          void* stream);

/* RACE bucket statistics (Section 3.1: each table softly assigns keys to hypercube
 * buckets and accumulates key/value statistics in them). With
 * u_lt(x) = scale <R_lt, x> and phi_{l,b}(x) = prod_t sigmoid(2 s_bt u_lt(x) / tau),
 * s_bt = +1 if bit t of b is set else -1 (the softmax over the 16 vertices of the
 * hypercube of <v_b, u_l> / tau), feature f = 16 l + b:
 *   planes_lr : fp32 [H, lr_tables, 4, d_h].
 *   A (out)   : fp32 [B, H, nA, d_h, r], A[c][e][f] = sum_{j in J_c} phi_f(K_j) V_j[e]
 *               (value channel e major, feature f minor).
 *   z (out)   : fp32 [B, H, nA, r],      z[c][f]    = sum_{j in J_c} phi_f(K_j).
 *   J_c = all keys (non-causal, nA = 1), or keys j < c C (causal: the statistics of
 *   the chunks strictly before chunk c).
 */
elsaa_status elsaa_lowrank_summary(const elsaa_params* p, const void* K, const void* V,
                                   const float* planes_lr, float* A, float* z, void* ws,
                                   size_t ws_bytes, void* stream);

/* Forward: sparse branch over the selection, low-rank readout, Eq. 5 and Eq. 4.
 *   Q, K, V          : [B, H, N, d_h] dtype; planes_lr as above.
 *   q_perm, k_perm   : from elsaa_select; A, z: from elsaa_lowrank_summary.
 *   lambda           : fp32 [H] (>= 0), the lambda of Eq. 5 per head.
 *   g_s, g_lr        : fp32 [B, H, N] gates g_sparse, g_lr of Eq. 4, or NULL for 1.
 *   O (out)          : [B, H, N, d_h] dtype, the fused output.
 *   O_s, O_lr (out)  : [B, H, N, d_h] dtype, the normalized branch outputs (saved
 *                      for elsaa_bwd).
 *   lse_s (out)      : fp32 [B, H, N], log d_sparse (log-sum-exp over the support).
 *   d_lr (out)       : fp32 [B, H, N], the low-rank denominator phi(Q_i)^T z.
 */
elsaa_status elsaa_fwd(const elsaa_params* p, const void* Q, const void* K, const void* V,
                       const float* planes_lr, const int32_t* q_perm, const int32_t* k_perm,
                       const float* A, const float* z, const float* lambda, const float* g_s,
                       const float* g_lr, void* O, void* O_s, void* O_lr, float* lse_s,
                       float* d_lr, void* ws, size_t ws_bytes, void* stream);

/* Backward of elsaa_fwd for training: the chain rule through Eq. 4, Eq. 5, the
 * exact block softmaxes and the RACE readout, with the selection held fixed (it is
 * piecewise constant in Q and K).
 *   dO                      : [B, H, N, d_h] dtype, gradient of the loss w.r.t. O.
 *   O_s, O_lr, lse_s, d_lr  : as saved by elsaa_fwd for the same inputs.
 *   dQ, dK, dV (out)        : [B, H, N, d_h] dtype (overwritten).
 *   dlambda (out)           : fp32 [H] or NULL (overwritten; summed over the batch).
 *   dg_s, dg_lr (out)       : fp32 [B, H, N] or NULL (gradients w.r.t. the gates,
 *                             also when g_s / g_lr are NULL, i.e. at gate 1).
 */
elsaa_status elsaa_bwd(const elsaa_params* p, const void* Q, const void* K, const void* V,
                       const void* dO, const void* O_s, const void* O_lr,
                       const float* planes_lr, const int32_t* q_perm, const int32_t* k_perm,
                       const float* A, const float* z, const float* lse_s, const float* d_lr,
                       const float* lambda, const float* g_s, const float* g_lr, void* dQ,
                       void* dK, void* dV, float* dlambda, float* dg_s, float* dg_lr, void* ws,
                       size_t ws_bytes, void* stream);

/* Diagnostics, not a step of the operator: per-kernel timing. With profiling on,
 * every kernel the four calls launch is bracketed by two HIP events recorded on
 * the stream it is launched on. elsaa_profile(1) discards earlier records and
 * starts recording, elsaa_profile(0) stops. elsaa_profile_report waits for the
 * recorded events and writes one line per kernel, "name launches total_ms\n",
 * into buf (host memory, NUL-terminated, truncated to len bytes); *needed (if not
 * NULL) receives the untruncated length + 1. Returns ELSAA_ERR_HIP if an event
 * query fails. */
elsaa_status elsaa_profile(int32_t enable);
elsaa_status elsaa_profile_report(char* buf, size_t len, size_t* needed);

/* Message for the last non-OK status returned on this host thread ("" if none). */
const char* elsaa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ELSAA_H */
