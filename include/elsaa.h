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
 *   - Any pointer that is not 16-byte aligned is rejected with
 *     ELSAA_ERR_INVALID_ARG (the kernels read rows with 16-byte vector loads).
 *   - Sizes that are valid for the method but for which no kernel variant is
 *     built (LDS or register limits) return ELSAA_ERR_UNSUPPORTED; a call never
 *     returns ELSAA_OK without having enqueued all of its work.
 *
 * Deliberate differences from a minimal statement of the four calls:
 *   - elsaa_fwd returns the two normalized branch outputs O_s and O_lr next to the
 *     fused O, and elsaa_bwd takes them in place of O: the backward needs
 *     <dO, O_s> and <dO, O_lr> separately (Eq. 4 weighs them with different row
 *     factors), and recovering them from O alone would divide by a gate.
 *   - elsaa_workspace_size takes the call it sizes (the four calls need different
 *     scratch), instead of one size for all.
 *   - The low-rank statistics A are laid out [.., d_h, r] (value channel major):
 *     the kernels read a channel's statistics of all features as one row.
 *   - The RACE tables have 4 hyperplanes each (16 buckets, lr_bits = 4) and the
 *     sortLSH codes at most 12 bits: the sizes the kernels are built for.
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
  ELSAA_CALL_BWD = 3,
  ELSAA_CALL_GATES_BWD = 4,
  ELSAA_CALL_CHECK = 5,
  ELSAA_CALL_TOPK = 6
} elsaa_call;

/* Problem description.
 *   B, H, N, d_h : batch, heads, tokens, head dimension; d_h in {32, 64, 128};
 *                  N a multiple of 32 up to 2^24; B * H == 0 is a valid empty
 *                  problem; B * H <= 65535, and B * H times the number of sparse
 *                  blocks per head (causal: R log2(N/s) N/(2s) + N/s; otherwise
 *                  R N/s, R = hash_rounds) below 2^31 (larger batches are split
 *                  over calls).
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
 *   hash_rounds  : sortLSH hash tables R (Appendix C's L_s), 0 or 1 for one, at
 *                  most 4. Each round hashes with its own hyperplanes and sorts
 *                  independently; a query's sparse support is the union of the
 *                  rounds' supports, each pair counted once (Appendix C's
 *                  Omega_LSH). The per-query counts above then become upper bounds.
 *   extra_edges  : E, 0..64, keys listed per query that join the sparse support
 *                  (elsaa_fwd / elsaa_bwd's extra_idx); 0 for none.
 * Derived: levels Lv = log2(N / s) when causal (off-diagonal recursion levels), 1
 * when not; the permutation length P = R * Lv * N / 2 when causal, R * N when not
 * (the rounds' orders one after another); the number of summaries nA = N / C when
 * causal, 1 when not.
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
  int32_t hash_rounds;
  int32_t extra_edges;
} elsaa_params;

/* Bytes of workspace the given call needs for these parameters (written to
 * *bytes). Returns ELSAA_ERR_INVALID_ARG/UNSUPPORTED for parameters the call
 * would reject. */
elsaa_status elsaa_workspace_size(const elsaa_params* p, int32_t call, size_t* bytes);

/* sortLSH selection (Section 3.2: queries and keys are hashed, sorted by hash and
 * grouped into equal-size blocks; query block b pairs with key block b).
 *   Q, K      : [B, H, N, d_h] dtype.
 *   planes_s  : fp32 [H, R, hash_bits, d_h], the hyperplanes of each head and
 *               round.
 *   q_code, k_code (out): uint16 [B, H, R, N]. Bit b of a token's code is set iff the
 *               projection of its row x on hyperplane b is > 0, the projection being
 *               the fp64 fused-multiply-add chain acc = fma(x[j], R[b][j], acc) for
 *               j = 0..d_h-1 from acc = +0.0.
 *   q_perm, k_perm (out): int32 [B, H, P]. Tokens are ordered by the position of
 *               their code along the reflected Gray sequence, ties by ascending
 *               token index. Non-causal: round u's order of all N tokens at
 *               [u N, (u+1) N). Causal: for round u, level l in [0, Lv) and segment
 *               g of n = N >> l tokens starting at a = g n, the entries starting at
 *               (u Lv + l) N/2 + g n/2, n/2 of them, hold the sorted future half
 *               [a + n/2, a + n) (q_perm) and past half [a, a + n/2) (k_perm).
 *   ws        : device workspace of elsaa_workspace_size(p, ELSAA_CALL_SELECT) bytes
 *               (the hyperplanes widened to fp64).
 */
elsaa_status elsaa_select(const elsaa_params* p, const void* Q, const void* K,
                          const float* planes_s, uint16_t* q_code, uint16_t* k_code,
                          int32_t* q_perm, int32_t* k_perm, void* ws, size_t ws_bytes,
                          void* stream);

/* elsaa_select for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same selection, bit for bit, with no workspace argument. Its scratch (the
 * hyperplanes widened to fp64, 8 * H * hash_bits * d_h bytes) lives in a fixed
 * device array of at most 1 MiB that the library holds on every GPU it runs on
 * until the process ends; larger sizes return ELSAA_ERR_UNSUPPORTED. It calls no
 * allocation routine (the diagnostics of elsaa_profile skip its launches).
 * Calls on one GPU share that array: calls that overlap on one GPU (e.g. on two
 * streams) race on it and must be ordered by the caller. */
elsaa_status elsaa_select_noalloc(const elsaa_params* p, const void* Q, const void* K,
                                  const float* planes_s, uint16_t* q_code, uint16_t* k_code,
                                  int32_t* q_perm, int32_t* k_perm, void* stream);

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
 *   extra_idx        : int32 [B, H, N, E] with E = extra_edges, or NULL when E = 0:
 *                      keys listed per query that join its sparse support (Appendix
 *                      C's augmentation Omega = Omega_LSH u Omega_safe, whose
 *                      Bernoulli draw is the caller's; or any selector's picks,
 *                      e.g. elsaa_topk's). An entry j counts when 0 <= j < N (and
 *                      j <= i when causal); others (-1 padding) are ignored. The
 *                      support is a set: a key listed twice, or already selected
 *                      by sortLSH, counts once. elsaa_bwd takes the same list.
 *   lambda           : fp32 [H] (>= 0), the lambda of Eq. 5 per head.
 *   g_s, g_lr        : fp32 [B, H, N] gates g_sparse, g_lr of Eq. 4, or NULL for 1.
 *   O (out)          : [B, H, N, d_h] dtype, the fused output.
 *   O_s (out)        : fp32 [B, H, N, d_h], the normalized sparse output (Section
 *                      3.2), saved for elsaa_bwd. It is kept in fp32 because the
 *                      backward forms D_i = g_s m_i^2 <dO_i, O_s,i>, which nearly
 *                      cancels <dO_i, V_j> in dS_ij when a query's softmax is peaked.
 *   O_lr (out)       : [B, H, N, d_h] dtype, the normalized low-rank output (Section
 *                      3.1), saved for elsaa_bwd.
 *   lse_s (out)      : fp32 [B, H, N], log d_sparse (log-sum-exp over the support).
 *   d_lr (out)       : fp32 [B, H, N], the low-rank denominator phi(Q_i)^T z.
 */
elsaa_status elsaa_fwd(const elsaa_params* p, const void* Q, const void* K, const void* V,
                       const float* planes_lr, const int32_t* q_perm, const int32_t* k_perm,
                       const int32_t* extra_idx, const float* A, const float* z,
                       const float* lambda, const float* g_s,
                       const float* g_lr, void* O, float* O_s, void* O_lr, float* lse_s,
                       float* d_lr, void* ws, size_t ws_bytes, void* stream);

/* Backward of elsaa_fwd for training: the chain rule through Eq. 4, Eq. 5, the
 * exact block softmaxes and the RACE readout, with the selection held fixed (it is
 * piecewise constant in Q and K).
 *   dO                      : [B, H, N, d_h] dtype, gradient of the loss w.r.t. O.
 *   O_s (fp32), O_lr, lse_s, d_lr : as saved by elsaa_fwd for the same inputs.
 *   dQ, dK, dV (out)        : [B, H, N, d_h] dtype (overwritten).
 *   dlambda (out)           : fp32 [H] or NULL (overwritten; summed over the batch).
 *   dg_s, dg_lr (out)       : fp32 [B, H, N] or NULL (gradients w.r.t. the gates,
 *                             also when g_s / g_lr are NULL, i.e. at gate 1).
 */
elsaa_status elsaa_bwd(const elsaa_params* p, const void* Q, const void* K, const void* V,
                       const void* dO, const float* O_s, const void* O_lr,
                       const float* planes_lr, const int32_t* q_perm, const int32_t* k_perm,
                       const int32_t* extra_idx, const float* A, const float* z,
                       const float* lse_s, const float* d_lr,
                       const float* lambda, const float* g_s, const float* g_lr, void* dQ,
                       void* dK, void* dV, float* dlambda, float* dg_s, float* dg_lr, void* ws,
                       size_t ws_bytes, void* stream);

/* The whole non-causal forward in one launch (the paper's Section 8 names fused
 * GPU kernels as the next step): sortLSH codes and orders, the RACE summary, the
 * sparse block attention, the low-rank readout, Eq. 5 and Eq. 4, one workgroup per
 * (batch, head), every query row read once for both branches. Its outputs are
 * those of elsaa_select, elsaa_lowrank_summary and elsaa_fwd called in turn with
 * the same arguments, and feed elsaa_bwd the same way:
 *   Q, K, V, planes_s, planes_lr, lambda, g_s, g_lr : as for those calls.
 *   q_code, k_code (out) : uint16 [B, H, N];  q_perm, k_perm (out) : int32 [B, H, N].
 *   A, z (out)           : fp32 [B, H, 1, d_h, r], [B, H, 1, r].
 *   O, O_s, O_lr, lse_s, d_lr (out) : as for elsaa_fwd.
 * Taken for: causal = 0, hash_rounds <= 1, extra_edges = 0, hash_bits <= 10,
 * block <= 128, N <= 65536, and the head's rows, statistics and orders within one
 * workgroup's LDS (about 8 N bytes on top of the tiles); other parameters return
 * ELSAA_ERR_UNSUPPORTED and the two-call path serves them. Needs no workspace.
 * The summation order of A, z differs from elsaa_lowrank_summary's, so those (and
 * what depends on them) agree with the two-call path to rounding, not bit for bit;
 * codes and orders are the same bit for bit. */
elsaa_status elsaa_fwd_fused(const elsaa_params* p, const void* Q, const void* K, const void* V,
                             const float* planes_s, const float* planes_lr, const float* lambda,
                             const float* g_s, const float* g_lr, uint16_t* q_code,
                             uint16_t* k_code, int32_t* q_perm, int32_t* k_perm, float* A,
                             float* z, void* O, float* O_s, void* O_lr, float* lse_s,
                             float* d_lr, void* stream);

/* Exact per-query top-k key selection on Q K^T, the top-k kind of sparse selector
 * the paper lists beside sortLSH (Section 3), as an alternative to elsaa_select.
 * For query i the candidate keys are every j (causal: j <= i); the score of (i, j)
 * is the fp64 fused-multiply-add chain acc = fma(Q_i[c], K_j[c], acc), c = 0 ..
 * d_h-1, from +0.0 (the positive score scale does not change the order); the set
 * holds the min(k, #candidates) keys of largest score, ties to the lower index.
 *   p   : as for the other calls; B, H, N, d_h, dtype and causal are used.
 *   k   : 1 .. 256 keys per query (ELSAA_ERR_UNSUPPORTED above).
 *   idx (out): int32 [B, H, N, k], each query's set in ascending key order, -1
 *       past min(k, #candidates).
 *   ws  : elsaa_workspace_size(p, ELSAA_CALL_TOPK) bytes (the same for any k <= 256:
 *       per query a threshold, a bound, a count and a list of up to 320 keys with
 *       their fp32 scores).
 * The sets are exact: any correctly rounded fp64 implementation of the chain
 * selects the same keys. (fp32 scores on the matrix cores locate each query's
 * k-th best to within their rounding bound; only the keys within twice that bound
 * of it are rescored in fp64.) */
elsaa_status elsaa_topk(const elsaa_params* p, const void* Q, const void* K, int32_t k,
                        int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* Learnable gates of Eq. 4. The paper has g_sparse,i and g_lr,i learned with the
 * model (Section 7: shared by ELSAA and its Sort_Lsh_RACE ablation, and on NIAH
 * the gate learns to up-weight the low-rank branch; Section 8: gate schedules per
 * depth and head) but prints no formula; here they are the logistic function of
 * a per-head affine projection of the query:
 *   g_k,i = 1 / (1 + exp(-(<W[h][k], Q_i> + b[h][k]))),  k = 0: g_sparse, 1: g_lr.
 * elsaa_gates_fwd writes them for elsaa_fwd / elsaa_bwd (as their g_s, g_lr).
 *   W : fp32 [H, 2, d_h];  b : fp32 [H, 2];  g_s, g_lr (out): fp32 [B, H, N]. */
elsaa_status elsaa_gates_fwd(const elsaa_params* p, const void* Q, const float* W,
                             const float* b, float* g_s, float* g_lr, void* stream);

/* Backward of elsaa_gates_fwd: from dg_s, dg_lr (as elsaa_bwd returns them) it
 * ADDS the gate path's gradient to dQ ([B, H, N, d_h] dtype, in place: pass the
 * dQ of elsaa_bwd) and writes dW (fp32 [H, 2, d_h]) and db (fp32 [H, 2]), summed
 * over the batch in a fixed order. g_s, g_lr: the gates elsaa_gates_fwd returned.
 * ws: elsaa_workspace_size(p, ELSAA_CALL_GATES_BWD) bytes. */
elsaa_status elsaa_gates_bwd(const elsaa_params* p, const void* Q, const float* W,
                             const float* g_s, const float* g_lr, const float* dg_s,
                             const float* dg_lr, void* dQ, float* dW, float* db, void* ws,
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

/* Debug check of selection orders, for callers that build or modify q_perm /
 * k_perm themselves (the sparse kernels index rows by them without bounds
 * checks). For every order (round, and level when causal) of every head: each
 * entry must be a token of the range its position stands for (non-causal: 0..N-1;
 * causal level l: the future half [a + n/2, a + n) for q_perm, the past half
 * [a, a + n/2) for k_perm, of its segment of n = N >> l tokens at a), and each
 * range must hold each of its tokens exactly once.
 *   bad (out) : int32 [B * H], the number of violations found in each head's
 *               orders (entries out of range plus tokens missing or repeated);
 *               0 for valid orders.
 *   ws        : elsaa_workspace_size(p, ELSAA_CALL_CHECK) bytes.
 * With the environment variable ELSAA_CHECK_ORDERS set to 1, elsaa_fwd and
 * elsaa_bwd run this check first, wait for it, and return ELSAA_ERR_INVALID_ARG
 * without launching their kernels if any head's orders are invalid (a debugging
 * aid: it synchronizes the stream, so it does not suit graph capture).
 * Likewise ELSAA_CHECK_FINITE=1 makes them count the NaN and infinite entries of
 * Q, K, V (and dO) first and return ELSAA_ERR_INVALID_ARG, naming the tensor, if
 * there are any. Without it such values propagate: a non-finite key or value
 * reaches every query whose support or low-rank sums include it, a non-finite
 * query only its own outputs. */
elsaa_status elsaa_check_orders(const elsaa_params* p, const int32_t* q_perm,
                                const int32_t* k_perm, int32_t* bad, void* ws, size_t ws_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ELSAA_H */
