/*
 * elsaa_ref.h -- the oracle's own interface (TEST INFRASTRUCTURE ONLY).
 *
 * A plain, slow, fp64 CPU implementation of the ELSAA attention operator from
 * "ELSAA: Efficient Low-Rank and Sparse Attention Approximation for Training
 * Transformers" (Heidari, Rahimi, Moon, arXiv 2607.20214). Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never does, and the two share no code.
 *
 * Every array holds G independent heads (the paper applies the operator to each
 * head independently, Section 3), contiguous, row-major:
 *   Q, K, V, dO, O, O_s, O_lr, dQ, dK, dV : double [G][N][d]
 *   planes_s  : float  [G][rounds][hash_bits][d]   (sortLSH hyperplanes; rounds =
 *               hash_rounds, the L_s independent hash tables of Appendix C)
 *   planes_lr : float  [G][lr_tables][lr_bits][d]  (RACE hyperplanes)
 *   lambda    : double [G]
 *   g_s, g_lr : double [G][N] or NULL (NULL means every gate is 1)
 *   codes     : uint16 [G][rounds][N]
 *   perms     : int32  [G][rounds][levels][N/2] when causal (levels =
 *               log2(N/block)), int32 [G][rounds][1][N] when not
 * With several rounds the sparse support of a query is the union of the rounds'
 * supports (each pair counted once), Appendix C's Omega_LSH.
 *   extra     : int32  [G][N][extra_edges] or NULL: further keys listed per query,
 *               added to the sparse support (Appendix C's augmentation
 *               Omega = Omega_LSH u Omega_safe with Omega_safe,ij ~ Bernoulli(p):
 *               the random draw is the caller's, the edges come in as a list).
 *               An entry j counts when 0 <= j < N (and j <= i when causal); the
 *               support is a set, so a pair listed twice or already selected by
 *               sortLSH is counted once.
 *   A, z      : double [G][r][d], [G][r] (non-causal: sums over all keys);
 *               double [G][N/chunk][r][d], [G][N/chunk][r] (causal: sums over
 *               keys strictly before each chunk), with r = lr_tables << lr_bits.
 * All functions return 0 on success and a negative number on bad parameters.
 */
#ifndef ELSAA_REF_H
#define ELSAA_REF_H
#include <stdint.h>

typedef struct {
  int G, N, d;
  int causal;
  int block;       /* sortLSH block size s                       */
  int hash_bits;   /* sortLSH hyperplanes per head               */
  int lr_tables;   /* RACE tables L                              */
  int lr_bits;     /* RACE hyperplanes per table (gamma)         */
  int chunk;       /* causal RACE summary spacing C              */
  double tau, eps, scale;
  int hash_rounds; /* sortLSH hash tables L_s (0 or 1: one)             */
  int extra_edges; /* entries per query of the extra edge list (0: none) */
} ref_params;

int ref_select(const ref_params* p, const double* Q, const double* K,
               const float* planes_s, uint16_t* q_code, uint16_t* k_code,
               int32_t* q_perm, int32_t* k_perm);

int ref_lowrank_summary(const ref_params* p, const double* K, const double* V,
                        const float* planes_lr, double* A, double* z);

int ref_fwd(const ref_params* p, const double* Q, const double* K, const double* V,
            const float* planes_s, const float* planes_lr, const double* lambda,
            const double* g_s, const double* g_lr, const int32_t* extra,
            double* O, double* O_s, double* O_lr, double* lse, double* d_lr);

int ref_bwd(const ref_params* p, const double* Q, const double* K, const double* V,
            const double* dO, const float* planes_s, const float* planes_lr,
            const double* lambda, const double* g_s, const double* g_lr,
            const int32_t* extra, double* dQ, double* dK, double* dV, double* dlambda,
            double* dg_s, double* dg_lr);

/* Learnable gates of Eq. 4. The paper names g_sparse,i and g_lr,i, has them
 * learned with the model (Section 7: the branches' gates are shared with the
 * Sort_Lsh_RACE ablation, and on NIAH the gate learns to up-weight the low-rank
 * branch; Section 8: gate schedules per depth and head) but prints no formula.
 * Reading taken here: the logistic function of a per-head affine projection of
 * the query,
 *   g_k,i = 1 / (1 + exp(-(<W[k], Q_i> + b[k]))),  k = 0: g_sparse, 1: g_lr,
 * with W double [G][2][d] and b double [G][2]. ref_gates_bwd takes dL/dg_s and
 * dL/dg_lr (as ref_bwd returns them), ADDS the gate path's dL/dQ to dQ, and
 * writes dL/dW and dL/db. */
int ref_gates_fwd(const ref_params* p, const double* Q, const double* W, const double* b,
                  double* g_s, double* g_lr);
int ref_gates_bwd(const ref_params* p, const double* Q, const double* W, const double* b,
                  const double* dg_s, const double* dg_lr, double* dQ, double* dW, double* db);

/* Exact per-query top-k key selection on Q K^T (the "learned top-k" kind of sparse
 * selector the paper lists next to sortLSH in Section 3, here without learning):
 * for query i, the candidate keys are every j (or j <= i when causal), the score
 * of (i, j) is the fp64 fused-multiply-add chain acc = fma(Q_i[c], K_j[c], acc)
 * over c = 0..d-1 from +0.0 (the positive scale of Q K^T / sqrt(d_h) does not
 * change the order), and the selected set holds the min(k, #candidates) keys of
 * largest score, ties broken by the lower key index. idx: int32 [G][N][k], each
 * set in ascending key order, padded with -1. */
int ref_topk(const ref_params* p, const double* Q, const double* K, int k, int32_t* idx);

/* Exposed for the pins: the RACE soft bucket assignment of one row x[d]. */
int ref_features(const ref_params* p, const float* planes_lr_head, const double* x,
                 double* phi);

#endif
