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
 *   planes_s  : float  [G][hash_bits][d]           (sortLSH hyperplanes)
 *   planes_lr : float  [G][lr_tables][lr_bits][d]  (RACE hyperplanes)
 *   lambda    : double [G]
 *   g_s, g_lr : double [G][N] or NULL (NULL means every gate is 1)
 *   codes     : uint16 [G][N]
 *   perms     : int32  [G][levels][N/2] when causal (levels = log2(N/block)),
 *               int32  [G][1][N] when not
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
} ref_params;

int ref_select(const ref_params* p, const double* Q, const double* K,
               const float* planes_s, uint16_t* q_code, uint16_t* k_code,
               int32_t* q_perm, int32_t* k_perm);

int ref_lowrank_summary(const ref_params* p, const double* K, const double* V,
                        const float* planes_lr, double* A, double* z);

int ref_fwd(const ref_params* p, const double* Q, const double* K, const double* V,
            const float* planes_s, const float* planes_lr, const double* lambda,
            const double* g_s, const double* g_lr,
            double* O, double* O_s, double* O_lr, double* lse, double* d_lr);

int ref_bwd(const ref_params* p, const double* Q, const double* K, const double* V,
            const double* dO, const float* planes_s, const float* planes_lr,
            const double* lambda, const double* g_s, const double* g_lr,
            double* dQ, double* dK, double* dV, double* dlambda,
            double* dg_s, double* dg_lr);

/* Exposed for the pins: the RACE soft bucket assignment of one row x[d]. */
int ref_features(const ref_params* p, const float* planes_lr_head, const double* x,
                 double* phi);

#endif
