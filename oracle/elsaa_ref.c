/*
 * elsaa_ref.c -- the oracle (TEST INFRASTRUCTURE ONLY; see elsaa_ref.h).
 *
 * Plain fp64 loops, one head at a time, written from "ELSAA: Efficient Low-Rank
 * and Sparse Attention Approximation for Training Transformers" (arXiv 2607.20214):
 *   - Section 3: per-head operator; dense attention as the object approximated.
 *   - Section 3.1: RACE low-rank branch (soft hypercube buckets, bucket
 *     statistics, normalized ratio readout, causal prefix form).
 *   - Section 3.2: sortLSH sparse branch (hash, sort, equal-size blocks, diagonal
 *     block pairing, exact block softmax) and its causal divide-and-conquer with a
 *     log-sum-exp merge.
 *   - Section 3.3, Eq. 5: m_i = d_sparse,i / (d_sparse,i + lambda d_lr,i + eps).
 *   - Section 1, Eq. 4: O_i = g_sparse,i m_i O_sparse,i + g_lr,i O_lr,i.
 * The readings taken where the paper is silent (hash family, bucket order,
 * tie-break, causal base case, RACE soft assignment, gates) are stated at each
 * function. The backward pass is the chain rule through these definitions.
 */
#include "elsaa_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define RET_BAD (-1)

static int ilog2_exact(int x) {
  int l = 0;
  if (x <= 0) return -1;
  while ((1 << l) < x) ++l;
  return ((1 << l) == x) ? l : -1;
}

static int check_params(const ref_params* p) {
  if (!p || p->G <= 0 || p->N <= 0 || p->d <= 0) return RET_BAD;
  if (p->block <= 0 || p->N % p->block) return RET_BAD;
  if (p->hash_bits < 1 || p->hash_bits > 16) return RET_BAD;
  if (p->hash_rounds < 0 || p->hash_rounds > 16) return RET_BAD;
  if (p->extra_edges < 0) return RET_BAD;
  if (p->lr_tables < 1 || p->lr_bits < 0 || p->lr_bits > 8) return RET_BAD;
  if (p->causal) {
    if (ilog2_exact(p->N / p->block) < 0) return RET_BAD;
    if (p->chunk <= 0 || p->N % p->chunk) return RET_BAD;
  }
  return 0;
}

/* sortLSH hash tables (rounds); 0 means one. */
static int n_rounds(const ref_params* p) { return p->hash_rounds > 1 ? p->hash_rounds : 1; }

/* Number of off-diagonal recursion levels of the causal sparse branch. */
static int n_levels(const ref_params* p) {
  return p->causal ? ilog2_exact(p->N / p->block) : 1;
}

/* ------------------------------------------------------------------------- */
/* sortLSH selection (Section 3.2)                                            */
/* ------------------------------------------------------------------------- */

/* Hash code of one row: bit p is set when the projection of x on hyperplane p is
 * positive (sign random projection, the angular LSH family whose collision
 * probability Section 4 writes as rho_ij). The projection is evaluated as an fp64
 * fused multiply-add chain in index order starting from +0.0, so that any other
 * implementation using correctly rounded fp64 FMA in the same order reproduces
 * every bit. */
static uint16_t hash_row(const double* x, const float* planes, int bits, int d) {
  unsigned code = 0;
  for (int b = 0; b < bits; ++b) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc = fma(x[j], (double)planes[(size_t)b * d + j], acc);
    if (acc > 0.0) code |= 1u << b;
  }
  return (uint16_t)code;
}

/* Position of a code along the reflected binary Gray order, so that buckets
 * adjacent in the sort differ in one hyperplane ("sorted Hamming LSH"). */
static unsigned gray_rank(unsigned code) {
  unsigned r = 0;
  for (int sh = 0; sh < 16; ++sh) r ^= code >> sh;
  return r & 0xFFFFu;
}

/* Stable counting sort of the tokens idx[0..n) (given in ascending index order)
 * by rank; equal ranks keep ascending token index. */
static void sort_by_rank(const int32_t* idx, int n, const unsigned* rank, int nbins,
                         int32_t* out) {
  int* start = (int*)calloc((size_t)nbins + 1, sizeof(int));
  for (int t = 0; t < n; ++t) start[rank[idx[t]] + 1]++;
  for (int b = 0; b < nbins; ++b) start[b + 1] += start[b];
  for (int t = 0; t < n; ++t) out[start[rank[idx[t]]]++] = idx[t];
  free(start);
}

static void select_head(const ref_params* p, const double* Q, const double* K,
                        const float* planes, uint16_t* qc, uint16_t* kc,
                        int32_t* qperm, int32_t* kperm) {
  const int N = p->N, d = p->d, bits = p->hash_bits, nbins = 1 << bits;
  unsigned* qr = (unsigned*)malloc(sizeof(unsigned) * N);
  unsigned* kr = (unsigned*)malloc(sizeof(unsigned) * N);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * N);
  for (int t = 0; t < N; ++t) {
    qc[t] = hash_row(Q + (size_t)t * d, planes, bits, d);
    kc[t] = hash_row(K + (size_t)t * d, planes, bits, d);
    qr[t] = gray_rank(qc[t]);
    kr[t] = gray_rank(kc[t]);
  }
  if (!p->causal) {
    for (int t = 0; t < N; ++t) idx[t] = t;
    sort_by_rank(idx, N, qr, nbins, qperm);
    sort_by_rank(idx, N, kr, nbins, kperm);
  } else {
    /* Level l splits the sequence into segments of n = N >> l tokens. In each
     * segment the future half's queries and the past half's keys are sorted
     * (Section 3.2: the future-past block is handled by non-causal sortLSH). */
    const int L = n_levels(p), half = N / 2;
    for (int l = 0; l < L; ++l) {
      const int n = N >> l;
      for (int a = 0; a < N; a += n) {
        const size_t off = (size_t)l * half + (size_t)(a / n) * (n / 2);
        for (int t = 0; t < n / 2; ++t) idx[t] = a + n / 2 + t;
        sort_by_rank(idx, n / 2, qr, nbins, qperm + off);
        for (int t = 0; t < n / 2; ++t) idx[t] = a + t;
        sort_by_rank(idx, n / 2, kr, nbins, kperm + off);
      }
    }
  }
  free(qr); free(kr); free(idx);
}

static size_t perm_len(const ref_params* p) {
  return p->causal ? (size_t)n_levels(p) * (p->N / 2) : (size_t)p->N;
}

/* Every round's codes and orders of one head (round r uses its own hyperplanes). */
static void select_rounds(const ref_params* p, const double* Q, const double* K,
                          const float* planes, uint16_t* qc, uint16_t* kc, int32_t* qperm,
                          int32_t* kperm) {
  const size_t pl = perm_len(p), np = (size_t)p->hash_bits * p->d;
  for (int r = 0; r < n_rounds(p); ++r)
    select_head(p, Q, K, planes + r * np, qc + (size_t)r * p->N, kc + (size_t)r * p->N,
                qperm + r * pl, kperm + r * pl);
}

int ref_select(const ref_params* p, const double* Q, const double* K,
               const float* planes_s, uint16_t* q_code, uint16_t* k_code,
               int32_t* q_perm, int32_t* k_perm) {
  if (check_params(p)) return RET_BAD;
  const size_t nd = (size_t)p->N * p->d, R = n_rounds(p), pl = perm_len(p);
#pragma omp parallel for schedule(dynamic)
  for (int g = 0; g < p->G; ++g)
    select_rounds(p, Q + g * nd, K + g * nd, planes_s + (size_t)g * R * p->hash_bits * p->d,
                  q_code + (size_t)g * R * p->N, k_code + (size_t)g * R * p->N,
                  q_perm + g * R * pl, k_perm + g * R * pl);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Sparse branch (Section 3.2)                                                */
/* ------------------------------------------------------------------------- */

typedef struct {
  const ref_params* p;
  const double *Q, *K, *V;
  const int32_t *qperm, *kperm;
  const int32_t* extra; /* [N][extra_edges] or NULL */
} head_in;

/* Exact softmax attention of the queries qs[0..nq) over the keys ks[0..nk),
 * optionally restricted to keys at or before the query (causal). Writes the
 * normalized output and log-sum-exp of every query. */
static void block_attention(const head_in* h, const int32_t* qs, int nq, const int32_t* ks,
                            int nk, int causal, double* Oq /*[nq][d]*/, double* lseq) {
  const int d = h->p->d;
  double* e = (double*)malloc(sizeof(double) * nk);
  for (int a = 0; a < nq; ++a) {
    const int i = qs[a];
    double mx = -INFINITY;
    for (int b = 0; b < nk; ++b) {
      const int j = ks[b];
      if (causal && j > i) { e[b] = -INFINITY; continue; }
      double s = 0.0;
      for (int c = 0; c < d; ++c) s += h->Q[(size_t)i * d + c] * h->K[(size_t)j * d + c];
      e[b] = s * h->p->scale;
      if (e[b] > mx) mx = e[b];
    }
    double den = 0.0;
    for (int b = 0; b < nk; ++b) { e[b] = exp(e[b] - mx); den += e[b]; }
    double* o = Oq + (size_t)a * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int b = 0; b < nk; ++b) {
      if (e[b] == 0.0) continue;
      const double w = e[b] / den;
      for (int c = 0; c < d; ++c) o[c] += w * h->V[(size_t)ks[b] * d + c];
    }
    lseq[a] = mx + log(den);
  }
  free(e);
}

/* Non-causal sortLSH on already sorted query and key lists of equal length n:
 * query block b (positions b*s..b*s+s-1 of the sorted query list) attends to key
 * block b, i.e. only the diagonal blocks of the permuted score matrix. */
static void sortlsh_blocks(const head_in* h, const int32_t* qsorted, const int32_t* ksorted,
                           int n, double* Ob /*[s][d]*/, double* lseb /*[s]*/,
                           void (*emit)(void*, int, const double*, double), void* ctx) {
  const int s = h->p->block, d = h->p->d;
  for (int b = 0; b < n / s; ++b) {
    block_attention(h, qsorted + (size_t)b * s, s, ksorted + (size_t)b * s, s, 0, Ob, lseb);
    for (int a = 0; a < s; ++a) emit(ctx, qsorted[(size_t)b * s + a], Ob + (size_t)a * d, lseb[a]);
  }
}

typedef struct { double* O; double* lse; int d; } acc_ctx;

/* Store a block result for query i (first contribution). */
static void emit_store(void* vc, int i, const double* o, double lse) {
  acc_ctx* c = (acc_ctx*)vc;
  memcpy(c->O + (size_t)i * c->d, o, sizeof(double) * c->d);
  c->lse[i] = lse;
}

/* Merge a further contribution for query i with a log-sum-exp-aware combination,
 * which keeps the result equal to one softmax over the union of the supports. */
static void emit_merge(void* vc, int i, const double* o, double lse) {
  acc_ctx* c = (acc_ctx*)vc;
  double* Oi = c->O + (size_t)i * c->d;
  const double l1 = c->lse[i], l2 = lse;
  const double mx = l1 > l2 ? l1 : l2;
  const double tot = mx + log(exp(l1 - mx) + exp(l2 - mx));
  const double w1 = exp(l1 - tot), w2 = exp(l2 - tot);
  for (int k = 0; k < c->d; ++k) Oi[k] = w1 * Oi[k] + w2 * o[k];
  c->lse[i] = tot;
}

/* Causal sortLSH (Section 3.2, the divide-and-conquer it adopts from
 * HyperAttention): on the segment [a, a+n) at recursion depth l, the past and the
 * future halves are handled by recursive causal calls, the future-past block by
 * non-causal sortLSH (every key precedes every query), and the two contributions
 * of each future query are merged by log-sum-exp. Segments of at most one block
 * are computed densely with the causal mask (diagonal included). */
static void sparse_causal(const head_in* h, int a, int n, int l, acc_ctx* acc,
                          double* Ob, double* lseb) {
  const int s = h->p->block, N = h->p->N, d = h->p->d;
  if (n <= s) {
    int32_t* t = (int32_t*)malloc(sizeof(int32_t) * n);
    for (int k = 0; k < n; ++k) t[k] = a + k;
    block_attention(h, t, n, t, n, 1, Ob, lseb);
    for (int k = 0; k < n; ++k) emit_store(acc, a + k, Ob + (size_t)k * d, lseb[k]);
    free(t);
    return;
  }
  sparse_causal(h, a, n / 2, l + 1, acc, Ob, lseb);
  sparse_causal(h, a + n / 2, n / 2, l + 1, acc, Ob, lseb);
  const size_t off = (size_t)l * (N / 2) + (size_t)(a / n) * (n / 2);
  sortlsh_blocks(h, h->qperm + off, h->kperm + off, n / 2, Ob, lseb, emit_merge, acc);
}

static void sparse_head(const head_in* h, double* O_s, double* lse) {
  const int s = h->p->block, d = h->p->d;
  double* Ob = (double*)malloc(sizeof(double) * (size_t)s * d);
  double* lseb = (double*)malloc(sizeof(double) * s);
  acc_ctx acc = {O_s, lse, d};
  if (h->p->causal)
    sparse_causal(h, 0, h->p->N, 0, &acc, Ob, lseb);
  else
    sortlsh_blocks(h, h->qperm, h->kperm, h->p->N, Ob, lseb, emit_store, &acc);
  free(Ob); free(lseb);
}

/* Several hash rounds (Appendix C: L_s independent hash tables, the support
 * Omega_LSH being the union of what each table selects), and the listed extra
 * edges (Appendix C's Omega_safe). The union support of query i: its causal leaf,
 * for every round the key block paired with i's query block at every level where
 * i is a future query (one level when not causal), and its valid listed keys.
 * Written as mark[j] = 1 for the keys j in it (each key once). invq:
 * [rounds][levels][N], position of a token within its level's query order, or -1. */
static void union_support(const ref_params* p, const int32_t* qperm, const int32_t* kperm,
                          const int32_t* extra, const int32_t* invq, int i,
                          unsigned char* mark) {
  const int N = p->N, s = p->block, L = n_levels(p), R = n_rounds(p);
  const size_t pl = perm_len(p);
  memset(mark, 0, N);
  if (p->causal)
    for (int j = (i / s) * s; j <= i; ++j) mark[j] = 1;
  for (int r = 0; r < R; ++r)
    for (int l = 0; l < L; ++l) {
      const int t = invq[((size_t)r * L + l) * N + i];
      if (t < 0) continue;
      const int32_t* ks = kperm + r * pl + (size_t)l * (p->causal ? N / 2 : N) + (size_t)(t / s) * s;
      for (int b = 0; b < s; ++b) mark[ks[b]] = 1;
    }
  if (extra)
    for (int e = 0; e < p->extra_edges; ++e) {
      const int32_t j = extra[(size_t)i * p->extra_edges + e];
      if (j >= 0 && j < N && (!p->causal || j <= i)) mark[j] = 1;
    }
}

static int32_t* query_positions(const ref_params* p, const int32_t* qperm) {
  const int N = p->N, L = n_levels(p), R = n_rounds(p);
  const size_t pl = perm_len(p), len = p->causal ? (size_t)N / 2 : (size_t)N;
  int32_t* invq = (int32_t*)malloc(sizeof(int32_t) * (size_t)R * L * N);
  for (size_t e = 0; e < (size_t)R * L * N; ++e) invq[e] = -1;
  for (int r = 0; r < R; ++r)
    for (int l = 0; l < L; ++l)
      for (size_t t = 0; t < len; ++t)
        invq[((size_t)r * L + l) * N + qperm[r * pl + (size_t)l * len + t]] = (int32_t)t;
  return invq;
}

/* Sparse branch over the union support: one exact softmax per query. */
static void sparse_union_head(const head_in* h, double* O_s, double* lse) {
  const ref_params* p = h->p;
  const int N = p->N, d = p->d;
  int32_t* invq = query_positions(p, h->qperm);
  unsigned char* mark = (unsigned char*)malloc(N);
  double* e = (double*)malloc(sizeof(double) * N);
  for (int i = 0; i < N; ++i) {
    union_support(p, h->qperm, h->kperm, h->extra, invq, i, mark);
    double mx = -INFINITY;
    for (int j = 0; j < N; ++j) {
      if (!mark[j]) continue;
      double sc = 0.0;
      for (int c = 0; c < d; ++c) sc += h->Q[(size_t)i * d + c] * h->K[(size_t)j * d + c];
      e[j] = sc * p->scale;
      if (e[j] > mx) mx = e[j];
    }
    double den = 0.0;
    for (int j = 0; j < N; ++j)
      if (mark[j]) { e[j] = exp(e[j] - mx); den += e[j]; }
    double* o = O_s + (size_t)i * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j < N; ++j) {
      if (!mark[j]) continue;
      const double w = e[j] / den;
      for (int c = 0; c < d; ++c) o[c] += w * h->V[(size_t)j * d + c];
    }
    lse[i] = mx + log(den);
  }
  free(invq); free(mark); free(e);
}

/* ------------------------------------------------------------------------- */
/* Low-rank branch (Section 3.1)                                              */
/* ------------------------------------------------------------------------- */

/* RACE soft bucket assignment. Table l projects x on its lr_bits hyperplanes,
 * u_lt = scale <R_lt, x>, and assigns x softly to the 2^lr_bits vertices v_b of
 * the hypercube {-1,+1}^lr_bits: phi_lb = softmax_b(<v_b, u_l> / tau), with bit t
 * of b set meaning coordinate t of v_b is +1. Feature index l * 2^lr_bits + b. */
static void features_row(const ref_params* p, const float* R, const double* x, double* phi) {
  const int L = p->lr_tables, G = p->lr_bits, nb = 1 << G, d = p->d;
  double u[8];
  double* a = (double*)malloc(sizeof(double) * nb);
  for (int l = 0; l < L; ++l) {
    for (int t = 0; t < G; ++t) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += (double)R[((size_t)l * G + t) * d + j] * x[j];
      u[t] = p->scale * acc;
    }
    double mx = -INFINITY, den = 0.0;
    for (int b = 0; b < nb; ++b) {
      double v = 0.0;
      for (int t = 0; t < G; ++t) v += ((b >> t) & 1) ? u[t] : -u[t];
      a[b] = v / p->tau;
      if (a[b] > mx) mx = a[b];
    }
    for (int b = 0; b < nb; ++b) { a[b] = exp(a[b] - mx); den += a[b]; }
    for (int b = 0; b < nb; ++b) phi[(size_t)l * nb + b] = a[b] / den;
  }
  free(a);
}

int ref_features(const ref_params* p, const float* planes_lr_head, const double* x,
                 double* phi) {
  if (!p || p->lr_bits < 0 || p->lr_bits > 8 || p->lr_tables < 1) return RET_BAD;
  features_row(p, planes_lr_head, x, phi);
  return 0;
}

static int feat_dim(const ref_params* p) { return p->lr_tables << p->lr_bits; }

static void all_features(const ref_params* p, const float* R, const double* X, double* F) {
  const int r = feat_dim(p);
  for (int t = 0; t < p->N; ++t) features_row(p, R, X + (size_t)t * p->d, F + (size_t)t * r);
}

static void summary_head(const ref_params* p, const double* K, const double* V,
                         const float* R, double* A, double* z) {
  const int N = p->N, d = p->d, r = feat_dim(p);
  double* kf = (double*)malloc(sizeof(double) * (size_t)N * r);
  all_features(p, R, K, kf);
  double* S = (double*)calloc((size_t)r * d, sizeof(double));
  double* zs = (double*)calloc(r, sizeof(double));
  for (int j = 0; j < N; ++j) {
    if (p->causal && j % p->chunk == 0) {
      const int c = j / p->chunk;
      memcpy(A + (size_t)c * r * d, S, sizeof(double) * r * d);
      memcpy(z + (size_t)c * r, zs, sizeof(double) * r);
    }
    for (int f = 0; f < r; ++f) {
      const double kv = kf[(size_t)j * r + f];
      zs[f] += kv;
      for (int c = 0; c < d; ++c) S[(size_t)f * d + c] += kv * V[(size_t)j * d + c];
    }
  }
  if (!p->causal) {
    memcpy(A, S, sizeof(double) * r * d);
    memcpy(z, zs, sizeof(double) * r);
  }
  free(kf); free(S); free(zs);
}

int ref_lowrank_summary(const ref_params* p, const double* K, const double* V,
                        const float* planes_lr, double* A, double* z) {
  if (check_params(p)) return RET_BAD;
  const size_t nd = (size_t)p->N * p->d, r = feat_dim(p);
  const size_t nA = p->causal ? (size_t)(p->N / p->chunk) : 1;
  const size_t plr = (size_t)p->lr_tables * p->lr_bits * p->d;
#pragma omp parallel for schedule(dynamic)
  for (int g = 0; g < p->G; ++g)
    summary_head(p, K + g * nd, V + g * nd, planes_lr + g * plr, A + g * nA * r * p->d,
                 z + g * nA * r);
  return 0;
}

/* Normalized ratio readout: num_i = sum_j (phi(Q_i).phi(K_j)) V_j and
 * den_i = sum_j phi(Q_i).phi(K_j) over all keys (non-causal) or keys j <= i
 * (causal), accumulated as bucket statistics sum_j phi(K_j) V_j^T and
 * sum_j phi(K_j), running along the sequence when causal. */
static void readout_row(int r, int d, const double* q, const double* S, const double* zs,
                        double* num, double* den) {
  double dn = 0.0;
  for (int c = 0; c < d; ++c) num[c] = 0.0;
  for (int f = 0; f < r; ++f) {
    dn += q[f] * zs[f];
    for (int c = 0; c < d; ++c) num[c] += q[f] * S[(size_t)f * d + c];
  }
  *den = dn;
}

static void add_key(int r, int d, const double* k, const double* v, double* S, double* zs) {
  for (int f = 0; f < r; ++f) {
    zs[f] += k[f];
    for (int c = 0; c < d; ++c) S[(size_t)f * d + c] += k[f] * v[c];
  }
}

static void lowrank_head(const ref_params* p, const double* qf, const double* kf,
                         const double* V, double* num, double* den) {
  const int N = p->N, d = p->d, r = feat_dim(p);
  double* S = (double*)calloc((size_t)r * d, sizeof(double));
  double* zs = (double*)calloc(r, sizeof(double));
  if (!p->causal) {
    for (int j = 0; j < N; ++j) add_key(r, d, kf + (size_t)j * r, V + (size_t)j * d, S, zs);
    for (int i = 0; i < N; ++i)
      readout_row(r, d, qf + (size_t)i * r, S, zs, num + (size_t)i * d, den + i);
  } else {
    for (int i = 0; i < N; ++i) {
      add_key(r, d, kf + (size_t)i * r, V + (size_t)i * d, S, zs);
      readout_row(r, d, qf + (size_t)i * r, S, zs, num + (size_t)i * d, den + i);
    }
  }
  free(S); free(zs);
}

/* ------------------------------------------------------------------------- */
/* Forward: both branches and the fusion                                      */
/* ------------------------------------------------------------------------- */

typedef struct {
  double *O_s, *lse, *qf, *kf, *num, *den, *O_lr, *m;
  int32_t *qperm, *kperm;
  uint16_t *qc, *kc;
} head_fwd;

static void head_fwd_alloc(const ref_params* p, head_fwd* f) {
  const size_t N = p->N, d = p->d, r = feat_dim(p), pl = perm_len(p) * n_rounds(p);
  f->O_s = (double*)malloc(sizeof(double) * N * d);
  f->lse = (double*)malloc(sizeof(double) * N);
  f->qf = (double*)malloc(sizeof(double) * N * r);
  f->kf = (double*)malloc(sizeof(double) * N * r);
  f->num = (double*)malloc(sizeof(double) * N * d);
  f->den = (double*)malloc(sizeof(double) * N);
  f->O_lr = (double*)malloc(sizeof(double) * N * d);
  f->m = (double*)malloc(sizeof(double) * N);
  f->qperm = (int32_t*)malloc(sizeof(int32_t) * pl);
  f->kperm = (int32_t*)malloc(sizeof(int32_t) * pl);
  f->qc = (uint16_t*)malloc(sizeof(uint16_t) * N * n_rounds(p));
  f->kc = (uint16_t*)malloc(sizeof(uint16_t) * N * n_rounds(p));
}

static void head_fwd_free(head_fwd* f) {
  free(f->O_s); free(f->lse); free(f->qf); free(f->kf); free(f->num); free(f->den);
  free(f->O_lr); free(f->m); free(f->qperm); free(f->kperm); free(f->qc); free(f->kc);
}

/* Eq. 5, m = d_sparse / (d_sparse + c) with d_sparse = exp(lse) and
 * c = lambda d_lr + eps, together with w = d_sparse / (d_sparse + c)^2 (so that
 * dm/dc = -w and dm/dlse = c w). For lse >= 0 numerator and denominator are
 * divided by d_sparse, so exp(lse) is never formed where it could overflow. */
static void mass_ratio(double lse, double c, double* m, double* w) {
  if (lse >= 0.0) {
    const double t = exp(-lse), den = 1.0 + c * t;
    *m = 1.0 / den;
    *w = t / (den * den);
  } else {
    const double u = exp(lse), T = u + c;
    *m = u / T;
    *w = u / (T * T);
  }
}

/* One head forward. gs/glr may be NULL (gate 1). */
static void forward_head(const ref_params* p, const double* Q, const double* K,
                         const double* V, const float* Rs, const float* Rlr, double lam,
                         const double* gs, const double* glr, const int32_t* extra, head_fwd* f,
                         double* O) {
  const int N = p->N, d = p->d;
  select_rounds(p, Q, K, Rs, f->qc, f->kc, f->qperm, f->kperm);
  head_in h = {p, Q, K, V, f->qperm, f->kperm, extra};
  if (n_rounds(p) == 1 && !extra)
    sparse_head(&h, f->O_s, f->lse);
  else
    sparse_union_head(&h, f->O_s, f->lse);
  all_features(p, Rlr, Q, f->qf);
  all_features(p, Rlr, K, f->kf);
  lowrank_head(p, f->qf, f->kf, V, f->num, f->den);
  for (int i = 0; i < N; ++i) {
    for (int c = 0; c < d; ++c) f->O_lr[(size_t)i * d + c] = f->num[(size_t)i * d + c] / f->den[i];
    /* Eq. 5 with d_sparse,i = sum over the support of exp(score) = exp(lse_i). */
    double w;
    mass_ratio(f->lse[i], lam * f->den[i] + p->eps, &f->m[i], &w);
    const double a = (gs ? gs[i] : 1.0) * f->m[i], b = glr ? glr[i] : 1.0;
    for (int c = 0; c < d; ++c)
      O[(size_t)i * d + c] = a * f->O_s[(size_t)i * d + c] + b * f->O_lr[(size_t)i * d + c];
  }
}

int ref_fwd(const ref_params* p, const double* Q, const double* K, const double* V,
            const float* planes_s, const float* planes_lr, const double* lambda,
            const double* g_s, const double* g_lr, const int32_t* extra,
            double* O, double* O_s, double* O_lr, double* lse, double* d_lr) {
  if (check_params(p) || !lambda) return RET_BAD;
  if (p->extra_edges == 0) extra = NULL;
  const size_t ne = (size_t)p->N * p->extra_edges;
  const size_t N = p->N, nd = N * p->d;
  const size_t ps = (size_t)n_rounds(p) * p->hash_bits * p->d;
  const size_t plr = (size_t)p->lr_tables * p->lr_bits * p->d;
#pragma omp parallel for schedule(dynamic)
  for (int g = 0; g < p->G; ++g) {
    head_fwd f;
    head_fwd_alloc(p, &f);
    forward_head(p, Q + g * nd, K + g * nd, V + g * nd, planes_s + g * ps, planes_lr + g * plr,
                 lambda[g], g_s ? g_s + g * N : NULL, g_lr ? g_lr + g * N : NULL,
                 extra ? extra + g * ne : NULL, &f, O + g * nd);
    if (O_s) memcpy(O_s + g * nd, f.O_s, sizeof(double) * nd);
    if (O_lr) memcpy(O_lr + g * nd, f.O_lr, sizeof(double) * nd);
    if (lse) memcpy(lse + g * N, f.lse, sizeof(double) * N);
    if (d_lr) memcpy(d_lr + g * N, f.den, sizeof(double) * N);
    head_fwd_free(&f);
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Backward: the chain rule through the definitions above, selection held      */
/* fixed (sorting and hashing are piecewise constant in Q and K).              */
/* ------------------------------------------------------------------------- */

/* Gradient of one exact block softmax: scores s_ij = scale Q_i.K_j over the block,
 * p_ij = exp(s_ij - lse_i) with the query's final (union) log-sum-exp, upstream
 * gradients dOs_i on the normalized output and dlse_i on the log-sum-exp. */
static void block_attention_bwd(const head_in* h, const int32_t* qs, int nq, const int32_t* ks,
                                int nk, int causal, const double* O_s, const double* lse,
                                const double* dOs, const double* dlse, double* dQ, double* dK,
                                double* dV) {
  const int d = h->p->d;
  const double sc = h->p->scale;
  for (int a = 0; a < nq; ++a) {
    const int i = qs[a];
    double Di = 0.0;
    for (int c = 0; c < d; ++c) Di += dOs[(size_t)i * d + c] * O_s[(size_t)i * d + c];
    for (int b = 0; b < nk; ++b) {
      const int j = ks[b];
      if (causal && j > i) continue;
      double s = 0.0, dp = 0.0;
      for (int c = 0; c < d; ++c) {
        s += h->Q[(size_t)i * d + c] * h->K[(size_t)j * d + c];
        dp += dOs[(size_t)i * d + c] * h->V[(size_t)j * d + c];
      }
      const double pij = exp(s * sc - lse[i]);
      const double ds = pij * (dp - Di) + pij * dlse[i];
      for (int c = 0; c < d; ++c) {
        dV[(size_t)j * d + c] += pij * dOs[(size_t)i * d + c];
        dQ[(size_t)i * d + c] += sc * ds * h->K[(size_t)j * d + c];
        dK[(size_t)j * d + c] += sc * ds * h->Q[(size_t)i * d + c];
      }
    }
  }
}

/* Visit every block of the sparse support (same recursion as the forward). */
static void sparse_bwd_rec(const head_in* h, int a, int n, int l, const double* O_s,
                           const double* lse, const double* dOs, const double* dlse,
                           double* dQ, double* dK, double* dV) {
  const int s = h->p->block, N = h->p->N;
  if (n <= s) {
    int32_t* t = (int32_t*)malloc(sizeof(int32_t) * n);
    for (int k = 0; k < n; ++k) t[k] = a + k;
    block_attention_bwd(h, t, n, t, n, 1, O_s, lse, dOs, dlse, dQ, dK, dV);
    free(t);
    return;
  }
  sparse_bwd_rec(h, a, n / 2, l + 1, O_s, lse, dOs, dlse, dQ, dK, dV);
  sparse_bwd_rec(h, a + n / 2, n / 2, l + 1, O_s, lse, dOs, dlse, dQ, dK, dV);
  const size_t off = (size_t)l * (N / 2) + (size_t)(a / n) * (n / 2);
  for (int b = 0; b < (n / 2) / s; ++b)
    block_attention_bwd(h, h->qperm + off + (size_t)b * s, s, h->kperm + off + (size_t)b * s, s,
                        0, O_s, lse, dOs, dlse, dQ, dK, dV);
}

/* The same over the union support of several hash rounds, one query at a time. */
static void sparse_union_bwd(const head_in* h, const double* O_s, const double* lse,
                             const double* dOs, const double* dlse, double* dQ, double* dK,
                             double* dV) {
  const ref_params* p = h->p;
  const int N = p->N, d = p->d;
  const double sc = p->scale;
  int32_t* invq = query_positions(p, h->qperm);
  unsigned char* mark = (unsigned char*)malloc(N);
  for (int i = 0; i < N; ++i) {
    union_support(p, h->qperm, h->kperm, h->extra, invq, i, mark);
    double Di = 0.0;
    for (int c = 0; c < d; ++c) Di += dOs[(size_t)i * d + c] * O_s[(size_t)i * d + c];
    for (int j = 0; j < N; ++j) {
      if (!mark[j]) continue;
      double s = 0.0, dp = 0.0;
      for (int c = 0; c < d; ++c) {
        s += h->Q[(size_t)i * d + c] * h->K[(size_t)j * d + c];
        dp += dOs[(size_t)i * d + c] * h->V[(size_t)j * d + c];
      }
      const double pij = exp(s * sc - lse[i]);
      const double ds = pij * (dp - Di) + pij * dlse[i];
      for (int c = 0; c < d; ++c) {
        dV[(size_t)j * d + c] += pij * dOs[(size_t)i * d + c];
        dQ[(size_t)i * d + c] += sc * ds * h->K[(size_t)j * d + c];
        dK[(size_t)j * d + c] += sc * ds * h->Q[(size_t)i * d + c];
      }
    }
  }
  free(invq); free(mark);
}

/* Backward of phi = per-table softmax over hypercube vertices, then through the
 * projections u_lt = scale <R_lt, x>: adds d(loss)/dx to dx. */
static void features_row_bwd(const ref_params* p, const float* R, const double* phi,
                             const double* dphi, double* dx) {
  const int L = p->lr_tables, G = p->lr_bits, nb = 1 << G, d = p->d;
  for (int l = 0; l < L; ++l) {
    const double* ph = phi + (size_t)l * nb;
    const double* dph = dphi + (size_t)l * nb;
    double dot = 0.0;
    for (int b = 0; b < nb; ++b) dot += ph[b] * dph[b];
    for (int t = 0; t < G; ++t) {
      double du = 0.0;
      for (int b = 0; b < nb; ++b) {
        const double da = ph[b] * (dph[b] - dot); /* softmax backward */
        du += da * (((b >> t) & 1) ? 1.0 : -1.0) / p->tau;
      }
      for (int j = 0; j < d; ++j) dx[j] += p->scale * du * (double)R[((size_t)l * G + t) * d + j];
    }
  }
}

static void backward_head(const ref_params* p, const double* Q, const double* K, const double* V,
                          const double* dO, const float* Rs, const float* Rlr, double lam,
                          const double* gs, const double* glr, const int32_t* extra, double* dQ,
                          double* dK, double* dV, double* dlam, double* dgs, double* dglr) {
  const int N = p->N, d = p->d, r = feat_dim(p);
  head_fwd f;
  head_fwd_alloc(p, &f);
  double* O = (double*)malloc(sizeof(double) * (size_t)N * d);
  forward_head(p, Q, K, V, Rs, Rlr, lam, gs, glr, extra, &f, O);

  double* dOs = (double*)malloc(sizeof(double) * (size_t)N * d);
  double* dlse = (double*)malloc(sizeof(double) * N);
  double* dnum = (double*)malloc(sizeof(double) * (size_t)N * d);
  double* dden = (double*)malloc(sizeof(double) * N);
  double lam_grad = 0.0;
  for (int i = 0; i < N; ++i) {
    const double g1 = gs ? gs[i] : 1.0, g2 = glr ? glr[i] : 1.0;
    double dOOs = 0.0, dOOlr = 0.0, dOnum = 0.0;
    for (int c = 0; c < d; ++c) {
      dOOs += dO[(size_t)i * d + c] * f.O_s[(size_t)i * d + c];
      dOOlr += dO[(size_t)i * d + c] * f.O_lr[(size_t)i * d + c];
    }
    if (dgs) dgs[i] = f.m[i] * dOOs;
    if (dglr) dglr[i] = dOOlr;
    /* O = g_s m O_s + g_lr O_lr */
    const double dm = g1 * dOOs;
    for (int c = 0; c < d; ++c) {
      dOs[(size_t)i * d + c] = g1 * f.m[i] * dO[(size_t)i * d + c];
      dnum[(size_t)i * d + c] = g2 * dO[(size_t)i * d + c] / f.den[i];
      dOnum += g2 * dO[(size_t)i * d + c] * f.num[(size_t)i * d + c];
    }
    /* O_lr = num / den */
    dden[i] = -dOnum / (f.den[i] * f.den[i]);
    /* m = ds / (ds + c) with ds = exp(lse), c = lam den + eps:
     * dm/dlse = c w, dm/dc = -w, w = ds / (ds + c)^2 */
    const double c = lam * f.den[i] + p->eps;
    double mm, w;
    mass_ratio(f.lse[i], c, &mm, &w);
    dlse[i] = dm * c * w;
    dden[i] += -dm * lam * w;
    lam_grad += -dm * f.den[i] * w;
  }
  *dlam = lam_grad;

  memset(dQ, 0, sizeof(double) * (size_t)N * d);
  memset(dK, 0, sizeof(double) * (size_t)N * d);
  memset(dV, 0, sizeof(double) * (size_t)N * d);
  head_in h = {p, Q, K, V, f.qperm, f.kperm, extra};
  if (n_rounds(p) > 1 || extra)
    sparse_union_bwd(&h, f.O_s, f.lse, dOs, dlse, dQ, dK, dV);
  else if (p->causal)
    sparse_bwd_rec(&h, 0, N, 0, f.O_s, f.lse, dOs, dlse, dQ, dK, dV);
  else
    for (int b = 0; b < N / p->block; ++b)
      block_attention_bwd(&h, f.qperm + (size_t)b * p->block, p->block,
                          f.kperm + (size_t)b * p->block, p->block, 0, f.O_s, f.lse, dOs, dlse,
                          dQ, dK, dV);

  /* Low-rank branch: num_i = sum_{j in J_i} (qf_i.kf_j) V_j, den_i = sum_{j in J_i} qf_i.kf_j.
   * dqf_i = sum_{j in J_i} (dnum_i.V_j + dden_i) kf_j
   * dkf_j = sum_{i: j in J_i} (dnum_i.V_j + dden_i) qf_i
   * dV_j += sum_{i: j in J_i} (qf_i.kf_j) dnum_i
   * evaluated with running sums over keys (prefix, for dqf) and over queries
   * (suffix, for dkf and dV); non-causal J_i is every key. */
  double* dqf = (double*)calloc((size_t)N * r, sizeof(double));
  double* dkf = (double*)calloc((size_t)N * r, sizeof(double));
  double* S = (double*)calloc((size_t)r * d, sizeof(double)); /* sum kf V^T      */
  double* zs = (double*)calloc(r, sizeof(double));             /* sum kf          */
  double* G = (double*)calloc((size_t)r * d, sizeof(double)); /* sum qf dnum^T   */
  double* gz = (double*)calloc(r, sizeof(double));             /* sum qf dden     */
  if (!p->causal) {
    for (int j = 0; j < N; ++j)
      for (int f2 = 0; f2 < r; ++f2) {
        zs[f2] += f.kf[(size_t)j * r + f2];
        for (int c = 0; c < d; ++c) S[(size_t)f2 * d + c] += f.kf[(size_t)j * r + f2] * V[(size_t)j * d + c];
      }
    for (int i = 0; i < N; ++i)
      for (int f2 = 0; f2 < r; ++f2) {
        gz[f2] += f.qf[(size_t)i * r + f2] * dden[i];
        for (int c = 0; c < d; ++c) G[(size_t)f2 * d + c] += f.qf[(size_t)i * r + f2] * dnum[(size_t)i * d + c];
      }
  }
  for (int i = 0; i < N; ++i) { /* prefix over keys for dqf */
    if (p->causal)
      for (int f2 = 0; f2 < r; ++f2) {
        zs[f2] += f.kf[(size_t)i * r + f2];
        for (int c = 0; c < d; ++c) S[(size_t)f2 * d + c] += f.kf[(size_t)i * r + f2] * V[(size_t)i * d + c];
      }
    for (int f2 = 0; f2 < r; ++f2) {
      double v = zs[f2] * dden[i];
      for (int c = 0; c < d; ++c) v += S[(size_t)f2 * d + c] * dnum[(size_t)i * d + c];
      dqf[(size_t)i * r + f2] = v;
    }
  }
  for (int j = N - 1; j >= 0; --j) { /* suffix over queries for dkf, dV */
    if (p->causal)
      for (int f2 = 0; f2 < r; ++f2) {
        gz[f2] += f.qf[(size_t)j * r + f2] * dden[j];
        for (int c = 0; c < d; ++c) G[(size_t)f2 * d + c] += f.qf[(size_t)j * r + f2] * dnum[(size_t)j * d + c];
      }
    for (int f2 = 0; f2 < r; ++f2) {
      double v = gz[f2];
      for (int c = 0; c < d; ++c) v += G[(size_t)f2 * d + c] * V[(size_t)j * d + c];
      dkf[(size_t)j * r + f2] = v;
    }
    for (int c = 0; c < d; ++c) {
      double v = 0.0;
      for (int f2 = 0; f2 < r; ++f2) v += G[(size_t)f2 * d + c] * f.kf[(size_t)j * r + f2];
      dV[(size_t)j * d + c] += v;
    }
  }
  for (int t = 0; t < N; ++t) {
    features_row_bwd(p, Rlr, f.qf + (size_t)t * r, dqf + (size_t)t * r, dQ + (size_t)t * d);
    features_row_bwd(p, Rlr, f.kf + (size_t)t * r, dkf + (size_t)t * r, dK + (size_t)t * d);
  }
  free(dqf); free(dkf); free(S); free(zs); free(G); free(gz);
  free(dOs); free(dlse); free(dnum); free(dden); free(O);
  head_fwd_free(&f);
}

int ref_bwd(const ref_params* p, const double* Q, const double* K, const double* V,
            const double* dO, const float* planes_s, const float* planes_lr,
            const double* lambda, const double* g_s, const double* g_lr,
            const int32_t* extra, double* dQ, double* dK, double* dV, double* dlambda,
            double* dg_s, double* dg_lr) {
  if (check_params(p) || !lambda) return RET_BAD;
  if (p->extra_edges == 0) extra = NULL;
  const size_t ne = (size_t)p->N * p->extra_edges;
  const size_t N = p->N, nd = N * p->d;
  const size_t ps = (size_t)n_rounds(p) * p->hash_bits * p->d;
  const size_t plr = (size_t)p->lr_tables * p->lr_bits * p->d;
#pragma omp parallel for schedule(dynamic)
  for (int g = 0; g < p->G; ++g) {
    double dl = 0.0;
    backward_head(p, Q + g * nd, K + g * nd, V + g * nd, dO + g * nd, planes_s + g * ps,
                  planes_lr + g * plr, lambda[g], g_s ? g_s + g * N : NULL,
                  g_lr ? g_lr + g * N : NULL, extra ? extra + g * ne : NULL, dQ + g * nd,
                  dK + g * nd, dV + g * nd, &dl,
                  dg_s ? dg_s + g * N : NULL, dg_lr ? dg_lr + g * N : NULL);
    if (dlambda) dlambda[g] = dl;
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Learnable gates of Eq. 4: g_k,i = sigmoid(<W_k, Q_i> + b_k) per head.        */
/* ------------------------------------------------------------------------- */

static double gate_logit(const double* w, double b, const double* q, int d) {
  double t = b;
  for (int c = 0; c < d; ++c) t += w[c] * q[c];
  return t;
}

static double logistic(double t) { return 1.0 / (1.0 + exp(-t)); }

int ref_gates_fwd(const ref_params* p, const double* Q, const double* W, const double* b,
                  double* g_s, double* g_lr) {
  if (!p || p->G <= 0 || p->N <= 0 || p->d <= 0 || !Q || !W || !b || !g_s || !g_lr)
    return RET_BAD;
  const int N = p->N, d = p->d;
  for (int g = 0; g < p->G; ++g)
    for (int i = 0; i < N; ++i) {
      const double* q = Q + ((size_t)g * N + i) * d;
      g_s[(size_t)g * N + i] = logistic(gate_logit(W + (size_t)g * 2 * d, b[2 * g], q, d));
      g_lr[(size_t)g * N + i] = logistic(gate_logit(W + ((size_t)g * 2 + 1) * d, b[2 * g + 1], q, d));
    }
  return 0;
}

/* dL/dt = dL/dg g (1 - g) for t the gate's logit; t is linear in W, b and Q. */
int ref_gates_bwd(const ref_params* p, const double* Q, const double* W, const double* b,
                  const double* dg_s, const double* dg_lr, double* dQ, double* dW, double* db) {
  if (!p || p->G <= 0 || p->N <= 0 || p->d <= 0 || !Q || !W || !b || !dg_s || !dg_lr || !dQ ||
      !dW || !db)
    return RET_BAD;
  const int N = p->N, d = p->d;
  for (int g = 0; g < p->G; ++g) {
    for (int k = 0; k < 2; ++k) {
      db[2 * g + k] = 0.0;
      for (int c = 0; c < d; ++c) dW[((size_t)g * 2 + k) * d + c] = 0.0;
    }
    for (int i = 0; i < N; ++i) {
      const double* q = Q + ((size_t)g * N + i) * d;
      double* dq = dQ + ((size_t)g * N + i) * d;
      for (int k = 0; k < 2; ++k) {
        const double* w = W + ((size_t)g * 2 + k) * d;
        const double gv = logistic(gate_logit(w, b[2 * g + k], q, d));
        const double dt = (k == 0 ? dg_s : dg_lr)[(size_t)g * N + i] * gv * (1.0 - gv);
        db[2 * g + k] += dt;
        for (int c = 0; c < d; ++c) {
          dW[((size_t)g * 2 + k) * d + c] += dt * q[c];
          dq[c] += dt * w[c];
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Exact per-query top-k selection on Q K^T (ties: lower key index).          */
/* ------------------------------------------------------------------------- */

typedef struct {
  double s;
  int32_t j;
} scored_key;

/* Descending score, then ascending key index. */
static int by_score_then_index(const void* a, const void* b) {
  const scored_key* x = (const scored_key*)a;
  const scored_key* y = (const scored_key*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int by_index(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int ref_topk(const ref_params* p, const double* Q, const double* K, int k, int32_t* idx) {
  if (!p || p->G <= 0 || p->N <= 0 || p->d <= 0 || k <= 0 || !Q || !K || !idx) return RET_BAD;
  const int N = p->N, d = p->d;
#pragma omp parallel for schedule(dynamic)
  for (int g = 0; g < p->G; ++g) {
    scored_key* sk = (scored_key*)malloc(sizeof(scored_key) * N);
    for (int i = 0; i < N; ++i) {
      const double* q = Q + ((size_t)g * N + i) * d;
      const int nc = p->causal ? i + 1 : N;
      for (int j = 0; j < nc; ++j) {
        const double* kr = K + ((size_t)g * N + j) * d;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc = fma(q[c], kr[c], acc);
        sk[j].s = acc;
        sk[j].j = j;
      }
      qsort(sk, nc, sizeof(scored_key), by_score_then_index);
      const int m = nc < k ? nc : k;
      int32_t* out = idx + ((size_t)g * N + i) * k;
      for (int t = 0; t < m; ++t) out[t] = sk[t].j;
      qsort(out, m, sizeof(int32_t), by_index);
      for (int t = m; t < k; ++t) out[t] = -1;
    }
    free(sk);
  }
  return 0;
}
