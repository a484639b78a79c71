/*
 * mla_oracle.c -- plain, slow, fp64 CPU oracle for absorbed-weight MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; the two see the same seeded inputs and nothing else.
 *
 * What it computes (one decode step of Multi-head Latent Attention):
 *
 *   explicit form  -- the plain definition.  For every cached token t it
 *     rebuilds the per-head key k_t = W_UK[i] c_t and value v_t = W_UV[i] c_t
 *     ("Multi-Head Latent Attention: Low-Rank KV Compression, Decoupled RoPE,
 *     and Matrix Absorption", section "MLA: Low-Rank Key-Value Joint
 *     Compression"), appends the shared, already-rotated RoPE key to the key
 *     and the RoPE query to the query ("MLA, dim by dim" section 5.2, the
 *     concatenated per-head query and key), scores with one scale on the
 *     concatenated dot product, applies a textbook max-subtracted softmax and
 *     sums the values ("From Vanilla Transformers to Modern LLMs ... Part 3",
 *     section 3.o / 3.p).
 *
 *   absorbed form  -- a second, independent route used as a cross-check.
 *     q_abs = W_UK[i]^T q (the bilinear identity, "Mathematical Prerequisites
 *     for DeepSeek-V2" section 6), scores q_abs . c_t + q_R . k_R,t, softmax,
 *     c_bar = sum_t p_t c_t, o = W_UV[i] c_bar (linearity, same page section
 *     7; "MLA, dim by dim" section 4.2 cached-decode chains; "From Vanilla
 *     Transformers ..." sections 3.e.2 and 3.g).
 *
 * Conventions (the readings that the pages leave open):
 *   - weights are stored [h][d_h][d_c] row-major and act on column vectors,
 *     k = W_UK[i] c, as on the llms.blog page;
 *   - the score scale is one factor on the summed content + RoPE score;
 *     the caller passes it (default 1/sqrt(d_h + d_r), "MLA, dim by dim" 5.2);
 *   - the cache already holds every attended token; with n_q new query tokens
 *     per sequence, query m of sequence b sees tokens 0 .. L_b - n_q + m;
 *   - token t of sequence b lives in pool page page_table[b][t / page_size],
 *     row t % page_size of that page.
 *
 * Parity pins for every exported function live in the tests (worked
 * examples printed on the pages, closed forms, invariants, and a library
 * routine for a special case).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Problem description, shared by both forms.                                */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch, n_q, h, d_c, d_r, d_h;
  int32_t page_size, max_pages, num_pages;
  int32_t _pad;
  double scale;
  const double* q;            /* [batch][n_q][h][d_h]              */
  const double* q_r;          /* [batch][n_q][h][d_r] (rotated)    */
  const double* latent_pool;  /* [num_pages][page_size][d_c]       */
  const double* rope_pool;    /* [num_pages][page_size][d_r]       */
  const int32_t* page_table;  /* [batch][max_pages]                */
  const int32_t* context_lens;/* [batch]                           */
  const double* w_uk;         /* [h][d_h][d_c]                     */
  const double* w_uv;         /* [h][d_h][d_c]                     */
} mla_oracle_problem_t;

/* ------------------------------------------------------------------------ */
/* Linear-algebra primitives ("Mathematical Prerequisites for DeepSeek-V2"). */
/* ------------------------------------------------------------------------ */

/* y = A x, A is m x n row-major: y_i = sum_j A_ij x_j (section 1). */
void mla_oracle_matvec(int m, int n, const double* A, const double* x, double* y) {
  for (int i = 0; i < m; ++i) {
    double acc = 0.0;
    for (int j = 0; j < n; ++j) acc += A[(size_t)i * n + j] * x[j];
    y[i] = acc;
  }
}

/* y = A^T x, A is m x n row-major, x has m entries, y has n entries:
 * (A^T)_ji = A_ij (section 2), so y_j = sum_i A_ij x_i. */
void mla_oracle_matvec_t(int m, int n, const double* A, const double* x, double* y) {
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int i = 0; i < m; ++i) acc += A[(size_t)i * n + j] * x[i];
    y[j] = acc;
  }
}

/* a^T b for n-vectors. */
double mla_oracle_dot(int n, const double* a, const double* b) {
  double acc = 0.0;
  for (int k = 0; k < n; ++k) acc += a[k] * b[k];
  return acc;
}

/* Textbook softmax with the row maximum subtracted first; equal to the
 * plain exp(s_t) / sum exp(s) in exact arithmetic. */
void mla_oracle_softmax(int n, const double* s, double* p) {
  if (n <= 0) return;
  double mx = s[0];
  for (int t = 1; t < n; ++t) if (s[t] > mx) mx = s[t];
  double sum = 0.0;
  for (int t = 0; t < n; ++t) { p[t] = exp(s[t] - mx); sum += p[t]; }
  for (int t = 0; t < n; ++t) p[t] /= sum;
}

/* ------------------------------------------------------------------------ */
/* Cache access through the page table.                                       */
/* ------------------------------------------------------------------------ */
static const double* latent_row(const mla_oracle_problem_t* P, int b, int t) {
  int page = P->page_table[(size_t)b * P->max_pages + t / P->page_size];
  return P->latent_pool + ((size_t)page * P->page_size + (size_t)(t % P->page_size)) * P->d_c;
}

static const double* rope_row(const mla_oracle_problem_t* P, int b, int t) {
  int page = P->page_table[(size_t)b * P->max_pages + t / P->page_size];
  return P->rope_pool + ((size_t)page * P->page_size + (size_t)(t % P->page_size)) * P->d_r;
}

/* Copy the logical cache of sequence b (first n tokens) into contiguous
 * rows: C [n][d_c], KR [n][d_r]. */
void mla_oracle_gather(const mla_oracle_problem_t* P, int b, int n, double* C, double* KR) {
  for (int t = 0; t < n; ++t) {
    memcpy(C + (size_t)t * P->d_c, latent_row(P, b, t), sizeof(double) * (size_t)P->d_c);
    if (P->d_r > 0)
      memcpy(KR + (size_t)t * P->d_r, rope_row(P, b, t), sizeof(double) * (size_t)P->d_r);
  }
}

/* Argument check shared by both forms: returns 0 when usable. */
static int check_problem(const mla_oracle_problem_t* P, int n_sel, const int32_t* sel_b,
                         const int32_t* sel_head) {
  if (!P || P->batch < 0 || P->n_q < 1 || P->h < 1 || P->d_c < 1 || P->d_r < 0 ||
      P->d_h < 1 || P->page_size < 1 || P->max_pages < 1)
    return -1;
  for (int s = 0; s < n_sel; ++s) {
    int b = sel_b[s], i = sel_head[s];
    if (b < 0 || b >= P->batch || i < 0 || i >= P->h) return -2;
    int L = P->context_lens[b];
    if (L < P->n_q || L > P->max_pages * P->page_size) return -3;
    for (int j = 0; j < (L + P->page_size - 1) / P->page_size; ++j) {
      int pg = P->page_table[(size_t)b * P->max_pages + j];
      if (pg < 0 || pg >= P->num_pages) return -4;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Explicit form: rebuild K and V for every cached token, then attention.   */
/* ------------------------------------------------------------------------ */

/* Computes out[s][m][:] (d_h values) for every selected (sequence, head)
 * pair s and every query token m of that sequence.  Returns 0 on success. */
int mla_oracle_decode_explicit(const mla_oracle_problem_t* P, int n_sel,
                               const int32_t* sel_b, const int32_t* sel_head, double* out) {
  int rc = check_problem(P, n_sel, sel_b, sel_head);
  if (rc) return rc;
  const int d_c = P->d_c, d_r = P->d_r, d_h = P->d_h, n_q = P->n_q, h = P->h;
  const int dq = d_h + d_r; /* length of the concatenated query and key */
  int fail = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < n_sel; ++s) {
    const int b = sel_b[s], i = sel_head[s];
    const int L = P->context_lens[b];
    const double* Wk = P->w_uk + (size_t)i * d_h * d_c;
    const double* Wv = P->w_uv + (size_t)i * d_h * d_c;
    double* K = (double*)malloc(sizeof(double) * (size_t)L * dq);  /* [L][d_h + d_r] */
    double* V = (double*)malloc(sizeof(double) * (size_t)L * d_h); /* [L][d_h]       */
    double* sc = (double*)malloc(sizeof(double) * (size_t)L);
    double* p = (double*)malloc(sizeof(double) * (size_t)L);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dq);
    if (!K || !V || !sc || !p || !qt) {
#pragma omp atomic write
      fail = 1;
    } else {
      /* Per-head content key and value of every cached token, and the full
       * key [k_t ; k_R,t] with the shared RoPE key appended. */
      for (int t = 0; t < L; ++t) {
        const double* c = latent_row(P, b, t);
        mla_oracle_matvec(d_h, d_c, Wk, c, K + (size_t)t * dq);
        if (d_r > 0) memcpy(K + (size_t)t * dq + d_h, rope_row(P, b, t), sizeof(double) * d_r);
        mla_oracle_matvec(d_h, d_c, Wv, c, V + (size_t)t * d_h);
      }
      for (int m = 0; m < n_q; ++m) {
        const size_t row = (size_t)b * n_q + m;
        /* Full query [q ; q_R]. */
        memcpy(qt, P->q + (row * h + i) * d_h, sizeof(double) * d_h);
        if (d_r > 0) memcpy(qt + d_h, P->q_r + (row * h + i) * d_r, sizeof(double) * d_r);
        const int vis = L - n_q + m + 1; /* tokens 0 .. L - n_q + m */
        for (int t = 0; t < vis; ++t) sc[t] = P->scale * mla_oracle_dot(dq, qt, K + (size_t)t * dq);
        mla_oracle_softmax(vis, sc, p);
        double* o = out + ((size_t)s * n_q + m) * d_h;
        for (int a = 0; a < d_h; ++a) o[a] = 0.0;
        for (int t = 0; t < vis; ++t)
          for (int a = 0; a < d_h; ++a) o[a] += p[t] * V[(size_t)t * d_h + a];
      }
    }
    free(K); free(V); free(sc); free(p); free(qt);
  }
  return fail ? -5 : 0;
}

/* ------------------------------------------------------------------------ */
/* Absorbed form: each step on its own, then composed.                      */
/* ------------------------------------------------------------------------ */

/* Step 1: q_abs = W_UK_i^T q, W_UK_i is d_h x d_c. */
void mla_oracle_absorb_query(int d_h, int d_c, const double* w_uk_i, const double* q, double* q_abs) {
  mla_oracle_matvec_t(d_h, d_c, w_uk_i, q, q_abs);
}

/* Step 2: s_t = scale * (q_abs . C[t] + q_r . KR[t]) for t < n. */
void mla_oracle_latent_scores(int n, int d_c, int d_r, double scale, const double* q_abs,
                              const double* q_r, const double* C, const double* KR, double* s) {
  for (int t = 0; t < n; ++t) {
    double content = mla_oracle_dot(d_c, q_abs, C + (size_t)t * d_c);
    double rope = d_r > 0 ? mla_oracle_dot(d_r, q_r, KR + (size_t)t * d_r) : 0.0;
    s[t] = scale * (content + rope);
  }
}

/* Step 4: c_bar = sum_t p_t C[t]. */
void mla_oracle_weighted_latent(int n, int d_c, const double* p, const double* C, double* c_bar) {
  for (int f = 0; f < d_c; ++f) c_bar[f] = 0.0;
  for (int t = 0; t < n; ++t)
    for (int f = 0; f < d_c; ++f) c_bar[f] += p[t] * C[(size_t)t * d_c + f];
}

/* Step 5: o = W_UV_i c_bar. */
void mla_oracle_up_project(int d_h, int d_c, const double* w_uv_i, const double* c_bar, double* o) {
  mla_oracle_matvec(d_h, d_c, w_uv_i, c_bar, o);
}

/* Same outputs as the explicit form; also returns c_bar[s][m][:] (d_c values)
 * when cbar_out is not NULL.  The logical cache of a sequence is gathered
 * once and shared by all of its selected heads (the steps per head are the
 * ones above, unchanged). */
int mla_oracle_decode_absorbed(const mla_oracle_problem_t* P, int n_sel, const int32_t* sel_b,
                               const int32_t* sel_head, double* out, double* cbar_out) {
  int rc = check_problem(P, n_sel, sel_b, sel_head);
  if (rc) return rc;
  const int d_c = P->d_c, d_r = P->d_r, d_h = P->d_h, n_q = P->n_q, h = P->h;
  int fail = 0;
  char* done = (char*)calloc((size_t)(n_sel > 0 ? n_sel : 1), 1);
  if (!done) return -5;

  for (int s0 = 0; s0 < n_sel && !fail; ++s0) {
    if (done[s0]) continue;
    const int b = sel_b[s0];
    const int L = P->context_lens[b];
    double* C = (double*)malloc(sizeof(double) * (size_t)L * d_c);
    double* KR = (double*)malloc(sizeof(double) * ((size_t)L * (d_r > 0 ? d_r : 1)));
    if (!C || !KR) {
      fail = 1;
    } else {
      mla_oracle_gather(P, b, L, C, KR);
#pragma omp parallel for schedule(dynamic, 1)
      for (int s = s0; s < n_sel; ++s) {
        if (sel_b[s] != b) continue;
        done[s] = 1; /* each selection is handled by exactly one iteration */
        const int i = sel_head[s];
        double* sc = (double*)malloc(sizeof(double) * (size_t)L);
        double* p = (double*)malloc(sizeof(double) * (size_t)L);
        double* qa = (double*)malloc(sizeof(double) * (size_t)d_c);
        double* cb = (double*)malloc(sizeof(double) * (size_t)d_c);
        if (!sc || !p || !qa || !cb) {
#pragma omp atomic write
          fail = 1;
        } else {
          for (int m = 0; m < n_q; ++m) {
            const size_t row = (size_t)b * n_q + m;
            const int vis = L - n_q + m + 1;
            mla_oracle_absorb_query(d_h, d_c, P->w_uk + (size_t)i * d_h * d_c,
                                    P->q + (row * h + i) * d_h, qa);
            mla_oracle_latent_scores(vis, d_c, d_r, P->scale, qa,
                                     d_r > 0 ? P->q_r + (row * h + i) * d_r : NULL, C, KR, sc);
            mla_oracle_softmax(vis, sc, p);
            mla_oracle_weighted_latent(vis, d_c, p, C, cb);
            mla_oracle_up_project(d_h, d_c, P->w_uv + (size_t)i * d_h * d_c, cb,
                                  out + ((size_t)s * n_q + m) * d_h);
            if (cbar_out) memcpy(cbar_out + ((size_t)s * n_q + m) * d_c, cb, sizeof(double) * d_c);
          }
        }
        free(sc); free(p); free(qa); free(cb);
      }
    }
    free(C); free(KR);
  }
  free(done);
  return fail ? -5 : 0;
}

/* ------------------------------------------------------------------------ */
/* Output projection, the step after the decode path.                        */
/* ------------------------------------------------------------------------ */

/* u = [o_1 ; ... ; o_h] W^O for each of `rows` query rows.  The head
 * outputs of a row are concatenated head after head into one row vector of
 * k = h * d_h values and multiplied from the right by the output projection
 * W^O, a k x d matrix stored row-major ("From Vanilla Transformers to Modern
 * LLMs ... Part 3" sections 3.h and 3.p; "Multi-Head Latent Attention:
 * Low-Rank KV Compression, Decoupled RoPE, and Matrix Absorption", section
 * "Matrix Absorption", where the concatenated head outputs are multiplied by
 * W^O).  Written as the row vector's combination of the rows of W^O,
 * u[j] = sum_x o[x] W^O[x][j], summed in increasing x. */
void mla_oracle_output_project(int rows, int k, int d, const double* o, const double* w_o, double* u) {
  const int jb = 256;  /* columns per parallel block */
  const int nblk = (d + jb - 1) / jb;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int blk = 0; blk < nblk; ++blk) {
    const int j0 = blk * jb, j1 = j0 + jb < d ? j0 + jb : d;
    for (int r = 0; r < rows; ++r) {
      double* ur = u + (size_t)r * d;
      for (int j = j0; j < j1; ++j) ur[j] = 0.0;
      for (int x = 0; x < k; ++x) {
        const double ox = o[(size_t)r * k + x];
        const double* wx = w_o + (size_t)x * d;
        for (int j = j0; j < j1; ++j) ur[j] += ox * wx[j];
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Decoupled RoPE and the current token's projections (the steps before the */
/* decode path: what the cache and the query of a step are made from).      */
/* ------------------------------------------------------------------------ */

/* theta[j] = base^(-2 j / d) for the d/2 pairs j = 0 .. d/2 - 1: the pages'
 * theta_j = b^(-2 (j - 1) / d) with 1-based j ("MLA, dim by dim", the RoPE
 * paragraph of section 4). */
void mla_oracle_rope_thetas(int d, double base, double* theta) {
  for (int j = 0; j < d / 2; ++j) theta[j] = pow(base, -2.0 * j / d);
}

/* Rotary position embedding of a d-vector x at position t: each adjacent
 * pair (x[2j], x[2j+1]) is rotated by the angle t theta[j],
 *   y[2j]     = x[2j] cos(t theta_j) - x[2j+1] sin(t theta_j),
 *   y[2j + 1] = x[2j+1] cos(t theta_j) + x[2j] sin(t theta_j),
 * the element-wise form x cos + rotate_half(x) sin with rotate_half on
 * adjacent pairs ("MLA, dim by dim", RoPE paragraph of section 4); for one
 * pair and theta = pi/2 this is the toy rotation by 90 degrees per position
 * of "From Vanilla Transformers ... Part 3" (section "What RoPE does"). */
void mla_oracle_rope(int d, const double* x, double t, const double* theta, double* y) {
  for (int j = 0; j < d / 2; ++j) {
    const double a = t * theta[j], c = cos(a), s = sin(a);
    const double x0 = x[2 * j], x1 = x[2 * j + 1];
    y[2 * j] = x0 * c - x1 * s;
    y[2 * j + 1] = x1 * c + x0 * s;
  }
}

/* The cache append of one decode step.  For each of n new tokens r with
 * hidden state x[r] (d_model values), sequence seq[r] and position pos[r]:
 * the latent c = W_DKV x ([d_c][d_model] acting on a column vector;
 * "Multi-Head Latent Attention: ...", section "MLA: Low-Rank Key-Value
 * Joint Compression") and the decoupled RoPE key k_R = RoPE(W_KR x, pos)
 * ([d_r][d_model]; "MLA, dim by dim" section 5.2, the shared key cached
 * after rotation; "From Vanilla Transformers ..." sections 3.b and 3.k) go
 * to row pos % page_size of page page_table[seq][pos / page_size] of the
 * latent and RoPE pools.  Returns 0, or -1 when a row's page lies outside
 * the table or the pool. */
int mla_oracle_cache_append(int n, int d_model, int d_c, int d_r, const double* x, const double* w_dkv,
                            const double* w_kr, const int32_t* seq, const int32_t* pos, const double* theta,
                            const int32_t* page_table, int max_pages, int page_size, int num_pages,
                            double* latent_pool, double* rope_pool) {
  double* kr = (double*)malloc(sizeof(double) * (size_t)(d_r > 0 ? d_r : 1));
  int rc = 0;
  for (int r = 0; r < n && rc == 0; ++r) {
    const int j = pos[r] / page_size;
    const int page = (pos[r] >= 0 && j < max_pages) ? page_table[(size_t)seq[r] * max_pages + j] : -1;
    if (page < 0 || page >= num_pages) {
      rc = -1;
      break;
    }
    const size_t row = (size_t)page * page_size + (size_t)(pos[r] % page_size);
    const double* xr = x + (size_t)r * d_model;
    mla_oracle_matvec(d_c, d_model, w_dkv, xr, latent_pool + row * d_c);
    if (d_r > 0) {
      mla_oracle_matvec(d_r, d_model, w_kr, xr, kr);
      mla_oracle_rope(d_r, kr, (double)pos[r], theta, rope_pool + row * d_r);
    }
  }
  free(kr);
  return rc;
}

/* The query side of one decode step, for each of n query rows r with
 * hidden state x[r] and position pos[r]: the query latent c_Q = W_DQ x
 * ([d_qc][d_model]), then per head i the content query q_i = W_UQ[i] c_Q
 * ([h][d_h][d_qc]) and the RoPE query q_R,i = RoPE(W_QR[i] c_Q, pos)
 * ([h][d_r][d_qc]) ("Multi-Head Latent Attention: ...", the query
 * down-projection and per-head up-projections; "MLA, dim by dim" section
 * 4.3, the order (X W_DQ) W_UQ; "From Vanilla Transformers ..." sections
 * 3.d and 3.l).  q is [n][h][d_h], q_r [n][h][d_r]. */
void mla_oracle_query_project(int n, int d_model, int d_qc, int h, int d_h, int d_r, const double* x,
                              const double* w_dq, const double* w_uq, const double* w_qr, const int32_t* pos,
                              const double* theta, double* q, double* q_r) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int r = 0; r < n; ++r) {
    double* cq = (double*)malloc(sizeof(double) * (size_t)d_qc);
    double* qr0 = (double*)malloc(sizeof(double) * (size_t)(d_r > 0 ? d_r : 1));
    mla_oracle_matvec(d_qc, d_model, w_dq, x + (size_t)r * d_model, cq);
    for (int i = 0; i < h; ++i) {
      mla_oracle_matvec(d_h, d_qc, w_uq + (size_t)i * d_h * d_qc, cq, q + ((size_t)r * h + i) * d_h);
      if (d_r > 0) {
        mla_oracle_matvec(d_r, d_qc, w_qr + (size_t)i * d_r * d_qc, cq, qr0);
        mla_oracle_rope(d_r, qr0, (double)pos[r], theta, q_r + ((size_t)r * h + i) * d_r);
      }
    }
    free(cq);
    free(qr0);
  }
}

/* Sets the number of OpenMP threads later calls use (for timing the oracle
 * on a given number of cores; results do not depend on it). */
void mla_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Threads OpenMP will use for the parallel loops above (1 without OpenMP). */
int mla_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
