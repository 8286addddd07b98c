/*
 * dynconv_oracle.c -- plain fp64 CPU oracle of the dynamic short convolution
 * layer, forward and training backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes (source: "Dynamic Short Convolutions Improve
 * Transformers", gist.science Technical Summary, section Methodology ->
 * Dynamic Short Convolutions: the items Mechanism, Parameterization and
 * Placement; and section Efficient Training Implementation -> Fused Low-Rank
 * Kernel, which names the low-rank factors z and U and their product zU):
 *
 *   step 1  generator projection of the current hidden state h_t
 *             head-wise : u_t[e,j] = sum_i h_t[i] * W[i, e*k+j]
 *             low-rank  : z_t[q]   = sum_i h_t[i] * A[i, q]
 *                         v_t[c,j] = sum_q z_t[q] * U[q, c*k+j]
 *   step 2  per-position, per-channel filter
 *             w_t[c,j] = (u_t[head(c), j]  or  v_t[c,j]) + w0[c,j]
 *             head(c) = floor(c / (D / n_heads))   (consecutive-channel tying)
 *   step 3  causal depthwise conv with the residual added back
 *             y_t[c] = x_t[c] + sum_{j<k, t-j>=0} w_t[c,j] * x_{t-j}[c]
 *
 * Backward for L = sum dy*y (chain rule through steps 1-3):
 *   G_t[c,j]  = [t-j>=0] dy_t[c] * x_{t-j}[c]
 *   dx_s[c]   = dy_s[c] + sum_{j<k, s+j<=T-1} w_{s+j}[c,j] * dy_{s+j}[c]
 *   dw0[c,j]  = sum_{b,t} G_t[c,j]
 *   head-wise : du_t[e,j] = sum_{c in head e} G_t[c,j]
 *               dW[i,e*k+j] = sum_{b,t} h_t[i] du_t[e,j]
 *               dh_t[i] = sum_{e,j} du_t[e,j] W[i,e*k+j]
 *   low-rank  : dU[q,c*k+j] = sum_{b,t} z_t[q] G_t[c,j]
 *               dz_t[q] = sum_{c,j} G_t[c,j] U[q,c*k+j]
 *               dA[i,q] = sum_{b,t} h_t[i] dz_t[q]
 *               dh_t[i] = sum_q dz_t[q] A[i,q]
 *
 * Readings where the pages leave a step open (all listed with reasons in the
 * design notes): tap j is the lag (j = 0 is the current token); tokens before
 * the start of each sequence are zero, and no state crosses batch rows; the
 * bias w0 is per channel [D,k] and applies to both parameterisations; there
 * is no nonlinearity anywhere in the layer.
 *
 * Packed documents: a batch row may hold several documents back to back
 * (shape field doc: the document index of every token, or NULL for one
 * document per row).  The causal window then stops at the start of each
 * document exactly as it stops at the start of a row: a term that would
 * reach a token of another document counts as zero.  So in every test
 * above, "t-j >= 0" reads "t-j >= 0 and token t-j is in t's document", and
 * "s+j <= T-1" reads "s+j <= T-1 and token s+j is in s's document".  (The
 * pages are silent on packing; one of their off-subject abstracts names
 * document packing as the practical obstacle for convolutions, and the
 * Mechanism item fixes only that the window looks back.)
 *
 * Everything is fp64, row-major and contiguous:
 *   h[B,T,d]  x,y,dy,dx[B,T,D]  W[d, n_heads*k]  A[d,r]  U[r, D*k]  w0[D,k]
 *   w[B,T,D,k] (materialised here on purpose: this is the plain path)
 * Parallelism is OpenMP over independent output rows or entries only; each
 * output element is accumulated in the fixed order of its defining sum.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_HEADWISE = 0, ORC_LOWRANK = 1 };

typedef struct {
  int64_t B, T, d, D;
  int32_t k, kind, n_heads, rank;
  const int64_t *doc; /* [B*T] document index of each token, or NULL: one document per row */
} orc_shape;

/* Whether token rows r1 and r2 (flat indices into [B*T]) lie in one document;
 * the callers only ask about two rows of the same batch row. */
static int same_doc(const orc_shape *s, int64_t r1, int64_t r2) {
  return s->doc == NULL || s->doc[r1] == s->doc[r2];
}

enum { ORC_OK = 0, ORC_E_SHAPE = -1, ORC_E_NULL = -2 };

static int check_shape(const orc_shape *s) {
  if (!s) return ORC_E_NULL;
  if (s->B < 0 || s->T < 0 || s->d <= 0 || s->D <= 0 || s->k <= 0) return ORC_E_SHAPE;
  if (s->kind == ORC_HEADWISE) {
    if (s->n_heads <= 0 || s->D % s->n_heads != 0) return ORC_E_SHAPE;
  } else if (s->kind == ORC_LOWRANK) {
    if (s->rank <= 0) return ORC_E_SHAPE;
  } else {
    return ORC_E_SHAPE;
  }
  return ORC_OK;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Number of generator outputs per token: n_heads*k (head-wise) or r. */
static int64_t gen_cols(const orc_shape *s) {
  return s->kind == ORC_HEADWISE ? (int64_t)s->n_heads * s->k : (int64_t)s->rank;
}

/*
 * Steps 1 and 2.  Writes w[B*T, D, k]; if gen != NULL also the step-1
 * projection (u[B*T, n_heads*k] or z[B*T, r]).  w0 may be NULL (zero bias).
 */
int orc_filters(const orc_shape *s, const double *h, const double *W,
                const double *A, const double *U, const double *w0,
                double *w, double *gen) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!h || !w) return ORC_E_NULL;
  if (s->kind == ORC_HEADWISE && !W) return ORC_E_NULL;
  if (s->kind == ORC_LOWRANK && (!A || !U)) return ORC_E_NULL;
  const int64_t BT = s->B * s->T, d = s->d, D = s->D, k = s->k;
  const int64_t N = gen_cols(s);
  const int64_t hd = s->kind == ORC_HEADWISE ? D / s->n_heads : 0;

#pragma omp parallel
  {
    double *p = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < BT; ++t) {
      const double *ht = h + t * d;
      /* step 1: p = h_t . (W or A) */
      const double *M = s->kind == ORC_HEADWISE ? W : A;
      for (int64_t n = 0; n < N; ++n) p[n] = 0.0;
      for (int64_t i = 0; i < d; ++i) {
        const double hi = ht[i];
        const double *Mi = M + i * N;
        for (int64_t n = 0; n < N; ++n) p[n] += hi * Mi[n];
      }
      if (gen) memcpy(gen + t * N, p, sizeof(double) * (size_t)N);
      /* step 2: w_t[c,j] */
      double *wt = w + t * D * k;
      if (s->kind == ORC_HEADWISE) {
        for (int64_t c = 0; c < D; ++c) {
          const int64_t e = c / hd;
          for (int64_t j = 0; j < k; ++j) wt[c * k + j] = p[e * k + j];
        }
      } else {
        for (int64_t m = 0; m < D * k; ++m) wt[m] = 0.0;
        for (int64_t q = 0; q < N; ++q) {
          const double zq = p[q];
          const double *Uq = U + q * D * k;
          for (int64_t m = 0; m < D * k; ++m) wt[m] += zq * Uq[m];
        }
      }
      if (w0)
        for (int64_t m = 0; m < D * k; ++m) wt[m] += w0[m];
    }
    free(p);
  }
  return ORC_OK;
}

/* Step 3: y = x + causal depthwise conv of x with the per-token filters w. */
int orc_conv(const orc_shape *s, const double *w, const double *x, double *y) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!w || !x || !y) return ORC_E_NULL;
  const int64_t B = s->B, T = s->T, D = s->D, k = s->k;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < T; ++t) {
      const int64_t row = b * T + t;
      const double *wt = w + row * D * k;
      for (int64_t c = 0; c < D; ++c) {
        double acc = x[row * D + c];
        for (int64_t j = 0; j < k; ++j) {
          if (t - j < 0 || !same_doc(s, row, row - j)) break;
          acc += wt[c * k + j] * x[(row - j) * D + c];
        }
        y[row * D + c] = acc;
      }
    }
  return ORC_OK;
}

/*
 * Backward.  Inputs: h, the generator weights, x, the filters w from
 * orc_filters, and dy.  Outputs (each may be NULL to skip): dx[B,T,D],
 * dh[B,T,d], dW[d, n_heads*k] (head-wise) or dA[d,r] and dU[r, D*k]
 * (low-rank), dw0[D,k].  All outputs are overwritten.
 */
int orc_backward(const orc_shape *s, const double *h, const double *W,
                 const double *A, const double *U, const double *x,
                 const double *w, const double *dy, double *dx, double *dh,
                 double *dW, double *dA, double *dU, double *dw0) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!h || !x || !w || !dy) return ORC_E_NULL;
  if (s->kind == ORC_HEADWISE && !W) return ORC_E_NULL;
  if (s->kind == ORC_LOWRANK && (!A || !U)) return ORC_E_NULL;
  const int64_t B = s->B, T = s->T, BT = B * T, d = s->d, D = s->D, k = s->k;
  const int64_t N = gen_cols(s);

  /* dx: the transpose of step 3 (the residual contributes dy itself). */
  if (dx) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < T; ++t) {
        const int64_t row = b * T + t;
        for (int64_t c = 0; c < D; ++c) {
          double acc = dy[row * D + c];
          for (int64_t j = 0; j < k; ++j) {
            if (t + j > T - 1 || !same_doc(s, row, row + j)) break;
            acc += w[(row + j) * D * k + c * k + j] * dy[(row + j) * D + c];
          }
          dx[row * D + c] = acc;
        }
      }
  }

  /* G_t[c,j] = [t-j>=0, same document] dy_t[c] x_{t-j}[c], written out as a function. */
#define G_AT(b_, t_, c_, j_)                                                   \
  (((t_) - (j_) < 0 || !same_doc(s, (b_) * T + (t_), (b_) * T + (t_) - (j_)))  \
       ? 0.0                                                                   \
       : dy[((b_) * T + (t_)) * D + (c_)] * x[((b_) * T + (t_) - (j_)) * D + (c_)])

  if (dw0) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < D; ++c)
      for (int64_t j = 0; j < k; ++j) {
        double acc = 0.0;
        for (int64_t b = 0; b < B; ++b)
          for (int64_t t = 0; t < T; ++t) acc += G_AT(b, t, c, j);
        dw0[c * k + j] = acc;
      }
  }

  /* g = du (head-wise) or dz (low-rank), [BT, N]. */
  double *g = (double *)calloc((size_t)(BT > 0 ? BT : 1) * (size_t)N, sizeof(double));
  double *z = NULL;
  if (!g) return ORC_E_NULL;

  if (s->kind == ORC_HEADWISE) {
    const int64_t hd = D / s->n_heads;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < T; ++t) {
        double *gt = g + (b * T + t) * N;
        for (int64_t e = 0; e < s->n_heads; ++e)
          for (int64_t j = 0; j < k; ++j) {
            double acc = 0.0;
            for (int64_t c = e * hd; c < (e + 1) * hd; ++c) acc += G_AT(b, t, c, j);
            gt[e * k + j] = acc;
          }
      }
    if (dW) {
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < d; ++i) {
        double *dWi = dW + i * N;
        for (int64_t n = 0; n < N; ++n) dWi[n] = 0.0;
        for (int64_t t = 0; t < BT; ++t) {
          const double hi = h[t * d + i];
          const double *gt = g + t * N;
          for (int64_t n = 0; n < N; ++n) dWi[n] += hi * gt[n];
        }
      }
    }
  } else {
    /* recompute z = h A (step 1 of the forward) */
    z = (double *)calloc((size_t)(BT > 0 ? BT : 1) * (size_t)N, sizeof(double));
    if (!z) { free(g); return ORC_E_NULL; }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < BT; ++t)
      for (int64_t i = 0; i < d; ++i) {
        const double hi = h[t * d + i];
        for (int64_t q = 0; q < N; ++q) z[t * N + q] += hi * A[i * N + q];
      }
    /* dz_t[q] = sum_{c,j} G_t[c,j] U[q, c*k+j] */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < T; ++t) {
        double *gt = g + (b * T + t) * N;
        for (int64_t q = 0; q < N; ++q) {
          double acc = 0.0;
          for (int64_t c = 0; c < D; ++c)
            for (int64_t j = 0; j < k; ++j) acc += G_AT(b, t, c, j) * U[q * D * k + c * k + j];
          gt[q] = acc;
        }
      }
    /* dU[q, c*k+j] = sum_{b,t} z_t[q] G_t[c,j] */
    if (dU) {
#pragma omp parallel for schedule(static)
      for (int64_t c = 0; c < D; ++c) {
        for (int64_t q = 0; q < N; ++q)
          for (int64_t j = 0; j < k; ++j) dU[q * D * k + c * k + j] = 0.0;
        for (int64_t b = 0; b < B; ++b)
          for (int64_t t = 0; t < T; ++t) {
            const int64_t row = b * T + t;
            for (int64_t q = 0; q < N; ++q) {
              const double zq = z[row * N + q];
              for (int64_t j = 0; j < k; ++j) dU[q * D * k + c * k + j] += zq * G_AT(b, t, c, j);
            }
          }
      }
    }
    /* dA[i,q] = sum_{b,t} h_t[i] dz_t[q] */
    if (dA) {
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < d; ++i) {
        double *dAi = dA + i * N;
        for (int64_t q = 0; q < N; ++q) dAi[q] = 0.0;
        for (int64_t t = 0; t < BT; ++t) {
          const double hi = h[t * d + i];
          for (int64_t q = 0; q < N; ++q) dAi[q] += hi * g[t * N + q];
        }
      }
    }
  }
#undef G_AT

  /* dh_t[i] = sum_n g_t[n] M[i, n], with M = W (head-wise) or A (low-rank) */
  if (dh) {
    const double *M = s->kind == ORC_HEADWISE ? W : A;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < BT; ++t)
      for (int64_t i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += g[t * N + n] * M[i * N + n];
        dh[t * d + i] = acc;
      }
  }
  free(z);
  free(g);
  return ORC_OK;
}

/*
 * The producing projection the layer sits after (gist.science, Methodology ->
 * Dynamic Short Convolutions, Placement: the convolution is applied to the
 * query, key and value projections, or after any linear layer):
 *   x_t[c] = sum_i h_t[i] * Wp[i, c]        Wp[d, D]
 * The layer's input x is this projection of the same hidden state h that
 * generates the filter, so a fused implementation reads h once for both.
 */
int orc_proj(const orc_shape *s, const double *h, const double *Wp, double *x) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!h || !Wp || !x) return ORC_E_NULL;
  const int64_t BT = s->B * s->T, d = s->d, D = s->D;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < BT; ++t)
    for (int64_t c = 0; c < D; ++c) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; ++i) acc += h[t * d + i] * Wp[i * D + c];
      x[t * D + c] = acc;
    }
  return ORC_OK;
}
