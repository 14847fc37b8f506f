/*
 * Host symmetric eigensolver for the Rayleigh-Ritz step of the subspace
 * iteration (plain C, float64).
 *
 *   H = Q T Q^T   Householder reduction to tridiagonal form T, with Q
 *                 accumulated backwards from the stored reflectors;
 *   T = S L S^T   implicit symmetric QR steps with the Wilkinson shift and
 *                 bottom-up deflation, every rotation also applied to Q.
 *
 * The eigenvectors of H are the columns of Q S.  They are kept as the rows of
 * Qt = (Q S)^T so that each plane rotation touches two contiguous rows.
 * References: Golub & Van Loan, Matrix Computations, the Householder vector
 * (section 5.1), tridiagonalisation (section 8.3.1) and the implicit
 * symmetric QR step (section 8.3.3).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Householder vector for x (length m): v[0] = 1, P = I - beta v v^T, P x = mu e_1, mu = |x|. */
static void house(int m, const double* x, double* v, double* beta, double* mu) {
  double sigma = 0.0;
  for (int i = 1; i < m; ++i) sigma += x[i] * x[i];
  v[0] = 1.0;
  for (int i = 1; i < m; ++i) v[i] = x[i];
  if (sigma == 0.0) {
    *beta = (x[0] < 0.0) ? 2.0 : 0.0;
    *mu = fabs(x[0]);
    return;
  }
  double nrm = sqrt(x[0] * x[0] + sigma);
  double v0 = (x[0] <= 0.0) ? x[0] - nrm : -sigma / (x[0] + nrm);
  *beta = 2.0 * v0 * v0 / (sigma + v0 * v0);
  for (int i = 1; i < m; ++i) v[i] /= v0;
  *mu = nrm;
}

/* Reduce symmetric A (n x n, row-major, lower triangle used and overwritten) to
 * tridiagonal (d, e).  On return Qt holds Q^T, where A_in = Q T Q^T.
 *
 * Step k takes the Householder vector v of column k below the diagonal and forms
 * p = beta A22 v, w = p - (beta/2)(p.v) v; A22 <- A22 - v w^T - w v^T.  Only the lower
 * triangle of A22 is kept, and the update of step k is fused with the product of
 * step k + 1: once column k + 1 of the updated matrix is known (its Householder vector
 * v' follows), one pass over the rest of the lower triangle updates each element and
 * adds its contributions a_ij v'_j to p'_i and a_ij v'_i to p'_j. */
static int tridiagonalize(int n, double* A, double* d, double* e, double* Qt) {
  double* V = (double*)calloc((size_t)n * n, sizeof(double));   /* reflector k in row k */
  double* beta = (double*)calloc((size_t)n, sizeof(double));
  double* p = (double*)malloc((size_t)n * sizeof(double));
  double* w = (double*)malloc((size_t)n * sizeof(double));
  double* col = (double*)malloc((size_t)n * sizeof(double));
  double* Q = (double*)malloc((size_t)n * n * sizeof(double));
  if (!V || !beta || !p || !w || !col || !Q) {
    free(V); free(beta); free(p); free(w); free(col); free(Q);
    return -1;
  }
  /* Step 0's product: p = A22 v over the (not yet updated) lower triangle. */
  int have_p = 0;
  for (int k = 0; k + 2 < n; ++k) {
    const int m = n - k - 1;                 /* trailing size */
    double* v = V + (size_t)k * n;
    double mu;
    for (int i = 0; i < m; ++i) col[i] = A[(size_t)(k + 1 + i) * n + k];   /* column k below the diagonal */
    house(m, col, v, &beta[k], &mu);
    d[k] = A[(size_t)k * n + k];
    e[k] = mu;
    const double b = beta[k];
    if (!have_p) {
      /* p = A22 v from the lower triangle (rows k+1.., columns k+1..) */
      for (int i = 0; i < m; ++i) p[i] = 0.0;
      for (int i = 0; i < m; ++i) {
        const double* row = A + (size_t)(k + 1 + i) * n + k + 1;
        const double vi = v[i];
        double s = 0.0;
        for (int j = 0; j < i; ++j) {
          s += row[j] * v[j];
          p[j] += row[j] * vi;
        }
        p[i] += s + row[i] * vi;
      }
    }
    have_p = 0;
    if (b == 0.0) continue;
    /* w = beta p - (beta/2)(beta p . v) v */
    for (int i = 0; i < m; ++i) p[i] *= b;
    double pv = 0.0;
    for (int i = 0; i < m; ++i) pv += p[i] * v[i];
    const double half = 0.5 * b * pv;
    for (int i = 0; i < m; ++i) w[i] = p[i] - half * v[i];
    if (k + 3 < n) {
      /* Column k+1 of the updated matrix (local index 0 of A22), then the next
       * Householder vector, then the fused update + product over local rows 1.. */
      const int m2 = m - 1;
      double* v2 = V + (size_t)(k + 1) * n;
      for (int i = 0; i < m; ++i) {
        double* a0 = A + (size_t)(k + 1 + i) * n + k + 1;
        *a0 -= v[i] * w[0] + w[i] * v[0];
      }
      for (int i = 0; i < m2; ++i) col[i] = A[(size_t)(k + 2 + i) * n + k + 1];
      double mu2;
      house(m2, col, v2, &beta[k + 1], &mu2);
      /* local rows/columns 1..m-1 of A22 are rows/columns 0..m2-1 of the next A22 */
      for (int i = 0; i < m2; ++i) p[i] = 0.0;
      for (int i = 0; i < m2; ++i) {
        double* row = A + (size_t)(k + 2 + i) * n + k + 2;
        const double vi = v[i + 1], wi = w[i + 1], ui = v2[i];
        const double* vj = v + 1;
        const double* wj = w + 1;
        double s = 0.0;
        for (int j = 0; j < i; ++j) {
          const double a = row[j] - vi * wj[j] - wi * vj[j];
          row[j] = a;
          s += a * v2[j];
          p[j] += a * ui;
        }
        const double a = row[i] - vi * wj[i] - wi * vj[i];
        row[i] = a;
        p[i] += s + a * ui;
      }
      have_p = 1;
      /* the next step recomputes its column k+2.. from A (already updated above) and
       * reuses v2 and beta[k + 1] through V and beta (house is deterministic) */
    } else {
      for (int i = 0; i < m; ++i) {
        double* row = A + (size_t)(k + 1 + i) * n + k + 1;
        const double vi = v[i], wi = w[i];
        for (int j = 0; j <= i; ++j) row[j] -= vi * w[j] + wi * v[j];
      }
    }
  }
  if (n >= 2) {
    d[n - 2] = A[(size_t)(n - 2) * n + n - 2];
    e[n - 2] = A[(size_t)(n - 1) * n + n - 2];
  }
  d[n - 1] = A[(size_t)(n - 1) * n + n - 1];

  /* Q = P_0 P_1 ... P_{n-3}, accumulated from the right end in blocks of NB reflectors:
   * P_kb ... P_{kb+nb-1} = I - Y T Y^T (compact WY; Y holds the reflectors, T is upper
   * triangular), applied as Q22 -= Y (T (Y^T Q22)) with Q22 = rows and columns kb+1...
   * Columns are taken in panels of QC so that the nb x QC product stays in cache. */
  for (size_t i = 0; i < (size_t)n * n; ++i) Q[i] = 0.0;
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  {
    enum { NB = 32, QC = 128 };
    double* Tm = (double*)malloc((size_t)NB * NB * sizeof(double));
    double* Wp = (double*)malloc((size_t)NB * QC * sizeof(double));
    double* Yt = (double*)malloc((size_t)NB * n * sizeof(double));   /* Y^T: reflector c in row c */
    if (!Tm || !Wp || !Yt) {
      free(Tm); free(Wp); free(Yt);
      free(V); free(beta); free(p); free(w); free(col); free(Q);
      return -1;
    }
    const int nref = n - 2;   /* reflectors 0 .. n-3 */
    for (int kb = ((nref - 1) / NB) * NB; kb >= 0; kb -= NB) {
      const int nb = nref - kb < NB ? nref - kb : NB;
      const int r0 = kb + 1, M = n - r0;
      /* Yt[c][i] = component of reflector kb+c at row r0 + i (zero above its start) */
      for (int c = 0; c < nb; ++c) {
        double* y = Yt + (size_t)c * n;
        const double* v = V + (size_t)(kb + c) * n;
        for (int i = 0; i < M; ++i) y[i] = i < c ? 0.0 : v[i - c];
      }
      /* T: T[c][c] = beta_c, T[0:c, c] = -beta_c T[0:c, 0:c] (Y[:, 0:c]^T y_c) */
      for (int c = 0; c < nb; ++c) {
        const double bc = beta[kb + c];
        const double* yc = Yt + (size_t)c * n;
        for (int a = 0; a < c; ++a) {
          const double* ya = Yt + (size_t)a * n;
          double t = 0.0;
          for (int i = c; i < M; ++i) t += ya[i] * yc[i];
          w[a] = t;
        }
        for (int a = 0; a < c; ++a) {
          double t = 0.0;
          for (int b2 = a; b2 < c; ++b2) t += Tm[a * NB + b2] * w[b2];
          Tm[a * NB + c] = -bc * t;
        }
        Tm[c * NB + c] = bc;
        for (int a = c + 1; a < NB; ++a) Tm[a * NB + c] = 0.0;
      }
      for (int j0 = 0; j0 < M; j0 += QC) {
        const int jw = M - j0 < QC ? M - j0 : QC;
        /* Wp = Y^T Q22[:, j0:j0+jw] */
        for (int c = 0; c < nb; ++c)
          for (int j = 0; j < jw; ++j) Wp[c * QC + j] = 0.0;
        for (int i = 0; i < M; ++i) {
          const double* row = Q + (size_t)(r0 + i) * n + r0 + j0;
          for (int c = 0; c < nb; ++c) {
            const double yci = Yt[(size_t)c * n + i];
            if (yci == 0.0) continue;
            double* wc = Wp + c * QC;
            for (int j = 0; j < jw; ++j) wc[j] += yci * row[j];
          }
        }
        /* Wp = T Wp (upper triangular, in place, top row first) */
        for (int a = 0; a < nb; ++a) {
          double* wa = Wp + a * QC;
          const double taa = Tm[a * NB + a];
          for (int j = 0; j < jw; ++j) wa[j] *= taa;
          for (int b2 = a + 1; b2 < nb; ++b2) {
            const double tab = Tm[a * NB + b2];
            const double* wb = Wp + b2 * QC;
            for (int j = 0; j < jw; ++j) wa[j] += tab * wb[j];
          }
        }
        /* Q22[:, j0:j0+jw] -= Y Wp */
        for (int i = 0; i < M; ++i) {
          double* row = Q + (size_t)(r0 + i) * n + r0 + j0;
          for (int c = 0; c < nb; ++c) {
            const double yci = Yt[(size_t)c * n + i];
            if (yci == 0.0) continue;
            const double* wc = Wp + c * QC;
            for (int j = 0; j < jw; ++j) row[j] -= yci * wc[j];
          }
        }
      }
    }
    free(Tm); free(Wp); free(Yt);
  }
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) Qt[(size_t)j * n + i] = Q[(size_t)i * n + j];

  free(V); free(beta); free(p); free(w); free(col); free(Q);
  return 0;
}

/* Rows k, k+1 of Qt <- [c s; -s c] applied to them (columns k, k+1 of Q). */
static void rotate_rows(int n, double* Qt, int k, double c, double s) {
  double* a = Qt + (size_t)k * n;
  double* b = a + n;
  for (int j = 0; j < n; ++j) {
    const double x = a[j], y = b[j];
    a[j] = c * x + s * y;
    b[j] = c * y - s * x;
  }
}

/* One implicit QR step with Wilkinson shift on the unreduced block [l, m]. */
static void qr_step(int n, double* d, double* e, double* Qt, int l, int m) {
  const double delta = 0.5 * (d[m - 1] - d[m]);
  const double bb = e[m - 1];
  const double den = delta + copysign(hypot(delta, bb), delta == 0.0 ? 1.0 : delta);
  const double shift = d[m] - bb * bb / den;
  double x = d[l] - shift;
  double z = e[l];
  for (int k = l; k < m; ++k) {
    const double r = hypot(x, z);
    double c = 1.0, s = 0.0;
    if (r != 0.0) { c = x / r; s = z / r; }
    if (k > l) e[k - 1] = r;
    const double a = d[k], b = e[k], dd = d[k + 1];
    d[k] = c * c * a + 2.0 * c * s * b + s * s * dd;
    d[k + 1] = s * s * a - 2.0 * c * s * b + c * c * dd;
    e[k] = c * s * (dd - a) + (c * c - s * s) * b;
    if (k + 1 < m) {
      z = s * e[k + 1];        /* bulge at (k, k+2) */
      e[k + 1] *= c;
      x = e[k];
    }
    rotate_rows(n, Qt, k, c, s);
  }
}

typedef struct { double key; int idx; } keyed;
static int cmp_desc(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return x->idx - y->idx;
}

/* All n eigenvalues of symmetric H, descending, into w (length n); the eigenvectors of the
 * nvec largest as the columns of Z (n x nvec).  Returns 0 on success, -1 on allocation
 * failure, -2 if the QR iteration did not converge. */
__attribute__((visibility("hidden"))) int xkv_eigh_desc_impl(int n, const double* H, int nvec, double* w,
                                                              double* Z) {
  if (n <= 0 || nvec <= 0 || nvec > n) return -3;
  double* A = (double*)malloc((size_t)n * n * sizeof(double));
  double* Qt = (double*)malloc((size_t)n * n * sizeof(double));
  double* d = (double*)malloc((size_t)n * sizeof(double));
  double* e = (double*)calloc((size_t)n, sizeof(double));
  keyed* idx = (keyed*)malloc((size_t)n * sizeof(keyed));
  int rc = 0;
  if (!A || !Qt || !d || !e || !idx) { rc = -1; goto done; }
  /* Symmetrise: use the mean of the two triangles. */
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j)
      A[(size_t)i * n + j] = 0.5 * (H[(size_t)i * n + j] + H[(size_t)j * n + i]);
  if (tridiagonalize(n, A, d, e, Qt) != 0) { rc = -1; goto done; }

  {
    const double eps = 2.220446049250313e-16;
    double tnorm = 0.0;
    for (int i = 0; i < n; ++i) tnorm = fmax(tnorm, fabs(d[i]) + (i + 1 < n ? fabs(e[i]) : 0.0));
    const double tiny = eps * eps * (tnorm > 0 ? tnorm : 1.0);
    long budget = 60L * n + 100;
    int m = n - 1;
    while (m > 0) {
      if (fabs(e[m - 1]) <= eps * (fabs(d[m - 1]) + fabs(d[m])) || fabs(e[m - 1]) <= tiny) {
        e[m - 1] = 0.0;
        --m;
        continue;
      }
      int l = m - 1;
      while (l > 0 && fabs(e[l - 1]) > eps * (fabs(d[l - 1]) + fabs(d[l])) && fabs(e[l - 1]) > tiny) --l;
      if (l > 0) e[l - 1] = 0.0;
      qr_step(n, d, e, Qt, l, m);
      if (--budget < 0) { rc = -2; goto done; }
    }
  }

  for (int i = 0; i < n; ++i) { idx[i].key = d[i]; idx[i].idx = i; }
  qsort(idx, (size_t)n, sizeof(keyed), cmp_desc);
  for (int j = 0; j < n; ++j) w[j] = idx[j].key;
  for (int j = 0; j < nvec; ++j) {
    const double* v = Qt + (size_t)idx[j].idx * n;
    for (int i = 0; i < n; ++i) Z[(size_t)i * nvec + j] = v[i];
  }
done:
  free(A); free(Qt); free(d); free(e); free(idx);
  return rc;
}
