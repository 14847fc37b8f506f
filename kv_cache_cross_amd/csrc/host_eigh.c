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

/* Reduce symmetric A (n x n, row-major, overwritten) to tridiagonal (d, e).
 * On return Qt holds Q^T, where A_in = Q T Q^T. */
static int tridiagonalize(int n, double* A, double* d, double* e, double* Qt) {
  double* V = (double*)calloc((size_t)n * n, sizeof(double));   /* reflector k in row k */
  double* beta = (double*)calloc((size_t)n, sizeof(double));
  double* p = (double*)malloc((size_t)n * sizeof(double));
  double* w = (double*)malloc((size_t)n * sizeof(double));
  double* Q = (double*)malloc((size_t)n * n * sizeof(double));
  if (!V || !beta || !p || !w || !Q) {
    free(V); free(beta); free(p); free(w); free(Q);
    return -1;
  }
  for (int k = 0; k + 2 < n; ++k) {
    const int m = n - k - 1;                 /* trailing size */
    double* v = V + (size_t)k * n;
    double mu;
    /* Column k below the diagonal equals row k right of the diagonal (symmetry). */
    house(m, A + (size_t)k * n + k + 1, v, &beta[k], &mu);
    d[k] = A[(size_t)k * n + k];
    e[k] = mu;
    const double b = beta[k];
    if (b == 0.0) continue;
    /* p = beta * A22 v */
    for (int i = 0; i < m; ++i) {
      const double* row = A + (size_t)(k + 1 + i) * n + k + 1;
      double s = 0.0;
      for (int j = 0; j < m; ++j) s += row[j] * v[j];
      p[i] = b * s;
    }
    /* w = p - (beta/2)(p^T v) v */
    double pv = 0.0;
    for (int i = 0; i < m; ++i) pv += p[i] * v[i];
    const double half = 0.5 * b * pv;
    for (int i = 0; i < m; ++i) w[i] = p[i] - half * v[i];
    /* A22 -= v w^T + w v^T */
    for (int i = 0; i < m; ++i) {
      double* row = A + (size_t)(k + 1 + i) * n + k + 1;
      const double vi = v[i], wi = w[i];
      for (int j = 0; j < m; ++j) row[j] -= vi * w[j] + wi * v[j];
    }
  }
  if (n >= 2) {
    d[n - 2] = A[(size_t)(n - 2) * n + n - 2];
    e[n - 2] = A[(size_t)(n - 2) * n + n - 1];
  }
  d[n - 1] = A[(size_t)(n - 1) * n + n - 1];

  /* Q = P_0 P_1 ... P_{n-3}, accumulated from the right end. */
  for (size_t i = 0; i < (size_t)n * n; ++i) Q[i] = 0.0;
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  for (int k = n - 3; k >= 0; --k) {
    const int m = n - k - 1;
    const double* v = V + (size_t)k * n;
    const double b = beta[k];
    if (b == 0.0) continue;
    /* u = v^T Q22 ; Q22 -= beta v u^T */
    for (int j = 0; j < m; ++j) w[j] = 0.0;
    for (int i = 0; i < m; ++i) {
      const double* row = Q + (size_t)(k + 1 + i) * n + k + 1;
      const double vi = v[i];
      for (int j = 0; j < m; ++j) w[j] += vi * row[j];
    }
    for (int i = 0; i < m; ++i) {
      double* row = Q + (size_t)(k + 1 + i) * n + k + 1;
      const double f = b * v[i];
      for (int j = 0; j < m; ++j) row[j] -= f * w[j];
    }
  }
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) Qt[(size_t)j * n + i] = Q[(size_t)i * n + j];

  free(V); free(beta); free(p); free(w); free(Q);
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
