/*
 * Host symmetric eigensolver for the Rayleigh-Ritz step of the subspace
 * iteration (plain C, float64; AVX2 + FMA, which the x86-64-v3 build target
 * guarantees).
 *
 *   H = Q T Q^T   Householder reduction to tridiagonal form T; Q is kept as
 *                 its reflectors;
 *   T = S L S^T   implicit symmetric QR steps with the Wilkinson shift and
 *                 bottom-up deflation; the plane rotations are recorded, not
 *                 applied while the iteration runs.
 *
 * The rotation and product kernels use AVX-512 where the CPU has it.  The reduction's
 * O(n^2) row passes can be shared by two threads (xkv_eigh_values_pair).
 *
 * Only the nvec wanted eigenvectors are formed: the recorded rotations are
 * applied, last first, to the nvec unit vectors that select the wanted columns
 * of S (rotations cost 6 nvec flops each instead of 6 n), then Q is applied to
 * the n x nvec result as blocks of reflectors in compact-WY form, whose products
 * run through a register-tiled matrix product.
 * References: Golub & Van Loan, Matrix Computations, the Householder vector
 * (section 5.1), the WY representation of a product of reflectors (section
 * 5.1.7), tridiagonalisation (section 8.3.1) and the implicit symmetric QR step
 * (section 8.3.3).
 */
#include <math.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>
#include <immintrin.h>
#include "host_eigh.h"

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

/* Two threads' meeting point: a spin barrier (a generation count), the failure flag of the
 * start and the worker's next job, all plain ints read and written through atomics or
 * ordered by the barrier. */
static void pair_wait(xkv_eigh_pair* pr) {
  const int g = __atomic_load_n(&pr->gen, __ATOMIC_ACQUIRE);
  if (__atomic_add_fetch(&pr->count, 1, __ATOMIC_ACQ_REL) == 2) {
    __atomic_store_n(&pr->count, 0, __ATOMIC_RELAXED);
    __atomic_store_n(&pr->gen, g + 1, __ATOMIC_RELEASE);
    return;
  }
  for (int spins = 0; __atomic_load_n(&pr->gen, __ATOMIC_ACQUIRE) == g; ++spins) {
    if (spins < 20000) _mm_pause();
    else sched_yield();   /* the partner is not running: give it the core */
  }
}

/* Row passes of the reduction, over local rows [i0, i1) of their trailing block; a pass
 * that forms a product adds its terms into pacc. */
enum { JOB_DONE = 0, JOB_COPY, JOB_SYM, JOB_PRODUCT, JOB_FUSED };
typedef struct {
  int n;
  const double* H;
  double* A;
  const double* V;
  const double* w;
  xkv_eigh_pair* pr;   /* NULL: one thread */
  double* p1;          /* the worker's product terms */
  double* cb;          /* a fused pass's first updated column, contiguous */
} team;

/* the rows a job covers: all n for the symmetrisation, else the trailing block's size */
static int job_rows(int job, int n, int k) {
  return job == JOB_COPY || job == JOB_SYM ? n : job == JOB_PRODUCT ? n - k - 1 : n - k - 2;
}
static int job_has_product(int job) { return job == JOB_PRODUCT || job == JOB_FUSED; }

static void job_pass(const team* t, int job, int k, int i0, int i1, double* pacc) {
  const int n = t->n;
  double* A = t->A;
  if (job == JOB_COPY) {
    /* H row by row (it may sit in memory the host reads slowly across rows, such as a
     * device's pinned staging) */
    for (int i = i0; i < i1; ++i) memcpy(A + (size_t)i * n, t->H + (size_t)i * n, (size_t)n * sizeof(double));
  } else if (job == JOB_SYM) {
    /* the lower triangle takes the mean of the two triangles (the upper one is read only) */
    for (int i = i0; i < i1; ++i)
      for (int j = 0; j < i; ++j) A[(size_t)i * n + j] = 0.5 * (A[(size_t)i * n + j] + A[(size_t)j * n + i]);
  } else if (job == JOB_PRODUCT) {
    /* pacc += A22 v from the lower triangle (rows and columns k+1..) */
    const double* v = t->V + (size_t)k * n;
    for (int i = i0; i < i1; ++i) {
      const double* row = A + (size_t)(k + 1 + i) * n + k + 1;
      const double vi = v[i];
      double s = 0.0;
      for (int j = 0; j < i; ++j) {
        s += row[j] * v[j];
        pacc[j] += row[j] * vi;
      }
      pacc[i] += s + row[i] * vi;
    }
  } else {
    /* the update of step k on local rows/columns 1..m-1 of its A22 (rows/columns 0..m2-1 of
     * the next A22) fused with the product by the next Householder vector v2; the updated
     * first column of the next A22 is copied out to cb */
    const double* v = t->V + (size_t)k * n;
    const double* v2 = v + n;
    const double* w = t->w;
    const double* vj = v + 1;
    const double* wj = w + 1;
    for (int i = i0; i < i1; ++i) {
      double* row = A + (size_t)(k + 2 + i) * n + k + 2;
      const double vi = v[i + 1], wi = w[i + 1], ui = v2[i];
      /* four-wide: a = row - vi w - wi v, then s += a v2 (four partial sums) and pacc += ui a */
      const __m256d vvi = _mm256_set1_pd(vi), vwi = _mm256_set1_pd(wi), vui = _mm256_set1_pd(ui);
      __m256d s4 = _mm256_setzero_pd();
      int j = 0;
      for (; j + 4 <= i; j += 4) {
        __m256d a = _mm256_fnmadd_pd(vvi, _mm256_loadu_pd(wj + j), _mm256_loadu_pd(row + j));
        a = _mm256_fnmadd_pd(vwi, _mm256_loadu_pd(vj + j), a);
        _mm256_storeu_pd(row + j, a);
        s4 = _mm256_fmadd_pd(a, _mm256_loadu_pd(v2 + j), s4);
        _mm256_storeu_pd(pacc + j, _mm256_fmadd_pd(a, vui, _mm256_loadu_pd(pacc + j)));
      }
      double s = 0.0;
      for (; j < i; ++j) {
        const double a = row[j] - vi * wj[j] - wi * vj[j];
        row[j] = a;
        s += a * v2[j];
        pacc[j] += a * ui;
      }
      {
        double part[4];
        _mm256_storeu_pd(part, s4);
        s += (part[0] + part[1]) + (part[2] + part[3]);
      }
      const double a = row[i] - vi * wj[i] - wi * vj[i];
      row[i] = a;
      pacc[i] += s + a * ui;
      t->cb[i] = row[0];
    }
  }
}

/* The leader runs a job: alone over all its rows, or with the worker taking the rows from
 * `split` on (row i of a triangle costs ~i, so the split at 1/sqrt(2) halves the work), their
 * product terms then added into p.  p[0, rows) is zero on entry for a product. */
static void run_job(const team* t, int job, int k, double* p) {
  const int rows = job_rows(job, t->n, k);
  if (!t->pr) {
    job_pass(t, job, k, 0, rows, p);
    return;
  }
  const int split = job == JOB_COPY ? rows / 2 : (int)(rows * 0.7071067811865476);   /* rows, or a triangle */
  t->pr->job = job;
  t->pr->k = k;
  t->pr->split = split;
  pair_wait(t->pr);   /* the job is published */
  job_pass(t, job, k, 0, split, p);
  pair_wait(t->pr);   /* both halves done */
  if (job_has_product(job))
    for (int i = 0; i < rows; ++i) p[i] += t->p1[i];
}

/* The worker's side of a paired reduction: jobs until JOB_DONE. */
static void worker_loop(const team* t) {
  for (;;) {
    pair_wait(t->pr);
    const int job = t->pr->job, k = t->pr->k, split = t->pr->split;
    if (job == JOB_DONE) return;
    const int rows = job_rows(job, t->n, k);
    if (job_has_product(job)) memset(t->p1, 0, (size_t)rows * sizeof(double));
    job_pass(t, job, k, split, rows, t->p1);
    pair_wait(t->pr);
  }
}

/* Reduce symmetric A (n x n, row-major, lower triangle used and overwritten) to
 * tridiagonal (d, e), A_in = Q T Q^T with Q = P_0 P_1 ... P_{n-3}, P_k = I - beta_k v_k v_k^T
 * acting on rows and columns k+1..n-1.  On return row k of V (n x n) holds v_k (v_k[0] = 1,
 * component i for row k+1+i) and beta[k] its factor.  p, w and u are n doubles of scratch,
 * t->cb too.
 *
 * Step k takes the Householder vector v of column k below the diagonal and forms
 * p = beta A22 v, w = p - (beta/2)(p.v) v; A22 <- A22 - v w^T - w v^T.  Only the lower
 * triangle of A22 is kept, and the update of step k is fused with the product of
 * step k + 1: once column k + 1 of the updated matrix is known (its Householder vector
 * v' follows), one pass over the rest of the lower triangle updates each element and
 * adds its contributions a_ij v'_j to p'_i and a_ij v'_i to p'_j.  That pass also copies the
 * first column of what it updated to cb, so the next step takes its column (and the one
 * after it) from contiguous memory: the column of A is not read again.  The O(n^2) passes
 * are jobs (run_job), shared with a worker thread when t->pr is set; the O(n) work of a step
 * stays in the calling thread. */
static void tridiagonalize(const team* t, double* d, double* e, double* V, double* beta, double* p, double* w,
                           double* u) {
  const int n = t->n;
  double* A = t->A;
  double* cb = t->cb;
  /* have_next: v_k, beta[k], d[k], e[k], p = A22 v_k and cb = column k+1 from k+1 down are
   * known from the step before */
  int have_next = 0;
  for (int k = 0; k + 2 < n; ++k) {
    const int m = n - k - 1;                 /* trailing size */
    double* v = V + (size_t)k * n;
    if (!have_next) {
      double mu;
      for (int i = 0; i < m; ++i) u[i] = A[(size_t)(k + 1 + i) * n + k];   /* column k below the diagonal */
      house(m, u, v, &beta[k], &mu);
      d[k] = A[(size_t)k * n + k];
      e[k] = mu;
      if (beta[k] == 0.0) continue;
      for (int i = 0; i < m; ++i) p[i] = 0.0;
      run_job(t, JOB_PRODUCT, k, p);
      for (int i = 0; i < m; ++i) cb[i] = A[(size_t)(k + 1 + i) * n + k + 1];
    }
    have_next = 0;
    const double b = beta[k];
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
      for (int i = 0; i < m; ++i) u[i] = cb[i] - (v[i] * w[0] + w[i] * v[0]);
      double mu2;
      house(m2, u + 1, v2, &beta[k + 1], &mu2);
      d[k + 1] = u[0];
      e[k + 1] = mu2;
      for (int i = 0; i < m2; ++i) p[i] = 0.0;
      run_job(t, JOB_FUSED, k, p);
      have_next = 1;
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
}

/* Rotation t of the log acts on rows/columns k[t], k[t] + 1 of the eigenvector matrix,
 * which becomes S <- S G_t with G_t = [c -s; s c] in that 2 x 2 block. */
typedef xkv_rotlog rotlog;

static int rotlog_push(rotlog* L, int k, double c, double s) {
  if (L->n == L->cap) {
    const long cap = L->cap ? 2 * L->cap : 4096;
    double* nc = (double*)realloc(L->c, (size_t)cap * sizeof(double));
    if (nc) L->c = nc;
    double* ns = (double*)realloc(L->s, (size_t)cap * sizeof(double));
    if (ns) L->s = ns;
    int* nk = (int*)realloc(L->k, (size_t)cap * sizeof(int));
    if (nk) L->k = nk;
    if (!nc || !ns || !nk) return -1;
    L->cap = cap;
  }
  L->c[L->n] = c;
  L->s[L->n] = s;
  L->k[L->n] = k;
  ++L->n;
  return 0;
}

/* One implicit QR step with Wilkinson shift on the unreduced block [l, m]; its rotations are
 * appended to the log.  Returns -1 if the log cannot grow. */
static int qr_step(double* d, double* e, rotlog* log, int l, int m) {
  const double delta = 0.5 * (d[m - 1] - d[m]);
  const double bb = e[m - 1];
  const double den = delta + copysign(hypot(delta, bb), delta == 0.0 ? 1.0 : delta);
  const double shift = d[m] - bb * bb / den;
  double x = d[l] - shift;
  double z = e[l];
  for (int k = l; k < m; ++k) {
    /* sqrt(x^2 + z^2) where neither square can overflow or lose the result to underflow;
     * hypot (slower, scaled) otherwise */
    double r = sqrt(x * x + z * z);
    if (!(r > 1e-150 && r < 1e150)) r = hypot(x, z);
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
    if (rotlog_push(log, k, c, s) != 0) return -1;
  }
  return 0;
}

/* S (n x ncol, row-major) <- G_1 G_2 ... G_N S: the logged rotations, last first, each on two
 * rows of S.  S is copied into panels of RC columns stored row after row.  The log splits into
 * runs in which k rises by one from each rotation to the next (a QR sweep); taken last first, a
 * run walks down the rows, so a run is applied to 16 columns at a time with the row shared by
 * consecutive rotations carried in registers: one row load and one row store per rotation.
 * P is n * RC doubles of scratch. */
/* AVX-512 (8 doubles per register) where the CPU has it: the rotation and product kernels
 * below have a 512-bit twin, chosen at run time; both give the same results element by
 * element (the same operations in the same order). */
static int have_avx512(void) { return __builtin_cpu_supports("avx512f"); }

enum { RC = 128 };   /* column panel of apply_rotations_reverse */
static void apply_rotations_reverse_avx512(const rotlog* L, int n, int ncol, double* S, double* P);
static void apply_rotations_reverse(const rotlog* L, int n, int ncol, double* S, double* P) {
  if (have_avx512()) {
    apply_rotations_reverse_avx512(L, n, ncol, S, P);
    return;
  }
  /* The wanted columns start as unit vectors; early rotations leave long runs of entries far
   * below 1e-300 that decay through the subnormal range, where x86 arithmetic is ~100 times
   * slower.  Subnormal results and inputs are taken as zero here (flush-to-zero and
   * denormals-are-zero, this thread only, restored on return): they change no entry by more
   * than 2.3e-308 of a unit vector. */
  const unsigned int csr = _mm_getcsr();
  _mm_setcsr(csr | 0x8040u);
  for (int j0 = 0; j0 < ncol; j0 += RC) {
    const int jw = ncol - j0 < RC ? ncol - j0 : RC;
    for (int i = 0; i < n; ++i) {
      memcpy(P + (size_t)i * RC, S + (size_t)i * ncol + j0, (size_t)jw * sizeof(double));
      for (int j = jw; j < RC; ++j) P[(size_t)i * RC + j] = 0.0;
    }
    for (long t = L->n - 1; t >= 0;) {
      long t0 = t;   /* the run: rotations t0 .. t, k[u] = k[t] - (t - u) */
      while (t0 > 0 && L->k[t0 - 1] == L->k[t0] - 1) --t0;
      const int ktop = L->k[t];
      for (int j = 0; j < RC; j += 16) {
        double* top = P + (size_t)(ktop + 1) * RC + j;
        __m256d y0 = _mm256_loadu_pd(top), y1 = _mm256_loadu_pd(top + 4), y2 = _mm256_loadu_pd(top + 8),
                y3 = _mm256_loadu_pd(top + 12);
        double* row = top;   /* row k + 1 of the current rotation */
        for (long u = t; u >= t0; --u) {
          double* xr = row - RC;   /* row k */
          const __m256d vc = _mm256_set1_pd(L->c[u]), vs = _mm256_set1_pd(L->s[u]);
          const __m256d x0 = _mm256_loadu_pd(xr), x1 = _mm256_loadu_pd(xr + 4), x2 = _mm256_loadu_pd(xr + 8),
                        x3 = _mm256_loadu_pd(xr + 12);
          /* row k + 1 <- s x + c y (final for this run); row k <- c x - s y (carried: one
           * dependent operation per rotation, c x is formed off the chain) */
          _mm256_storeu_pd(row, _mm256_fmadd_pd(vs, x0, _mm256_mul_pd(vc, y0)));
          _mm256_storeu_pd(row + 4, _mm256_fmadd_pd(vs, x1, _mm256_mul_pd(vc, y1)));
          _mm256_storeu_pd(row + 8, _mm256_fmadd_pd(vs, x2, _mm256_mul_pd(vc, y2)));
          _mm256_storeu_pd(row + 12, _mm256_fmadd_pd(vs, x3, _mm256_mul_pd(vc, y3)));
          y0 = _mm256_fnmadd_pd(vs, y0, _mm256_mul_pd(vc, x0));
          y1 = _mm256_fnmadd_pd(vs, y1, _mm256_mul_pd(vc, x1));
          y2 = _mm256_fnmadd_pd(vs, y2, _mm256_mul_pd(vc, x2));
          y3 = _mm256_fnmadd_pd(vs, y3, _mm256_mul_pd(vc, x3));
          row = xr;
        }
        _mm256_storeu_pd(row, y0);
        _mm256_storeu_pd(row + 4, y1);
        _mm256_storeu_pd(row + 8, y2);
        _mm256_storeu_pd(row + 12, y3);
      }
      t = t0 - 1;
    }
    for (int i = 0; i < n; ++i) memcpy(S + (size_t)i * ncol + j0, P + (size_t)i * RC, (size_t)jw * sizeof(double));
  }
  _mm_setcsr(csr);
}

/* apply_rotations_reverse with 32 columns (four 8-wide registers) per pass of a run. */
__attribute__((target("avx512f"))) static void apply_rotations_reverse_avx512(const rotlog* L, int n, int ncol,
                                                                             double* S, double* P) {
  const unsigned int csr = _mm_getcsr();
  _mm_setcsr(csr | 0x8040u);   /* flush subnormals, as in the AVX2 version */
  for (int j0 = 0; j0 < ncol; j0 += RC) {
    const int jw = ncol - j0 < RC ? ncol - j0 : RC;
    for (int i = 0; i < n; ++i) {
      memcpy(P + (size_t)i * RC, S + (size_t)i * ncol + j0, (size_t)jw * sizeof(double));
      for (int j = jw; j < RC; ++j) P[(size_t)i * RC + j] = 0.0;
    }
    for (long t = L->n - 1; t >= 0;) {
      long t0 = t;
      while (t0 > 0 && L->k[t0 - 1] == L->k[t0] - 1) --t0;
      const int ktop = L->k[t];
      for (int j = 0; j < RC; j += 32) {
        double* top = P + (size_t)(ktop + 1) * RC + j;
        __m512d y0 = _mm512_loadu_pd(top), y1 = _mm512_loadu_pd(top + 8), y2 = _mm512_loadu_pd(top + 16),
                y3 = _mm512_loadu_pd(top + 24);
        double* row = top;
        for (long u = t; u >= t0; --u) {
          double* xr = row - RC;
          const __m512d vc = _mm512_set1_pd(L->c[u]), vs = _mm512_set1_pd(L->s[u]);
          const __m512d x0 = _mm512_loadu_pd(xr), x1 = _mm512_loadu_pd(xr + 8), x2 = _mm512_loadu_pd(xr + 16),
                        x3 = _mm512_loadu_pd(xr + 24);
          _mm512_storeu_pd(row, _mm512_fmadd_pd(vs, x0, _mm512_mul_pd(vc, y0)));
          _mm512_storeu_pd(row + 8, _mm512_fmadd_pd(vs, x1, _mm512_mul_pd(vc, y1)));
          _mm512_storeu_pd(row + 16, _mm512_fmadd_pd(vs, x2, _mm512_mul_pd(vc, y2)));
          _mm512_storeu_pd(row + 24, _mm512_fmadd_pd(vs, x3, _mm512_mul_pd(vc, y3)));
          y0 = _mm512_fnmadd_pd(vs, y0, _mm512_mul_pd(vc, x0));
          y1 = _mm512_fnmadd_pd(vs, y1, _mm512_mul_pd(vc, x1));
          y2 = _mm512_fnmadd_pd(vs, y2, _mm512_mul_pd(vc, x2));
          y3 = _mm512_fnmadd_pd(vs, y3, _mm512_mul_pd(vc, x3));
          row = xr;
        }
        _mm512_storeu_pd(row, y0);
        _mm512_storeu_pd(row + 8, y1);
        _mm512_storeu_pd(row + 16, y2);
        _mm512_storeu_pd(row + 24, y3);
      }
      t = t0 - 1;
    }
    for (int i = 0; i < n; ++i) memcpy(S + (size_t)i * ncol + j0, P + (size_t)i * RC, (size_t)jw * sizeof(double));
  }
  _mm_setcsr(csr);
}

/* C (m x n) += sgn * A (m x k) B (k x n), row-major with leading dimensions lda, ldb, ldc.
 * The first n - n % 8 columns of B are first packed into Bp (k x (n - n % 8) doubles) as
 * panels of 8 columns, each panel's k rows contiguous; tiles of 4 rows x 8 columns of C are
 * then accumulated in registers over all of k, reading A's rows and one packed panel
 * front to back. */
static void gemm_acc_avx512(int m, int n, int k, double sgn, const double* A, int lda, const double* B, int ldb,
                            double* C, int ldc, double* Bp);
static void gemm_acc(int m, int n, int k, double sgn, const double* A, int lda, const double* B, int ldb,
                     double* C, int ldc, double* Bp) {
  if (have_avx512()) {
    gemm_acc_avx512(m, n, k, sgn, A, lda, B, ldb, C, ldc, Bp);
    return;
  }
  const int m4 = m & ~3, n8 = n & ~7;
  for (int j0 = 0; j0 < n8; j0 += 8) {
    double* panel = Bp + (size_t)j0 * k;
    for (int q = 0; q < k; ++q) {
      _mm256_storeu_pd(panel + 8 * q, _mm256_loadu_pd(B + (size_t)q * ldb + j0));
      _mm256_storeu_pd(panel + 8 * q + 4, _mm256_loadu_pd(B + (size_t)q * ldb + j0 + 4));
    }
  }
  const __m256d vsg = _mm256_set1_pd(sgn);
  for (int i0 = 0; i0 < m4; i0 += 4) {
    const double* a0 = A + (size_t)i0 * lda;
    for (int j0 = 0; j0 < n8; j0 += 8) {
      __m256d c00 = _mm256_setzero_pd(), c01 = _mm256_setzero_pd(), c10 = _mm256_setzero_pd(),
              c11 = _mm256_setzero_pd(), c20 = _mm256_setzero_pd(), c21 = _mm256_setzero_pd(),
              c30 = _mm256_setzero_pd(), c31 = _mm256_setzero_pd();
      const double* bp = Bp + (size_t)j0 * k;
      for (int q = 0; q < k; ++q, bp += 8) {
        const __m256d b0 = _mm256_loadu_pd(bp), b1 = _mm256_loadu_pd(bp + 4);
        __m256d av = _mm256_broadcast_sd(a0 + q);
        c00 = _mm256_fmadd_pd(av, b0, c00);
        c01 = _mm256_fmadd_pd(av, b1, c01);
        av = _mm256_broadcast_sd(a0 + lda + q);
        c10 = _mm256_fmadd_pd(av, b0, c10);
        c11 = _mm256_fmadd_pd(av, b1, c11);
        av = _mm256_broadcast_sd(a0 + 2 * (size_t)lda + q);
        c20 = _mm256_fmadd_pd(av, b0, c20);
        c21 = _mm256_fmadd_pd(av, b1, c21);
        av = _mm256_broadcast_sd(a0 + 3 * (size_t)lda + q);
        c30 = _mm256_fmadd_pd(av, b0, c30);
        c31 = _mm256_fmadd_pd(av, b1, c31);
      }
      double* cp = C + (size_t)i0 * ldc + j0;
      _mm256_storeu_pd(cp, _mm256_fmadd_pd(vsg, c00, _mm256_loadu_pd(cp)));
      _mm256_storeu_pd(cp + 4, _mm256_fmadd_pd(vsg, c01, _mm256_loadu_pd(cp + 4)));
      cp += ldc;
      _mm256_storeu_pd(cp, _mm256_fmadd_pd(vsg, c10, _mm256_loadu_pd(cp)));
      _mm256_storeu_pd(cp + 4, _mm256_fmadd_pd(vsg, c11, _mm256_loadu_pd(cp + 4)));
      cp += ldc;
      _mm256_storeu_pd(cp, _mm256_fmadd_pd(vsg, c20, _mm256_loadu_pd(cp)));
      _mm256_storeu_pd(cp + 4, _mm256_fmadd_pd(vsg, c21, _mm256_loadu_pd(cp + 4)));
      cp += ldc;
      _mm256_storeu_pd(cp, _mm256_fmadd_pd(vsg, c30, _mm256_loadu_pd(cp)));
      _mm256_storeu_pd(cp + 4, _mm256_fmadd_pd(vsg, c31, _mm256_loadu_pd(cp + 4)));
    }
  }
  /* ragged edges: the last n % 8 columns of the tiled rows, then the last m % 4 rows */
  for (int i = 0; i < m; ++i) {
    const int j_from = i < m4 ? n8 : 0;
    for (int j = j_from; j < n; ++j) {
      double t = 0.0;
      for (int q = 0; q < k; ++q) t += A[(size_t)i * lda + q] * B[(size_t)q * ldb + j];
      C[(size_t)i * ldc + j] += sgn * t;
    }
  }
}

/* gemm_acc with panels of 16 columns and tiles of 4 rows x 16 columns (eight 8-wide
 * accumulators); the ragged edges as there. */
__attribute__((target("avx512f"))) static void gemm_acc_avx512(int m, int n, int k, double sgn, const double* A,
                                                              int lda, const double* B, int ldb, double* C, int ldc,
                                                              double* Bp) {
  const int m4 = m & ~3, n16 = n & ~15;
  for (int j0 = 0; j0 < n16; j0 += 16) {
    double* panel = Bp + (size_t)j0 * k;
    for (int q = 0; q < k; ++q) {
      _mm512_storeu_pd(panel + 16 * q, _mm512_loadu_pd(B + (size_t)q * ldb + j0));
      _mm512_storeu_pd(panel + 16 * q + 8, _mm512_loadu_pd(B + (size_t)q * ldb + j0 + 8));
    }
  }
  const __m512d vsg = _mm512_set1_pd(sgn);
  for (int i0 = 0; i0 < m4; i0 += 4) {
    const double* a0 = A + (size_t)i0 * lda;
    for (int j0 = 0; j0 < n16; j0 += 16) {
      __m512d c00 = _mm512_setzero_pd(), c01 = _mm512_setzero_pd(), c10 = _mm512_setzero_pd(),
              c11 = _mm512_setzero_pd(), c20 = _mm512_setzero_pd(), c21 = _mm512_setzero_pd(),
              c30 = _mm512_setzero_pd(), c31 = _mm512_setzero_pd();
      const double* bp = Bp + (size_t)j0 * k;
      for (int q = 0; q < k; ++q, bp += 16) {
        const __m512d b0 = _mm512_loadu_pd(bp), b1 = _mm512_loadu_pd(bp + 8);
        __m512d av = _mm512_set1_pd(a0[q]);
        c00 = _mm512_fmadd_pd(av, b0, c00);
        c01 = _mm512_fmadd_pd(av, b1, c01);
        av = _mm512_set1_pd(a0[lda + q]);
        c10 = _mm512_fmadd_pd(av, b0, c10);
        c11 = _mm512_fmadd_pd(av, b1, c11);
        av = _mm512_set1_pd(a0[2 * (size_t)lda + q]);
        c20 = _mm512_fmadd_pd(av, b0, c20);
        c21 = _mm512_fmadd_pd(av, b1, c21);
        av = _mm512_set1_pd(a0[3 * (size_t)lda + q]);
        c30 = _mm512_fmadd_pd(av, b0, c30);
        c31 = _mm512_fmadd_pd(av, b1, c31);
      }
      double* cp = C + (size_t)i0 * ldc + j0;
      _mm512_storeu_pd(cp, _mm512_fmadd_pd(vsg, c00, _mm512_loadu_pd(cp)));
      _mm512_storeu_pd(cp + 8, _mm512_fmadd_pd(vsg, c01, _mm512_loadu_pd(cp + 8)));
      cp += ldc;
      _mm512_storeu_pd(cp, _mm512_fmadd_pd(vsg, c10, _mm512_loadu_pd(cp)));
      _mm512_storeu_pd(cp + 8, _mm512_fmadd_pd(vsg, c11, _mm512_loadu_pd(cp + 8)));
      cp += ldc;
      _mm512_storeu_pd(cp, _mm512_fmadd_pd(vsg, c20, _mm512_loadu_pd(cp)));
      _mm512_storeu_pd(cp + 8, _mm512_fmadd_pd(vsg, c21, _mm512_loadu_pd(cp + 8)));
      cp += ldc;
      _mm512_storeu_pd(cp, _mm512_fmadd_pd(vsg, c30, _mm512_loadu_pd(cp)));
      _mm512_storeu_pd(cp + 8, _mm512_fmadd_pd(vsg, c31, _mm512_loadu_pd(cp + 8)));
    }
  }
  for (int i = 0; i < m; ++i) {
    const int j_from = i < m4 ? n16 : 0;
    for (int j = j_from; j < n; ++j) {
      double t = 0.0;
      for (int q = 0; q < k; ++q) t += A[(size_t)i * lda + q] * B[(size_t)q * ldb + j];
      C[(size_t)i * ldc + j] += sgn * t;
    }
  }
}

/* S (n x ncol, row-major) <- Q S with Q = P_0 P_1 ... P_{n-3} the reflectors of
 * tridiagonalize, taken from the right end in blocks of NB: P_kb ... P_{kb+nb-1} =
 * I - Y T Y^T (compact WY; Y holds the reflectors, T is upper triangular), applied to rows
 * kb+1.. as S2 -= Y (T (Y^T S2)).  scr holds reflector_scratch(n, ncol) doubles. */
enum { NB = 32 };   /* reflectors per compact-WY block */
static size_t reflector_scratch(int n, int ncol) {
  return (size_t)NB * NB + 2 * (size_t)NB * n + 2 * (size_t)NB * ncol + NB + (size_t)n * ncol;
}
static void apply_reflectors(int n, const double* V, const double* beta, int ncol, double* S, double* scr) {
  const int nref = n - 2;   /* reflectors 0 .. n-3 */
  if (nref <= 0) return;
  double* Tm = scr;                          /* NB x NB */
  double* Yt = Tm + (size_t)NB * NB;         /* Y^T: reflector c in row c (NB x n) */
  double* Yr = Yt + (size_t)NB * n;          /* Y, row-major (n x NB) */
  double* W = Yr + (size_t)n * NB;           /* NB x ncol */
  double* W2 = W + (size_t)NB * ncol;        /* NB x ncol */
  double* tw = W2 + (size_t)NB * ncol;       /* NB */
  double* Bp = tw + NB;                      /* packed panels of the products (n x ncol) */
  for (int kb = ((nref - 1) / NB) * NB; kb >= 0; kb -= NB) {
    const int nb = nref - kb < NB ? nref - kb : NB;
    const int r0 = kb + 1, M = n - r0;
    /* Yt[c][i] = component of reflector kb+c at row r0 + i (zero above its start) */
    for (int c = 0; c < nb; ++c) {
      double* y = Yt + (size_t)c * n;
      const double* v = V + (size_t)(kb + c) * n;
      for (int i = 0; i < M; ++i) y[i] = i < c ? 0.0 : v[i - c];
    }
    for (int i = 0; i < M; ++i)
      for (int c = 0; c < nb; ++c) Yr[(size_t)i * NB + c] = Yt[(size_t)c * n + i];
    /* T: T[c][c] = beta_c, T[0:c, c] = -beta_c T[0:c, 0:c] (Y[:, 0:c]^T y_c) */
    for (int c = 0; c < nb; ++c) {
      const double bc = beta[kb + c];
      const double* yc = Yt + (size_t)c * n;
      for (int a = 0; a < c; ++a) {
        const double* ya = Yt + (size_t)a * n;
        double t = 0.0;
        for (int i = c; i < M; ++i) t += ya[i] * yc[i];
        tw[a] = t;
      }
      for (int a = 0; a < c; ++a) {
        double t = 0.0;
        for (int b2 = a; b2 < c; ++b2) t += Tm[a * NB + b2] * tw[b2];
        Tm[a * NB + c] = -bc * t;
      }
      Tm[c * NB + c] = bc;
      for (int a = c + 1; a < NB; ++a) Tm[a * NB + c] = 0.0;
    }
    double* S2 = S + (size_t)r0 * ncol;
    /* W = Y^T S2 (nb x ncol); W2 = T W; S2 -= Y W2 */
    memset(W, 0, (size_t)nb * ncol * sizeof(double));
    gemm_acc(nb, ncol, M, 1.0, Yt, n, S2, ncol, W, ncol, Bp);
    memset(W2, 0, (size_t)nb * ncol * sizeof(double));
    gemm_acc(nb, ncol, nb, 1.0, Tm, NB, W, ncol, W2, ncol, Bp);
    gemm_acc(M, ncol, nb, -1.0, Yr, NB, W2, ncol, S2, ncol, Bp);
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

/* The value phase's state in sc->buf: A (n x n), V (n x n), then vectors of n doubles at
 * slot(buf, n, S_*); the eigenvalue order (keyed) takes two slots. */
enum { S_BETA, S_D, S_E, S_P, S_W, S_COL, S_IDX, S_CB = S_IDX + 2, S_SLOTS };
static double* slot(double* buf, int n, int s) { return buf + 2 * (size_t)n * n + (size_t)s * n; }

/* Value phase: all n eigenvalues of symmetric H, descending, into w; the reflectors, the
 * rotation log and the order of the eigenvalues stay in sc for xkv_eigh_vectors.  sc keeps its
 * memory for the next call (a zero-filled struct on first use; xkv_eigh_scratch_release frees
 * it): repeated solves in several threads then neither map nor fault pages.  With pr set the
 * calling thread leads a pair whose worker runs worker_side; the worker's product terms are in
 * helper->buf, read only after the start barrier.  Returns 0 on success, -1 on
 * allocation failure, -2 if the QR iteration did not converge, -4 if H (the mean of its
 * triangles) has an entry that is not finite. */
static int values_impl(int n, const double* H, int nvec, double* w, xkv_eigh_scratch* sc, xkv_eigh_pair* pr,
                       const xkv_eigh_scratch* helper) {
  const size_t need = 2 * (size_t)n * n + S_SLOTS * (size_t)n;
  if (sc->cap < need) {
    free(sc->buf);
    sc->buf = (double*)malloc(need * sizeof(double));
    sc->cap = sc->buf ? need : 0;
  }
  if (pr) {
    /* both threads learn whether either lacks memory before any shared work */
    if (!sc->buf) __atomic_store_n(&pr->fail, 1, __ATOMIC_RELAXED);
    pair_wait(pr);
    if (__atomic_load_n(&pr->fail, __ATOMIC_RELAXED)) return -1;
  }
  if (!sc->buf) return -1;
  sc->n = n;
  sc->nvec = nvec;
  double* A = sc->buf;
  double* V = A + (size_t)n * n;
  double* beta = slot(sc->buf, n, S_BETA);
  double* d = slot(sc->buf, n, S_D);
  double* e = slot(sc->buf, n, S_E);
  double* tp = slot(sc->buf, n, S_P);
  double* tw = slot(sc->buf, n, S_W);
  double* tcol = slot(sc->buf, n, S_COL);
  keyed* idx = (keyed*)slot(sc->buf, n, S_IDX);
  memset(beta, 0, (size_t)n * sizeof(double));
  memset(e, 0, (size_t)n * sizeof(double));
  rotlog* log = &sc->log;
  log->n = 0;
  const team t = {n, H, A, V, tw, pr, pr ? helper->buf : NULL, slot(sc->buf, n, S_CB)};
  run_job(&t, JOB_COPY, 0, NULL);
  run_job(&t, JOB_SYM, 0, NULL);
  int finite = 1;
  for (int i = 0; i < n && finite; ++i)
    for (int j = 0; j <= i; ++j)
      if (!isfinite(A[(size_t)i * n + j])) {
        finite = 0;
        break;
      }
  if (finite) tridiagonalize(&t, d, e, V, beta, tp, tw, tcol);
  if (pr) {
    pr->job = JOB_DONE;
    pair_wait(pr);   /* the worker leaves */
  }
  if (!finite) return -4;

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
      if (qr_step(d, e, log, l, m) != 0) return -1;
      if (--budget < 0) return -2;
    }
  }

  for (int i = 0; i < n; ++i) { idx[i].key = d[i]; idx[i].idx = i; }
  qsort(idx, (size_t)n, sizeof(keyed), cmp_desc);
  for (int j = 0; j < n; ++j) w[j] = idx[j].key;
  return 0;
}

__attribute__((visibility("hidden"))) int xkv_eigh_values(int n, const double* H, int nvec, double* w,
                                                           xkv_eigh_scratch* sc) {
  if (n <= 0 || nvec <= 0 || nvec > n) return -3;
  return values_impl(n, H, nvec, w, sc, NULL, NULL);
}

/* The worker of a pair: its product terms in helper->buf, the shared state in the leader's sc
 * (read only after the start barrier, once the leader has its memory). */
static int worker_side(int n, const double* H, const xkv_eigh_scratch* sc, xkv_eigh_scratch* helper,
                       xkv_eigh_pair* pr, double* refl) {
  if (helper->cap < (size_t)n) {
    free(helper->buf);
    helper->buf = (double*)malloc((size_t)n * sizeof(double));
    helper->cap = helper->buf ? (size_t)n : 0;
  }
  if (!helper->buf) __atomic_store_n(&pr->fail, 1, __ATOMIC_RELAXED);
  pair_wait(pr);
  if (__atomic_load_n(&pr->fail, __ATOMIC_RELAXED)) return -1;
  double* A = sc->buf;
  const team t = {n, H, A, A + (size_t)n * n, slot(sc->buf, n, S_W), pr, helper->buf, slot(sc->buf, n, S_CB)};
  worker_loop(&t);
  /* the reflectors are final once the reduction is; the leader's QR iteration leaves them */
  if (refl) xkv_eigh_pack_reflectors(sc, refl);
  return 0;
}

__attribute__((visibility("hidden"))) int xkv_eigh_values_pair(int n, const double* H, int nvec, double* w,
                                                                xkv_eigh_scratch* sc, xkv_eigh_scratch* helper,
                                                                xkv_eigh_pair* pr, int tid, double* refl) {
  if (n <= 0 || nvec <= 0 || nvec > n) return -3;
  if (tid) return worker_side(n, H, sc, helper, pr, refl);
  return values_impl(n, H, nvec, w, sc, pr, helper);
}

/* Vector phase: Z[:, j0:j1] = Q G_1 ... G_N E, E the unit vectors of the wanted positions: the
 * rotations on E (last first), then the reflectors, in `work`'s memory, then one copy into Z
 * (which may be pinned host memory, slower to work in). */
__attribute__((visibility("hidden"))) int xkv_eigh_vectors(const xkv_eigh_scratch* state, int j0, int j1,
                                                            double* Z, xkv_eigh_scratch* work) {
  const int n = state->n, nvec = state->nvec, nc = j1 - j0;
  if (nc <= 0) return 0;
  const double* V = state->buf + (size_t)n * n;
  const double* beta = slot(state->buf, n, S_BETA);
  const keyed* idx = (const keyed*)slot(state->buf, n, S_IDX);
  const size_t need = (size_t)n * RC + reflector_scratch(n, nc) + (size_t)n * nc;
  if (work->vcap < need) {
    free(work->vbuf);
    work->vbuf = (double*)malloc(need * sizeof(double));
    work->vcap = work->vbuf ? need : 0;
    if (!work->vbuf) return -1;
  }
  double* panel = work->vbuf;
  double* rscr = panel + (size_t)n * RC;
  double* Zw = rscr + reflector_scratch(n, nc);
  memset(Zw, 0, (size_t)n * nc * sizeof(double));
  for (int j = j0; j < j1; ++j) Zw[(size_t)idx[j].idx * nc + (j - j0)] = 1.0;
  apply_rotations_reverse(&state->log, n, nc, Zw, panel);
  apply_reflectors(n, V, beta, nc, Zw, rscr);
  for (int i = 0; i < n; ++i) memcpy(Z + (size_t)i * nvec + j0, Zw + (size_t)i * nc, (size_t)nc * sizeof(double));
  return 0;
}

/* All n eigenvalues of symmetric H, descending, into w (length n); the eigenvectors of the
 * nvec largest as the columns of Z (n x nvec): the two phases in the calling thread. */
__attribute__((visibility("hidden"))) int xkv_eigh_desc_scratch(int n, const double* H, int nvec, double* w,
                                                                 double* Z, xkv_eigh_scratch* sc) {
  const int rc = xkv_eigh_values(n, H, nvec, w, sc);
  if (rc) return rc;
  return xkv_eigh_vectors(sc, 0, nvec, Z, sc);
}

/* The vector phase's inputs for a device, which forms column j of Z as the unit vector at
 * pos[j], then applies the logged rotations last first, a run at a time (a run is one QR sweep:
 * rotations t_lo..t_hi, rotation t on rows k_top - (t_hi - t) and the one below), then the
 * reflectors as blocks of XKV_EIGH_NBG, last block first, each as I - Y T Y^T.  A QR sweep
 * longer than maxlen rotations is cut into runs of at most maxlen (any cut gives the same
 * product). */
__attribute__((visibility("hidden"))) int xkv_eigh_runs(const xkv_eigh_scratch* st, int maxlen) {
  const rotlog* L = &st->log;
  int runs = 0;
  long t0 = 0;
  for (long t = 0; t < L->n; ++t)
    if (t == 0 || L->k[t] != L->k[t - 1] + 1 || t - t0 == maxlen) {
      ++runs;
      t0 = t;
    }
  return runs;
}

__attribute__((visibility("hidden"))) void xkv_eigh_pack_log(const xkv_eigh_scratch* st, int maxlen, int* runs,
                                                              double* cs) {
  const rotlog* L = &st->log;
  int q = -1;
  long t0 = 0;
  for (long t = 0; t < L->n; ++t) {
    if (t == 0 || L->k[t] != L->k[t - 1] + 1 || t - t0 == maxlen) {
      t0 = t;
      ++q;
      runs[4 * q] = (int)t;
      runs[4 * q + 3] = 0;
    }
    runs[4 * q + 1] = (int)t;        /* t_hi so far */
    runs[4 * q + 2] = L->k[t];       /* k_top: the row of rotation t_hi */
    cs[2 * t] = L->c[t];
    cs[2 * t + 1] = L->s[t];
  }
}

/* Fronts a device sweeps for group g = (q0, nb): from the highest start front (run b starts at
 * its top row minus b) to the lowest end front. */
static int group_fronts(const int* runs, const int* g) {
  int f0 = 0, f1 = 0;
  for (int b = 0; b < g[1]; ++b) {
    const int* R = runs + 4 * (g[0] - b);
    const int ab = R[2] - b, zb = R[2] - (R[1] - R[0]) - b;
    f0 = b ? (ab > f0 ? ab : f0) : ab;
    f1 = b ? (zb < f1 ? zb : f1) : zb;
  }
  return f0 - f1 + 1;
}

/* Groups of up to B runs that a device applies together, in the order they are applied (the
 * log's last run first): a group is runs q0, q0 - 1, ..., q0 - nb + 1, run b of it starting when
 * the front row is its top row minus b and ending when the front is its lowest row minus b.  A
 * run joins the group while every run's start and end stay within `spread` rows of the group's
 * first start and last end and the group spans at most maxsteps fronts.  groups: (q0, nb) pairs;
 * returns their number. */
__attribute__((visibility("hidden"))) int xkv_eigh_group_runs(const int* runs, int nruns, int B, int spread,
                                                               int maxsteps, int* groups) {
  int ng = 0;
  for (int q = nruns - 1; q >= 0;) {
    int f0 = 0, f1 = 0, nb = 0;
    int a[64], z[64];
    for (; nb < B && nb < 64 && q - nb >= 0; ++nb) {
      const int* R = runs + 4 * (q - nb);
      const int ab = R[2] - nb, zb = R[2] - (R[1] - R[0]) - nb;   /* start and end fronts */
      const int g0 = nb ? (ab > f0 ? ab : f0) : ab, g1 = nb ? (zb < f1 ? zb : f1) : zb;
      int ok = g0 - g1 + 1 <= maxsteps;
      a[nb] = ab;
      z[nb] = zb;
      for (int b = 0; b <= nb && ok; ++b) ok = g0 - a[b] <= spread && z[b] - g1 <= spread;
      if (!ok) break;
      f0 = g0;
      f1 = g1;
    }
    if (nb == 0) nb = 1;   /* a lone run always fits */
    groups[2 * ng] = q;
    groups[2 * ng + 1] = nb;
    ++ng;
    q -= nb;
  }
  return ng;
}

/* Cut a side's groups (in the order they are applied) into `parts` consecutive pieces of about
 * equal work: group q costs the fronts it sweeps (from its runs' first to last front, as a
 * device applies it) plus `overhead`.  bounds[p] is piece p's first group, bounds[parts] =
 * ngroups; pieces may be empty. */
__attribute__((visibility("hidden"))) void xkv_eigh_split_groups(const int* runs, const int* groups, int ngroups,
                                                                  int overhead, int parts, int* bounds) {
  long total = 0;
  for (int q = 0; q < ngroups; ++q) total += overhead + group_fronts(runs, groups + 2 * q);
  bounds[0] = 0;
  long acc = 0;
  int q = 0;
  for (int p = 1; p < parts; ++p) {
    /* the first group whose work before it reaches p / parts of the total */
    const long target = (total * p + parts - 1) / parts;
    while (q < ngroups && acc < target) acc += overhead + group_fronts(runs, groups + 2 * q++);
    bounds[p] = q;
  }
  bounds[parts] = ngroups;
}

__attribute__((visibility("hidden"))) size_t xkv_eigh_refl_doubles(int n) {
  const int nref = n - 2;
  if (nref <= 0) return 0;
  const int nblk = (nref + XKV_EIGH_NBG - 1) / XKV_EIGH_NBG;
  size_t y = 0;
  for (int b = 0; b < nblk; ++b) y += (size_t)(n - XKV_EIGH_NBG * b - 1) * XKV_EIGH_NBG;
  return y + (size_t)nblk * XKV_EIGH_NBG * XKV_EIGH_NBG;
}

/* Block b holds reflectors kb = NBG b .. kb + nb - 1 acting on rows r0 = kb + 1 .. n - 1:
 * Y_b (M = n - r0 rows of NBG, row-major; column c is reflector kb + c from its row c on, zero
 * above it and for c >= nb), the blocks one after another, then every T_b (NBG x NBG,
 * row-major, upper triangular) with P_kb ... P_{kb+nb-1} = I - Y_b T_b Y_b^T:
 * T[c][c] = beta_c, T[0:c, c] = -beta_c T[0:c, 0:c] (Y_b^T Y_b)[0:c, c]. */
__attribute__((visibility("hidden"))) void xkv_eigh_pack_reflectors(const xkv_eigh_scratch* st, double* out) {
  enum { NBG = XKV_EIGH_NBG };
  const int n = st->n, nref = n - 2;
  if (nref <= 0) return;
  const double* V = st->buf + (size_t)n * n;
  const double* beta = slot(st->buf, n, S_BETA);
  const int nblk = (nref + NBG - 1) / NBG;
  double* T = out + (xkv_eigh_refl_doubles(n) - (size_t)nblk * NBG * NBG);
  double* Y = out;
  for (int b = 0; b < nblk; ++b) {
    const int kb = NBG * b, nb = nref - kb < NBG ? nref - kb : NBG, M = n - kb - 1;
    double G[NBG][NBG];
    memset(G, 0, sizeof(G));
    for (int i = 0; i < M; ++i) {
      double* y = Y + (size_t)i * NBG;
      for (int c = 0; c < NBG; ++c) y[c] = (c < nb && i >= c) ? V[(size_t)(kb + c) * n + (i - c)] : 0.0;
      for (int a = 0; a < NBG; ++a)
        for (int c = a + 1; c < NBG; ++c) G[a][c] += y[a] * y[c];
    }
    double* Tb = T + (size_t)b * NBG * NBG;
    memset(Tb, 0, sizeof(double) * NBG * NBG);
    for (int c = 0; c < nb; ++c) {
      const double bc = beta[kb + c];
      for (int a = 0; a < c; ++a) {
        double t = 0.0;
        for (int b2 = a; b2 < c; ++b2) t += Tb[a * NBG + b2] * G[b2][c];
        Tb[a * NBG + c] = -bc * t;
      }
      Tb[c * NBG + c] = bc;
    }
    Y += (size_t)M * NBG;
  }
}

__attribute__((visibility("hidden"))) void xkv_eigh_positions(const xkv_eigh_scratch* st, int* pos) {
  const keyed* idx = (const keyed*)slot(st->buf, st->n, S_IDX);
  for (int j = 0; j < st->nvec; ++j) pos[j] = idx[j].idx;
}

__attribute__((visibility("hidden"))) void xkv_eigh_scratch_release(xkv_eigh_scratch* sc) {
  free(sc->buf);
  free(sc->vbuf);
  free(sc->log.c);
  free(sc->log.s);
  free(sc->log.k);
  memset(sc, 0, sizeof(*sc));
}

/* As xkv_eigh_desc_scratch with memory of its own, freed on return. */
__attribute__((visibility("hidden"))) int xkv_eigh_desc_impl(int n, const double* H, int nvec, double* w,
                                                              double* Z) {
  xkv_eigh_scratch sc;
  memset(&sc, 0, sizeof(sc));
  const int rc = xkv_eigh_desc_scratch(n, H, nvec, w, Z, &sc);
  xkv_eigh_scratch_release(&sc);
  return rc;
}
