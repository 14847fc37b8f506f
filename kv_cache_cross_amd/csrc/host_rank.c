/*
 * Rank diagnostics of a spectrum (plain C, float64), from the eigenvalues of a
 * side's Gram C = X^T X (the squared singular values of X):
 *
 *   energy rank   the smallest k whose k largest eigenvalues hold a fraction f of
 *                 the total (xKV blog, figure 2(c): the rank that keeps 95 % of
 *                 the cumulative eigenvalues); works on a leading part of the
 *                 spectrum when the total (trace of C) is given;
 *   effective rank and NER (KV-CoRE, section 2.B): exp of the entropy of the
 *                 singular values sigma_i / sum_j sigma_j over the numerical rank
 *                 r (sigma_i > n * eps * sigma_1), and erank / r; they need the
 *                 whole spectrum.
 */
#include <float.h>
#include <math.h>
#include <stdlib.h>

static int desc_cmp(const void* a, const void* b) {
  const double x = *(const double*)a, y = *(const double*)b;
  return (x < y) - (x > y);
}

/* Returns 0, or -1 when out of host memory.  vals: n eigenvalues (any order). */
int xkv_rank_stats_impl(const double* vals, int n, double total, double frac, int complete, int* energy_rank,
                        double* covered, int* num_rank, double* erank, double* ner) {
  double* lam = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  if (!lam) return -1;
  for (int i = 0; i < n; ++i) lam[i] = vals[i] > 0.0 ? vals[i] : 0.0;
  qsort(lam, (size_t)n, sizeof(double), desc_cmp);
  /* Summed in the same (descending) order as the cumulative sums below, so that
   * frac = 1 of the spectrum's own total is reached exactly. */
  double sum = 0.0;
  for (int i = 0; i < n; ++i) sum += lam[i];
  const double tot = total > 0.0 ? total : sum;
  *covered = tot > 0.0 ? sum / tot : 0.0;
  *energy_rank = -1;
  if (tot <= 0.0) {
    *energy_rank = 0;
  } else {
    double c = 0.0;
    for (int i = 0; i < n; ++i) {
      c += lam[i];
      if (c >= frac * tot) {
        *energy_rank = i + 1;
        break;
      }
    }
  }
  *num_rank = -1;
  *erank = NAN;
  *ner = NAN;
  if (complete) {
    int k = 0;
    const double s1 = n > 0 ? sqrt(lam[0]) : 0.0;
    if (s1 > 0.0) {
      const double cut = (double)n * DBL_EPSILON * s1;
      while (k < n && sqrt(lam[k]) > cut) ++k;
    }
    *num_rank = k;
    if (k == 0) {
      *erank = 0.0;
      *ner = 0.0;
    } else {
      double ssum = 0.0;
      for (int i = 0; i < k; ++i) ssum += sqrt(lam[i]);
      double h = 0.0;
      for (int i = 0; i < k; ++i) {
        const double p = sqrt(lam[i]) / ssum;
        h -= p * log(p);
      }
      *erank = exp(h);
      *ner = *erank / k;
    }
  }
  free(lam);
  return 0;
}

/*
 * Adaptive rank at a fixed budget (KV-CoRE, implications: compressibility differs
 * across layers and should guide a layer-aware compression strategy).  Side s keeps
 * r_s of its leading eigenvalues, r_s a multiple of `granule` in [r_min, r_max], with
 * sum r_s <= budget, so as to keep the most energy sum_s sum_{i < r_s} lambda_i^(s)
 * (by Eckart-Young, the least total squared reconstruction error).  Because each
 * side's eigenvalues are non-increasing, so are the energies of its successive
 * granules, and taking granules one at a time from the side whose next granule holds
 * the most energy (ties to the lower side) reaches the optimum.
 *
 * eig: n_sides rows of ld >= r_max values, each row descending.  Returns 0, -1 (bad
 * arguments or a budget below r_min on every side) or -2 (out of host memory).
 */
int xkv_rank_allocate_impl(const double* eig, int n_sides, int ld, int r_max, long budget, int granule, int r_min,
                           int* ranks, double* kept) {
  if (!eig || !ranks || n_sides <= 0 || granule <= 0 || r_min < 0 || r_min % granule || r_max % granule ||
      r_min > r_max || ld < r_max || budget < (long)n_sides * r_min)
    return -1;
  double* next = (double*)malloc(sizeof(double) * (size_t)n_sides);
  if (!next) return -2;
  double total = 0.0;
  long left = budget;
  for (int s = 0; s < n_sides; ++s) {
    ranks[s] = r_min;
    for (int i = 0; i < r_min; ++i) total += eig[(long)s * ld + i] > 0.0 ? eig[(long)s * ld + i] : 0.0;
    left -= r_min;
  }
  /* energy of the granule after side s's current rank (-1 when at r_max) */
  for (int s = 0; s < n_sides; ++s) {
    double e = -1.0;
    if (ranks[s] < r_max) {
      e = 0.0;
      for (int i = ranks[s]; i < ranks[s] + granule; ++i) e += eig[(long)s * ld + i] > 0.0 ? eig[(long)s * ld + i] : 0.0;
    }
    next[s] = e;
  }
  while (left >= granule) {
    int best = -1;
    for (int s = 0; s < n_sides; ++s)
      if (next[s] >= 0.0 && (best < 0 || next[s] > next[best])) best = s;
    if (best < 0) break;
    total += next[best];
    ranks[best] += granule;
    left -= granule;
    double e = -1.0;
    if (ranks[best] < r_max) {
      e = 0.0;
      for (int i = ranks[best]; i < ranks[best] + granule; ++i)
        e += eig[(long)best * ld + i] > 0.0 ? eig[(long)best * ld + i] : 0.0;
    }
    next[best] = e;
  }
  free(next);
  if (kept) *kept = total;
  return 0;
}
