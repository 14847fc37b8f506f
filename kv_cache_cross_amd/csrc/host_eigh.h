/* Host symmetric eigensolver of the Rayleigh-Ritz step (host_eigh.c). */
#pragma once
#include <stddef.h>
#ifdef __cplusplus
extern "C" {
#endif

/* The plane rotations of the QR iteration, in the order they were taken. */
typedef struct {
  double* c;
  double* s;
  int* k;
  long n, cap;
} xkv_rotlog;

/* Memory of one eigensolve, kept between calls of one thread (it only grows): one block of
 * doubles carved per call, and the rotation log.  Zero-fill before first use. */
typedef struct xkv_eigh_scratch {
  double* buf;
  size_t cap;
  xkv_rotlog log;
} xkv_eigh_scratch;

/* All n eigenvalues of symmetric H (n x n, row-major), descending, into w; the eigenvectors
 * of the nvec largest as the columns of Z (n x nvec, row-major).  Returns 0 on success,
 * -1 on allocation failure, -2 if the QR iteration did not converge, -3 on bad sizes. */
int xkv_eigh_desc_scratch(int n, const double* H, int nvec, double* w, double* Z, xkv_eigh_scratch* sc);
void xkv_eigh_scratch_release(xkv_eigh_scratch* sc);
/* The same with memory of its own, freed on return. */
int xkv_eigh_desc_impl(int n, const double* H, int nvec, double* w, double* Z);

#ifdef __cplusplus
}
#endif
