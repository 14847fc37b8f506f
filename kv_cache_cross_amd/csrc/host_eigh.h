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

/* Memory of one eigensolve, kept between calls (it only grows): the state of the value phase
 * (the reduction's reflectors, the rotation log, the eigenvalue order) in buf, the working
 * memory of the vector phase in vbuf.  Zero-fill before first use. */
typedef struct xkv_eigh_scratch {
  double* buf;
  size_t cap;
  double* vbuf;
  size_t vcap;
  xkv_rotlog log;
  int n, nvec;
} xkv_eigh_scratch;

/* All n eigenvalues of symmetric H (n x n, row-major), descending, into w; the eigenvectors
 * of the nvec largest as the columns of Z (n x nvec, row-major).  Returns 0 on success,
 * -1 on allocation failure, -2 if the QR iteration did not converge, -3 on bad sizes. */
int xkv_eigh_desc_scratch(int n, const double* H, int nvec, double* w, double* Z, xkv_eigh_scratch* sc);
/* The same in two phases.  xkv_eigh_values: all eigenvalues into w, the state for the vectors
 * kept in sc (same return codes).  xkv_eigh_vectors: columns [j0, j1) of Z (n x nvec,
 * row-major) from that state, with the working memory of `work` (which may be `state`);
 * calls on disjoint column ranges with distinct `work` may run in parallel threads.
 * Returns 0, or -1 on allocation failure. */
int xkv_eigh_values(int n, const double* H, int nvec, double* w, xkv_eigh_scratch* sc);
int xkv_eigh_vectors(const xkv_eigh_scratch* state, int j0, int j1, double* Z, xkv_eigh_scratch* work);
void xkv_eigh_scratch_release(xkv_eigh_scratch* sc);
/* The same with memory of its own, freed on return. */
int xkv_eigh_desc_impl(int n, const double* H, int nvec, double* w, double* Z);

#ifdef __cplusplus
}
#endif
