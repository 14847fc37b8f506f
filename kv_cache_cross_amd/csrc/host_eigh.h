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
 * -1 on allocation failure, -2 if the QR iteration did not converge, -3 on bad sizes, -4 if H
 * has an entry that is not finite. */
int xkv_eigh_desc_scratch(int n, const double* H, int nvec, double* w, double* Z, xkv_eigh_scratch* sc);
/* The same in two phases.  xkv_eigh_values: all eigenvalues into w, the state for the vectors
 * kept in sc (same return codes).  xkv_eigh_vectors: columns [j0, j1) of Z (n x nvec,
 * row-major) from that state, with the working memory of `work` (which may be `state`);
 * calls on disjoint column ranges with distinct `work` may run in parallel threads.
 * Returns 0, or -1 on allocation failure. */
int xkv_eigh_values(int n, const double* H, int nvec, double* w, xkv_eigh_scratch* sc);
/* Where two threads of a paired value phase meet (zero-fill before the call; plain ints, used
 * through atomics). */
typedef struct {
  int count, gen;        /* the barrier */
  int fail;              /* either thread lacks memory */
  int job, k, split;     /* the worker's next row pass */
} xkv_eigh_pair;
/* xkv_eigh_values with the reduction's row passes shared by two threads: both call it at once
 * with the same arguments and pr, tid 0 (the leader, whose result and state are those of
 * xkv_eigh_values) and tid 1 (the worker, whose only memory is helper->buf; it returns 0, or
 * -1/-3 as the leader does).  The eigenvalues agree with xkv_eigh_values to rounding (the
 * product terms are summed in another order).  The two must run concurrently: each waits for
 * the other.  With refl set, the worker also writes xkv_eigh_pack_reflectors' output there
 * while the leader runs the QR iteration. */
int xkv_eigh_values_pair(int n, const double* H, int nvec, double* w, xkv_eigh_scratch* sc,
                         xkv_eigh_scratch* helper, xkv_eigh_pair* pr, int tid, double* refl);
int xkv_eigh_vectors(const xkv_eigh_scratch* state, int j0, int j1, double* Z, xkv_eigh_scratch* work);
void xkv_eigh_scratch_release(xkv_eigh_scratch* sc);

/* The vector phase on a device instead (one lane per wanted column: the unit vector at pos[j],
 * the logged rotations last first one run at a time, then the reflector blocks last first),
 * from the state of xkv_eigh_values:
 *   xkv_eigh_runs       the number of runs in the rotation log (QR sweeps, cut into pieces of
 *                       at most maxlen rotations);
 *   xkv_eigh_pack_log   runs as 4 ints (t_lo, t_hi, k_top, 0; rotation t acts on rows
 *                       k_top - (t_hi - t) and the one below) and (c, s) of every rotation;
 *   xkv_eigh_pack_reflectors  the reflectors as blocks of XKV_EIGH_NBG: every block's Y
 *                       (n - NBG b - 1 rows of NBG), then every block's T (NBG x NBG),
 *                       xkv_eigh_refl_doubles(n) doubles in all;
 *   xkv_eigh_positions  the nvec wanted positions, largest eigenvalue first. */
enum { XKV_EIGH_NBG = 64 };
int xkv_eigh_runs(const xkv_eigh_scratch* st, int maxlen);
void xkv_eigh_pack_log(const xkv_eigh_scratch* st, int maxlen, int* runs, double* cs);
/* Groups of up to B consecutive runs (in the order they are applied) whose starts and ends
 * lie within `spread` rows of one another and that span at most maxsteps rows, as (first run,
 * count) pairs, at most nruns of them; returns their number. */
int xkv_eigh_group_runs(const int* runs, int nruns, int B, int spread, int maxsteps, int* groups);
/* Pieces of a side's groups for a device that applies them in parallel (piece 0 to the wanted
 * unit vectors, each later piece to the identity, the results then multiplied together):
 * bounds[0..parts] are the pieces' first groups (bounds[parts] = ngroups), cut where the fronts
 * swept (plus `overhead` per group) reach equal shares. */
void xkv_eigh_split_groups(const int* runs, const int* groups, int ngroups, int overhead, int parts, int* bounds);
size_t xkv_eigh_refl_doubles(int n);
void xkv_eigh_pack_reflectors(const xkv_eigh_scratch* st, double* out);
void xkv_eigh_positions(const xkv_eigh_scratch* st, int* pos);
/* The same with memory of its own, freed on return. */
int xkv_eigh_desc_impl(int n, const double* H, int nvec, double* w, double* Z);

#ifdef __cplusplus
}
#endif
