// Host-side launchers of the libxkv HIP kernels.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xkv {

// Device pointers passed by value in the kernel arguments (2 KiB).
constexpr int kMaxPtrs = 256;
struct PtrTable {
  const void* p[kMaxPtrs];
};

// ---- Gram: C = X^T X of the horizontally concatenated layers ---------------
// layers.p[s*G + l] is layer l of side s (T x d_kv, row stride ld).  C (and the
// optional float copy C32) are n x n per side with side stride n*n.
hipError_t launch_gram_bf16(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                            double* C, float* C32, hipStream_t st);
hipError_t launch_gram_f32(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                           double* C, float* C32, hipStream_t st);

// ---- Batched GEMM on MFMA: C = alpha op(A) op(B) + beta C ------------------
enum GType { GF32 = 0, GF64 = 1 };
struct GemmDesc {
  int M, N, K;
  int ta, tb;                 // 0: as stored, 1: transposed
  int typeA, typeB, typeC;    // GType of each operand in memory
  int acc;                    // GType of the MFMA arithmetic
  const void* A; long lda, sA;
  const void* B; long ldb, sB;
  void* C; long ldc, sC;
  double alpha, beta;
  int batch;
  int sym;                    // C symmetric (M == N, e.g. A^T A): only tiles on or above the
                              // diagonal are computed, each written at its mirror too
  int ksplit;                 // > 1: K in that many ranges, their products written to `part`
  double* part;               // (ksplit x batch x M x N doubles) and summed into C (double, ldc = N)
};
hipError_t gemm(const GemmDesc& d, hipStream_t st);

// ---- Cholesky helpers -----------------------------------------------------
// Factor the nb x nb diagonal block at (j0, j0) of each side's W (lower), write
// it into L and its inverse into Dinv (64 x 64 per side).  wdiag holds the
// diagonal of W before factorisation (n_sides x kb, side stride sDiag); a pivot
// below 1e-14 of it sets info[side] = 1, or with `clamp` is raised to that floor.
hipError_t launch_potrf_diag(const double* W, long ldw, long sW, double* L, long ldl, long sL,
                             double* Dinv, long sD, int j0, int nb, const double* wdiag, long sDiag,
                             int clamp, int n_sides, int* info, hipStream_t st);
hipError_t launch_copy_diag(const double* W, long ldw, long sW, double* dg, long sD, int n, int n_sides,
                            hipStream_t st);
hipError_t launch_zero_i32(int* p, long n, hipStream_t st);
// dst[i] = src[i] as float64, i < n.
hipError_t launch_widen(const float* src, double* dst, long n, hipStream_t st);
// tr[s] = trace of the n x n float64 matrix C + s*sC, for s < n_sides.
hipError_t launch_trace(const double* C, long sC, int n, int n_sides, double* tr, hipStream_t st);
// Z (n x r float64 per side, side stride zs) <- the logged QR rotations of a side's Rayleigh-Ritz
// eigensolve applied last first to the unit vectors at pos (r per side): runs (lo, hi, ktop, 0)
// of at most ritz_grouping().run_cap rotations, (c, s) pairs, groups (first run, count) of runs
// applied together as the host eigensolver forms them with ritz_grouping()'s limits, and per
// side meta = (first run, first pair, first group, groups).  scr: working memory of
// ritz_scratch_doubles(n, r) doubles per side (side stride scr_s).
struct RitzGrouping {
  int run_cap, per_group, spread, max_steps;
  int overhead;   // a group's fixed cost in fronts, for cutting a log into pieces of equal work
};
hipError_t launch_ritz_rotate(const int4* runs, const double2* cs, const int2* groups, const long long* meta,
                              const int* pos, int n, int r, double* Z, long zs, double* scr, long scr_s, int n_sides,
                              hipStream_t st);
RitzGrouping ritz_grouping();
// Pieces (1, 2 or 4) of a side's rotation log that the vector phase applies side by side.
int ritz_parts(int kb);
long ritz_scratch_doubles(int n, int r);
// res2[s*r + i] = || YZ[:, i] - theta[s*r + i] * Vr[:, i] ||^2 (n x r float64 per side, side stride n*r).
hipError_t launch_ritz_residual(const double* YZ, const double* Vr, const double* theta, int n, int r,
                                double* res2, int n_sides, hipStream_t st);

// ---- Subspace iteration helpers ------------------------------------------
hipError_t launch_init_q(float* Q, int rows, int k, long sQ, int n_sides, uint64_t seed, hipStream_t st);
// Vr (n x r float64 per side) -> Bt outputs (n x r, storage dtype, one pointer per side) and the
// transposed copy VrT (r x n, storage dtype, side stride sVT) used by the projection.
hipError_t launch_vr_outputs(const double* Vr, long sVr, int n, int r, const PtrTable& Bt, int bf16,
                             void* VrT, long sVT, int n_sides, hipStream_t st);

// ---- Projection A = X V_r and landmarks -----------------------------------
hipError_t launch_project_bf16(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                               const uint16_t* VrT, long sVT, int r, const PtrTable& A_out,
                               hipStream_t st);
hipError_t launch_project_f32(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                              const float* VrT, long sVT, int r, const PtrTable& A_out,
                              hipStream_t st);
// lm_out.p[s*G + l] receives n_kv_heads x (T/chunk) x head_dim for layer l of side s; row 0
// of the layers sits at position pos0.
hipError_t launch_landmarks(const PtrTable& layers, int n_sides, int G, long ld, int T, int n_kv_heads,
                            int head_dim, int chunk, double theta, const PtrTable& lm_out, int bf16,
                            hipStream_t st, long pos0 = 0);
// VrT (r x n, row stride n) = Bt^T for an n x r basis Bt with row stride ldb.
hipError_t launch_transpose_basis(const void* Bt, long ldb, int n, int r, void* VrT, int bf16, hipStream_t st);

// ---- Selective Reconstruction decode --------------------------------------
struct SrParams;  // defined in decode.hip
hipError_t launch_topk(const float* scores, int rows, int n_cand, long ld, int k, int* sel, hipStream_t st);

// Decode scratch owned by the library (decode.hip), for callers that cannot allocate:
// kSrScratchBytes of device memory per GPU, held until the process ends.
// sr_scratch_setup(device) looks up its address on `device` (which must be current)
// once; sr_scratch_ptr(device) returns it afterwards (NULL before).
constexpr size_t kSrScratchBytes = size_t(64) << 20;
constexpr int kSrScratchDevices = 64;
hipError_t sr_scratch_setup(int device);
void* sr_scratch_ptr(int device);

}  // namespace xkv
