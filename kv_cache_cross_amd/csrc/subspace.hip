// Kernels of the block subspace iteration besides the GEMMs:
//   * factor of a diagonal block of W = Y^T Y for the blocked Cholesky of
//     CholeskyQR (Q = Y R^-1 with W = R^T R), with the block's inverse;
//   * the Gaussian start block;
//   * conversion of V_r to the stored Bt = V_r and its transpose.
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int NB = 64;

// One workgroup per side: load the nb x nb diagonal block of W at (j0, j0), factor it
// as L L^T in LDS (right-looking, column by column) and invert L alongside: X = L^-1
// solves L X = I by the same right-looking sweep (at column k, row k of the right-hand
// side is divided by the pivot and row k's multiples L[i][k] X[k][.] leave the rows
// below), so both share the column loop's barriers.  Writes L and L^-1.
__global__ __launch_bounds__(256) void potrf_diag_kernel(const double* W, long ldw, long sW,
                                                         double* L, long ldl, long sL,
                                                         double* Dinv, long sD, int j0, int nb,
                                                         const double* wdiag, long sDiag, int clamp,
                                                         int* info) {
  __shared__ double a[NB][NB + 1];
  __shared__ double inv[NB][NB + 1];
  __shared__ double floor_s[NB];   // the pivots' breakdown floors
  __shared__ int bad;
  const int side = blockIdx.x, tid = threadIdx.x;
  const int ti = tid >> 4, tj = tid & 15;   // a 16 x 16 thread grid
  const double* w = W + side * sW + (long)j0 * ldw + j0;
  if (tid == 0) bad = 0;
  if (tid < nb) floor_s[tid] = 1e-14 * wdiag[side * sDiag + j0 + tid];
  for (int i = ti; i < NB; i += 16)
    for (int j = tj; j < NB; j += 16) {
      a[i][j] = (i < nb && j < nb && j <= i) ? w[(long)i * ldw + j] : 0.0;
      inv[i][j] = (i == j) ? 1.0 : 0.0;
    }
  __syncthreads();
  for (int k = 0; k < nb; ++k) {
    if (tid == 0) {
      // The pivot is the squared distance of column j0+k of Y from the span of the
      // previous columns.  Below 1e-14 of the column's squared norm it is either a
      // breakdown (float64 sweeps: reported) or, with `clamp` (float32 sweeps, whose Y
      // carries float32 noise), raised to that floor, which damps the near-dependent
      // direction instead of amplifying noise.
      double piv = a[k][k];
      const double floor_k = floor_s[k];
      if (!isfinite(piv)) {
        bad = 1;
        piv = 1.0;
      } else if (!(piv > floor_k)) {
        if (clamp && floor_k > 0.0) {
          piv = floor_k;
        } else {
          bad = 1;
          piv = 1.0;
        }
      }
      a[k][k] = sqrt(piv);
    }
    __syncthreads();
    const double rdk = 1.0 / a[k][k];
    // column k of L below the pivot, and row k of X (columns c <= k)
    if (tid < 64) {
      for (int i = k + 1 + tid; i < nb; i += 64) a[i][k] *= rdk;
    } else if (tid - 64 <= k) {
      inv[k][tid - 64] *= rdk;
    }
    __syncthreads();
    // trailing update of the lower triangle (k < j <= i), and the rows of X below k
    for (int i = k + 1 + ti; i < nb; i += 16) {
      const double aik = a[i][k];
      for (int j = k + 1 + tj; j <= i; j += 16) a[i][j] -= aik * a[j][k];
      for (int c = tj; c <= k; c += 16) inv[i][c] -= aik * inv[k][c];
    }
    __syncthreads();
  }
  double* l = L + side * sL + (long)j0 * ldl + j0;
  double* dv = Dinv + side * sD;
  for (int i = ti; i < nb; i += 16)
    for (int j = tj; j < nb; j += 16) l[(long)i * ldl + j] = (j <= i) ? a[i][j] : 0.0;
  for (int i = ti; i < NB; i += 16)
    for (int j = tj; j < NB; j += 16) dv[i * NB + j] = (i < nb && j < nb && j <= i) ? inv[i][j] : 0.0;
  if (tid == 0 && bad) info[side] = 1;
}

__global__ void copy_diag_kernel(const double* W, long ldw, long sW, double* dg, long sD, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dg[blockIdx.y * sD + i] = W[blockIdx.y * sW + (long)i * ldw + i];
}

// Squared residual norm of each Ritz pair: one thread per (row group, column).
__global__ __launch_bounds__(256) void ritz_residual_kernel(const double* YZ, const double* Vr,
                                                            const double* theta, int n, int r, double* res2) {
  __shared__ double part[4][64];
  const int side = blockIdx.y;
  const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + c;
  const long off = (long)side * n * r;
  double s = 0.0;
  if (i < r) {
    const double th = theta[(long)side * r + i];
    for (int j = rg; j < n; j += 4) {
      const double e = YZ[off + (long)j * r + i] - th * Vr[off + (long)j * r + i];
      s += e * e;
    }
  }
  part[rg][c] = s;
  __syncthreads();
  if (rg == 0 && i < r) res2[(long)side * r + i] = part[0][c] + part[1][c] + part[2][c] + part[3][c];
}

__global__ void widen_kernel(const float* src, double* dst, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = (double)src[i];
}

__global__ void zero_i32_kernel(int* p, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// tr[s] = sum_i C_s[i][i] (float64), one block per side: the total energy ||X||_F^2 of
// the side, i.e. the sum of all eigenvalues of C.
__global__ __launch_bounds__(256) void trace_kernel(const double* C, long sC, int n, double* tr) {
  __shared__ double part[256];
  const int s = blockIdx.x, tid = threadIdx.x;
  const double* Cs = C + (long)s * sC;
  double acc = 0.0;
  for (int i = tid; i < n; i += 256) acc += Cs[(long)i * n + i];
  part[tid] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) tr[s] = part[0];
}

// splitmix64 finaliser: a counter-based source of uniform bits.
XKV_DEV uint64_t mix64(uint64_t z) {
  z += 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// Gaussian start block (Box-Muller on two 53-bit uniforms per entry).
__global__ void init_q_kernel(float* Q, int rows, int k, long sQ, uint64_t seed) {
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int side = blockIdx.y;
  if (e >= (long)rows * k) return;
  // The same start block for every side, so a side's result does not depend on its batch slot.
  const uint64_t base = mix64(seed ^ 0x51deull) + 2ull * (uint64_t)e;
  const double u1 = ((mix64(base) >> 11) + 1.0) * (1.0 / 9007199254740993.0);
  const double u2 = (mix64(base + 1) >> 11) * (1.0 / 9007199254740992.0);
  Q[side * sQ + e] = (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

struct VrArgs {
  PtrTable Bt;
  const double* Vr;
  long sVr;
  int n, r, bf16;
  void* VrT;
  long sVT;
};

// Bt (n x r) <- Vr and VrT (r x n) <- Vr^T, via a 32 x 32 LDS transpose.
__global__ __launch_bounds__(256) void vr_outputs_kernel(VrArgs a) {
  __shared__ double tile[32][33];
  const int side = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;   // i: row of Vr (0..n), j: rank index
  const double* V = a.Vr + side * a.sVr;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    const int i = i0 + yy, j = j0 + tx;
    double v = (i < a.n && j < a.r) ? V[(long)i * a.r + j] : 0.0;
    tile[yy][tx] = v;
    if (i < a.n && j < a.r) {
      if (a.bf16) ((uint16_t*)a.Bt.p[side])[(long)i * a.r + j] = f32_to_bf16_bits((float)v);
      else ((float*)a.Bt.p[side])[(long)i * a.r + j] = (float)v;
    }
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int j = j0 + yy, i = i0 + tx;
    if (i < a.n && j < a.r) {
      const double v = tile[tx][yy];
      if (a.bf16) ((uint16_t*)a.VrT)[side * a.sVT + (long)j * a.n + i] = f32_to_bf16_bits((float)v);
      else ((float*)a.VrT)[side * a.sVT + (long)j * a.n + i] = (float)v;
    }
  }
}

}  // namespace

hipError_t launch_potrf_diag(const double* W, long ldw, long sW, double* L, long ldl, long sL,
                             double* Dinv, long sD, int j0, int nb, const double* wdiag, long sDiag,
                             int clamp, int n_sides, int* info, hipStream_t st) {
  if (nb > NB) return hipErrorInvalidValue;
  hipLaunchKernelGGL(potrf_diag_kernel, dim3(n_sides), dim3(256), 0, st, W, ldw, sW, L, ldl, sL, Dinv,
                     sD, j0, nb, wdiag, sDiag, clamp, info);
  return hipGetLastError();
}

hipError_t launch_copy_diag(const double* W, long ldw, long sW, double* dg, long sD, int n, int n_sides,
                            hipStream_t st) {
  hipLaunchKernelGGL(copy_diag_kernel, dim3((n + 255) / 256, n_sides), dim3(256), 0, st, W, ldw, sW, dg, sD, n);
  return hipGetLastError();
}

hipError_t launch_ritz_residual(const double* YZ, const double* Vr, const double* theta, int n, int r,
                                double* res2, int n_sides, hipStream_t st) {
  hipLaunchKernelGGL(ritz_residual_kernel, dim3((r + 63) / 64, n_sides), dim3(256), 0, st, YZ, Vr, theta, n, r, res2);
  return hipGetLastError();
}

hipError_t launch_trace(const double* C, long sC, int n, int n_sides, double* tr, hipStream_t st) {
  hipLaunchKernelGGL(trace_kernel, dim3(n_sides), dim3(256), 0, st, C, sC, n, tr);
  return hipGetLastError();
}

hipError_t launch_widen(const float* src, double* dst, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(widen_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int* p, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_init_q(float* Q, int rows, int k, long sQ, int n_sides, uint64_t seed, hipStream_t st) {
  const long total = (long)rows * k;
  hipLaunchKernelGGL(init_q_kernel, dim3((unsigned)((total + 255) / 256), n_sides), dim3(256), 0, st, Q,
                     rows, k, sQ, seed);
  return hipGetLastError();
}

hipError_t launch_vr_outputs(const double* Vr, long sVr, int n, int r, const PtrTable& Bt, int bf16,
                             void* VrT, long sVT, int n_sides, hipStream_t st) {
  VrArgs a;
  a.Bt = Bt;
  a.Vr = Vr;
  a.sVr = sVr;
  a.n = n;
  a.r = r;
  a.bf16 = bf16;
  a.VrT = VrT;
  a.sVT = sVT;
  hipLaunchKernelGGL(vr_outputs_kernel, dim3((r + 31) / 32, (n + 31) / 32, n_sides), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace xkv
