// Kernels of the block subspace iteration besides the GEMMs:
//   * factor of a diagonal block of W = Y^T Y for the blocked Cholesky of
//     CholeskyQR (Q = Y R^-1 with W = R^T R), with the block's inverse;
//   * the Gaussian start block;
//   * conversion of V_r to the stored Bt = V_r and its transpose;
//   * the plane rotations of the Rayleigh-Ritz eigensolve's QR iteration applied to the
//     wanted unit vectors, or a piece of them to the identity (the first part of its vector
//     phase; the pieces' products and the reflectors follow as GEMMs).
#include <climits>
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int NB = 64;

// One workgroup per side: load the nb x nb diagonal block of W at (j0, j0) and factor it as
// L L^T with L^-1 alongside.  The elimination runs as L~ D L~^T (L~ unit lower): step k takes
// the pivot d_k = a[k][k] and subtracts a[i][k] a[j][k] / d_k from the trailing lower triangle,
// leaving column k unscaled (a[i][k] = l~_ik d_k), and X = L~^-1 comes from the same sweep (row
// i of X loses l~_ik times row k).  The block lives in registers: a 16 x 16 thread grid, thread
// (ti, tj) holding rows ti + 16 a and columns tj + 16 b (a, b < 4) of both a and X.  At step k
// the threads holding column k of a and row k of X put them in LDS (two buffers used in turn,
// so one barrier per step), and every thread updates its 4 x 4 pieces from them, taking the
// pivot decision itself.  At the end L = a D^-1/2 below the diagonal with sqrt(d) on it, and
// L^-1 = D^-1/2 X.
__global__ __launch_bounds__(256) void potrf_diag_kernel(const double* W, long ldw, long sW,
                                                         double* L, long ldl, long sL,
                                                         double* Dinv, long sD, int j0, int nb,
                                                         const double* wdiag, long sDiag, int clamp,
                                                         int* info) {
  __shared__ double colb[2][NB];   // column k of a
  __shared__ double rowb[2][NB];   // row k of X
  __shared__ double floor_s[NB];   // the pivots' breakdown floors
  __shared__ double piv_s[NB];     // the pivots taken
  __shared__ double rs_s[NB], sq_s[NB];
  __shared__ int bad;
  const int side = blockIdx.x, tid = threadIdx.x;
  const int ti = tid >> 4, tj = tid & 15;   // a 16 x 16 thread grid
  const double* w = W + side * sW + (long)j0 * ldw + j0;
  if (tid == 0) bad = 0;
  if (tid < nb) floor_s[tid] = 1e-14 * wdiag[side * sDiag + j0 + tid];
  double A[4][4], X[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = ti + 16 * a, j = tj + 16 * b;
      A[a][b] = (i < nb && j < nb && j <= i) ? w[(long)i * ldw + j] : 0.0;
      X[a][b] = i == j ? 1.0 : 0.0;
    }
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int k = 16 * kb + kk, par = kk & 1;
      if (k < nb) {
        if (tj == kk) {
#pragma unroll
          for (int a = 0; a < 4; ++a) colb[par][ti + 16 * a] = A[a][kb];
        }
        if (ti == kk) {
#pragma unroll
          for (int b = 0; b < 4; ++b) rowb[par][tj + 16 * b] = X[kb][b];
        }
        __syncthreads();
        // The pivot is the squared distance of column j0+k of Y from the span of the previous
        // columns.  Below 1e-14 of the column's squared norm it is either a breakdown (float64
        // sweeps: reported) or, with `clamp` (float32 sweeps, whose Y carries float32 noise),
        // raised to that floor, which damps the near-dependent direction instead of
        // amplifying noise.
        double piv = colb[par][k];
        const double floor_k = floor_s[k];
        bool brk = false;
        if (!isfinite(piv)) {
          brk = true;
          piv = 1.0;
        } else if (!(piv > floor_k)) {
          if (clamp && floor_k > 0.0) {
            piv = floor_k;
          } else {
            brk = true;
            piv = 1.0;
          }
        }
        if (tid == 0) {
          piv_s[k] = piv;
          if (brk) bad = 1;
        }
        const double rdk = 1.0 / piv;
        double cj[4], xr[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          cj[b] = colb[par][tj + 16 * b];
          xr[b] = rowb[par][tj + 16 * b];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int i = ti + 16 * a;
          const double lik = i > k ? colb[par][i] * rdk : 0.0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int j = tj + 16 * b;
            if (j > k && j <= i) A[a][b] -= lik * cj[b];
            X[a][b] -= lik * xr[b];   // row k of X is zero past column k
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid < nb) {
    const double sq = sqrt(piv_s[tid]);
    sq_s[tid] = sq;
    rs_s[tid] = 1.0 / sq;
  }
  __syncthreads();
  double* l = L + side * sL + (long)j0 * ldl + j0;
  double* dv = Dinv + side * sD;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = ti + 16 * a, j = tj + 16 * b;
      if (i < nb && j < nb) l[(long)i * ldl + j] = j < i ? A[a][b] * rs_s[j] : (j == i ? sq_s[j] : 0.0);
      dv[i * NB + j] = (i < nb && j < nb && j <= i) ? X[a][b] * rs_s[i] : 0.0;
    }
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


// One lane per wanted column j of one side (64 columns per workgroup): column j starts as the
// unit vector at pos[j]; the logged rotations are then applied last first, a run at a time.
// A run is rotations lo..hi of the log, rotation t acting on rows k = ktop - (hi - t) and
// k + 1 as [c -s; s c] (new row k+1 = s x + c y, new row k = c x - s y for x, y the old rows
// k, k+1).  Taken last first a run climbs the rows: the row the next rotation shares is
// carried in a register, and row k + 1 is final for the run once rotation k is applied.
//
// Runs go in groups of up to kB, applied together as a wavefront: at each step a front row f
// is loaded, run b applies its rotation at row f + b (it lags run b - 1 by one row, so both of
// its rows already hold every earlier run's result), passing its finished row f + b + 1 to
// run b + 1, and the last run's finished row f + kB is stored: one load and one store for kB
// rotations.  Outside its rows a run applies the identity (c = 1, s = 0), which passes the
// rows through; the fronts span the union of the group's runs.  Rows above and below the
// fronts' reach are zero padding (the identity multiplies them by zero, so they must be
// finite).
//
// The columns live in a scratch copy laid out per workgroup as rows of its 64 lanes (512
// bytes a row) on a buffer resource: a chunk's rows are a scalar base plus immediate offsets.
// A group's (c, s) pairs are staged in LDS, one slot per run in the order they are applied,
// identities around them.  The fronts go in chunks of CH, the next chunk's rows loaded while
// the current one is applied; a chunk's rows are not written before they are read (stores
// trail the loads by kB + 1 rows).  At the end the scratch rows are copied to Z (n x r).
// Lanes past r work on column r - 1 exactly as its own lane does and store nothing to Z.
constexpr int kRunCap = 1024;                 // rotations per run (longer sweeps are cut)
constexpr int kB = 4;                         // runs per group (even: slots are staged in pairs)
static_assert(kB % 2 == 0, "pair slots are staged two at a time");
constexpr int CH = 8;                         // fronts per chunk
constexpr int kSpread = 64;                   // rows a group's starts and ends may differ by
constexpr int kSlot = kSpread + kRunCap + kSpread + 2 * CH;   // LDS pairs per run
constexpr int kPadLo = 2 * CH + kB, kPadHi = kB;              // scratch rows before 0 and after n - 1
constexpr unsigned kRowB = 64 * 8;            // bytes per scratch row

using zrsrc = __amdgpu_buffer_rsrc_t;
typedef unsigned zbits __attribute__((__vector_size__(2 * sizeof(unsigned))));
__device__ __forceinline__ double zload(zrsrc z, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(z, voff, soff, 0));
}
__device__ __forceinline__ void zstore(zrsrc z, unsigned voff, unsigned soff, double v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(zbits, v), z, voff, soff, 0);
}
// byte offset of scratch row `row` (row >= -kPadLo)
__device__ __forceinline__ unsigned zrow(int row) { return (unsigned)(row + kPadLo) * kRowB; }

// Rows f - u, u < CH, from one base with immediate offsets.
__device__ __forceinline__ void front_load(double (&x)[CH], zrsrc z, unsigned loff, int f) {
  const unsigned b = zrow(f - (CH - 1));
#pragma unroll
  for (int u = 0; u < CH; ++u) x[u] = zload(z, loff + (CH - 1 - u) * kRowB, b);
}

// The first cnt fronts of a chunk (cnt uniform; CH for a whole chunk): front f - u feeds row
// f - u to run 0 and stores row f - u + kB.  gi[b] is run b's LDS index at front f.  The
// chunk's pairs are read up front, the second half's while the first half is applied.
template <bool WHOLE>
__device__ __forceinline__ void front_apply(const double (&x)[CH], zrsrc z, unsigned loff, int f, const int (&gi)[kB],
                                            const double2 (*cs_s)[kSlot], double (&y)[kB], int cnt) {
  const unsigned sb = zrow(f + kB - (CH - 1));
  double2 g[CH][kB];
#pragma unroll
  for (int u = 0; u < CH / 2; ++u)
#pragma unroll
    for (int b = 0; b < kB; ++b) g[u][b] = cs_s[b][gi[b] + u];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    if (u == 1) {
#pragma unroll
      for (int u2 = CH / 2; u2 < CH; ++u2)
#pragma unroll
        for (int b = 0; b < kB; ++b) g[u2][b] = cs_s[b][gi[b] + u2];
    }
    if (WHOLE || u < cnt) {
      double v = x[u];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const double cx = g[u][b].x * v;
        v = fma(g[u][b].y, v, g[u][b].x * y[b]);
        y[b] = fma(-g[u][b].y, y[b], cx);
      }
      zstore(z, loff + (CH - 1 - u) * kRowB, sb, v);
    }
  }
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void ritz_rotate_kernel(
    const int4* __restrict__ runs,
                                                         const double2* __restrict__ cs,
                                                         const int2* __restrict__ groups,
                                                         const long long* __restrict__ meta,
                                                         const int* __restrict__ pos, int n, int r,
                                                         double* __restrict__ Z, long zs,
                                                         double* __restrict__ scr, long scr_s) {
  __shared__ double2 cs_s[kB][kSlot];
  const int s = blockIdx.y, lane = threadIdx.x;
  const int j = (int)blockIdx.x * 64 + lane;
  const int jc = min(j, r - 1);
  const unsigned loff = 8u * (unsigned)lane;
  const int rows = kPadLo + n + kPadHi;
  const zrsrc z = __builtin_amdgcn_make_buffer_rsrc(scr + s * scr_s + (long)blockIdx.x * rows * 64, 0,
                                                    (int)((unsigned)rows * kRowB), 0x00020000);
  const int pj = pos[(long)s * r + jc];
  for (int i = -kPadLo; i < n + kPadHi; ++i) zstore(z, loff, zrow(i), i == pj ? 1.0 : 0.0);
  const long long run0 = meta[4 * s], cs0 = meta[4 * s + 1], grp0 = meta[4 * s + 2], ngrp = meta[4 * s + 3];
  for (long long gq = 0; gq < ngrp; ++gq) {
    const int2 G = groups[grp0 + gq];
    // the group's runs: b-th applied is run G.x - b of the side's log (read for every slot, so
    // that the four scalar loads are in flight together; slots past G.y are empty)
    int4 R[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) R[b] = runs[run0 + max(G.x - b, 0)];
    int kt[kB], len[kB];
    int f0 = INT_MIN, f1 = INT_MAX;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      len[b] = b < G.y ? R[b].y - R[b].x + 1 : 0;
      if (b < G.y) {
        f0 = max(f0, R[b].z - b);
        f1 = min(f1, R[b].z - len[b] + 1 - b);
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) kt[b] = b < G.y ? R[b].z : f0 + b;   // an empty slot: identities
    __syncthreads();   // the previous group's pairs are read
    // A slot: identities, then the run's pairs in the order applied from index kSpread on (the
    // m-th rotation applied is the run's pair len - 1 - m), then identities; each lane issues
    // two slots' loads before their LDS stores.
    constexpr int PT = (kSlot + 63) / 64;
#pragma unroll
    for (int b = 0; b < kB; b += 2) {   // two slots' loads in flight together
      double2 t[2][PT];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const double2* src = cs + cs0 + R[b + h].x;
#pragma unroll
        for (int q = 0; q < PT; ++q) {
          const int m = lane + 64 * q - kSpread;
          t[h][q] = (m >= 0 && m < len[b + h]) ? src[len[b + h] - 1 - m] : make_double2(1.0, 0.0);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < PT; ++q)
          if (lane + 64 * q < kSlot) cs_s[b + h][lane + 64 * q] = t[h][q];
    }
    __syncthreads();
    double y[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) y[b] = zload(z, loff, zrow(f0 + b + 1));
    int gi[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) gi[b] = kSpread + kt[b] - b - f0;
    const int steps = f0 - f1 + 1, nf = steps / CH, rem = steps % CH;
    int f = f0;
    double xa[CH], xb[CH];
    front_load(xa, z, loff, f);
    int c = 0;
    for (; c + 1 < nf; c += 2) {
      front_load(xb, z, loff, f - CH);
      front_apply<true>(xa, z, loff, f, gi, cs_s, y, CH);
      f -= CH;
#pragma unroll
      for (int b = 0; b < kB; ++b) gi[b] += CH;
      front_load(xa, z, loff, f - CH);
      front_apply<true>(xb, z, loff, f, gi, cs_s, y, CH);
      f -= CH;
#pragma unroll
      for (int b = 0; b < kB; ++b) gi[b] += CH;
    }
    if (c < nf) {   // xa holds the last whole chunk
      front_load(xb, z, loff, f - CH);
      front_apply<true>(xa, z, loff, f, gi, cs_s, y, CH);
      f -= CH;
#pragma unroll
      for (int b = 0; b < kB; ++b) gi[b] += CH;
      if (rem) front_apply<false>(xb, z, loff, f, gi, cs_s, y, rem);
    } else if (rem) {   // xa holds the partial chunk
      front_apply<false>(xa, z, loff, f, gi, cs_s, y, rem);
    }
    // rows f1 .. f1 + kB - 1 are final in the carried registers
#pragma unroll
    for (int b = 0; b < kB; ++b) zstore(z, loff, zrow(f1 + b), y[b]);
  }
  if (j < r) {
    double* zc = Z + s * zs + j;
    for (int i = 0; i < n; ++i) zc[(long)i * r] = zload(z, loff, zrow(i));
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

hipError_t launch_ritz_rotate(const int4* runs, const double2* cs, const int2* groups, const long long* meta,
                              const int* pos, int n, int r, double* Z, long zs, double* scr, long scr_s, int n_sides,
                              hipStream_t st) {
  if (n_sides <= 0 || r <= 0) return hipSuccess;
  if (n <= 0 || (long)(kPadLo + n + kPadHi) * kRowB > 0x7fffffffL) return hipErrorInvalidValue;   // 31-bit range
  if (scr_s < ritz_scratch_doubles(n, r)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ritz_rotate_kernel, dim3((r + 63) / 64, n_sides), dim3(64), 0, st, runs, cs, groups, meta, pos, n,
                     r, Z, zs, scr, scr_s);
  return hipGetLastError();
}

// A group's pair staging, with its one exposed memory latency, costs about as much as this many
// fronts (the weight of a group when a log is cut into pieces of equal work).
constexpr int kGroupOverhead = 32;
RitzGrouping ritz_grouping() { return RitzGrouping{kRunCap, kB, kSpread, kRunCap + kSpread, kGroupOverhead}; }

// One workgroup applies a log to 64 columns with one wave whose instructions issue one after
// another, so a half's 8 sides of r = 512 columns keep 64 of the 256 compute units busy for the
// whole log.  The log is therefore cut into pieces applied side by side (the first to the wanted
// unit vectors, the others to the identity) and multiplied together afterwards: 4 pieces up to
// k_b = 1024 (8 sides of k_b = 768 give 384 single-wave workgroups, two per compute unit by their
// LDS), 2 above it; none below k_b = 256, where the log is short.  The count depends on k_b
// alone, so that a side's result does not depend on how many sides share its call.
int ritz_parts(int kb) { return kb < 256 ? 1 : (kb <= 1024 ? 4 : 2); }

long ritz_scratch_doubles(int n, int r) { return (long)((r + 63) / 64) * (kPadLo + n + kPadHi) * 64; }

}  // namespace xkv
