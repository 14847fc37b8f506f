// Batched GEMM on the float32 / float64 matrix cores for the subspace
// iteration: C = alpha op(A) op(B) + beta C.
//
// 64 x 64 output tile per workgroup, K staged through LDS in steps of 16;
// 4 waves in a 2 x 2 grid, each owning 2 x 2 tiles of v_mfma_f32_16x16x4f32
// or v_mfma_f64_16x16x4f64.  Operands are converted to the arithmetic type
// while they are staged, so float32 data can feed float64 arithmetic
// (W = Y^T Y of a float32 block is summed in float64).
//
// Lane layouts (checked on gfx950): both instructions take A[m = lane%16]
// [k = lane/16] and B[k = lane/16][n = lane%16].  The float32 result holds
// D[4*(lane/16) + v][lane%16] in register v; the float64 result holds
// D[4*v + lane/16][lane%16].
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <typename T>
struct Mfma;
template <>
struct Mfma<float> {
  typedef f32x4_t acc_t;
  static XKV_DEV acc_t op(float a, float b, acc_t c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
  static XKV_DEV int row(int lane, int v) { return 4 * (lane >> 4) + v; }
};
template <>
struct Mfma<double> {
  typedef f64x4_t acc_t;
  static XKV_DEV acc_t op(double a, double b, acc_t c) { return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0); }
  static XKV_DEV int row(int lane, int v) { return 4 * v + (lane >> 4); }
};

struct Args {
  int M, N, K;
  const void* A; long lda, sA;
  const void* B; long ldb, sB;
  void* C; long ldc, sC;
  double alpha, beta;
};

template <typename TA, typename TB, typename TC, typename ACC, bool TA_T, bool TB_T>
__global__ __launch_bounds__(256) void gemm_kernel(Args p) {
  __shared__ ACC As[BK][BM + 4];
  __shared__ ACC Bs[BK][BN + 4];
  const int z = blockIdx.z;
  const TA* A = (const TA*)p.A + z * p.sA;
  const TB* B = (const TB*)p.B + z * p.sB;
  TC* C = (TC*)p.C + z * p.sC;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  typename Mfma<ACC>::acc_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0;

  for (int k0 = 0; k0 < p.K; k0 += BK) {
    // Stage op(A)[m0:m0+64, k0:k0+16] as As[k][m] and op(B)[k0:k0+16, n0:n0+64] as Bs[k][n].
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int mm, kk;
      if (TA_T) { kk = tid >> 4; mm = (tid & 15) * 4 + q; }   // A stored K x M: contiguous in m
      else      { mm = tid >> 2; kk = (tid & 3) * 4 + q; }    // A stored M x K: contiguous in k
      const int gm = m0 + mm, gk = k0 + kk;
      ACC v = 0;
      if (gm < p.M && gk < p.K) v = (ACC)(TA_T ? A[(long)gk * p.lda + gm] : A[(long)gm * p.lda + gk]);
      As[kk][mm] = v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int nn, kk;
      if (TB_T) { nn = tid >> 2; kk = (tid & 3) * 4 + q; }    // B stored N x K: contiguous in k
      else      { kk = tid >> 4; nn = (tid & 15) * 4 + q; }   // B stored K x N: contiguous in n
      const int gn = n0 + nn, gk = k0 + kk;
      ACC v = 0;
      if (gn < p.N && gk < p.K) v = (ACC)(TB_T ? B[(long)gn * p.ldb + gk] : B[(long)gk * p.ldb + gn]);
      Bs[kk][nn] = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 4) {
      ACC a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[ks + (lane >> 4)][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[ks + (lane >> 4)][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = Mfma<ACC>::op(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gm = m0 + wm * 32 + i * 16 + Mfma<ACC>::row(lane, v);
        const int gn = n0 + wn * 32 + j * 16 + (lane & 15);
        if (gm < p.M && gn < p.N) {
          TC* dst = C + (long)gm * p.ldc + gn;
          double r = p.alpha * (double)acc[i][j][v];
          if (p.beta != 0.0) r += p.beta * (double)*dst;
          *dst = (TC)r;
        }
      }
}

template <typename TA, typename TB, typename TC, typename ACC>
hipError_t run(const GemmDesc& d, hipStream_t st) {
  Args p{d.M, d.N, d.K, d.A, d.lda, d.sA, d.B, d.ldb, d.sB, d.C, d.ldc, d.sC, d.alpha, d.beta};
  dim3 grid((d.N + BN - 1) / BN, (d.M + BM - 1) / BM, d.batch);
  if (d.ta && d.tb) hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, true, true>), grid, dim3(256), 0, st, p);
  else if (d.ta)    hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, true, false>), grid, dim3(256), 0, st, p);
  else if (d.tb)    hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, false, true>), grid, dim3(256), 0, st, p);
  else              hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, false, false>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm(const GemmDesc& d, hipStream_t st) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  const int code = (d.typeA << 3) | (d.typeB << 2) | (d.typeC << 1) | d.acc;
  switch (code) {
    // A B C acc  (0 = float, 1 = double)
    case 0b0000: return run<float, float, float, float>(d, st);
    case 0b0011: return run<float, float, double, double>(d, st);
    case 0b0101: return run<float, double, float, double>(d, st);
    case 0b0111: return run<float, double, double, double>(d, st);
    case 0b1001: return run<double, float, float, double>(d, st);
    case 0b1011: return run<double, float, double, double>(d, st);
    case 0b1101: return run<double, double, float, double>(d, st);
    case 0b1111: return run<double, double, double, double>(d, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xkv
