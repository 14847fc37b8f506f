// Batched GEMM on the float32 / float64 matrix cores for the subspace
// iteration: C = alpha op(A) op(B) + beta C.
//
// 64 x 64 output tile per workgroup, K staged through LDS in slabs of 32 with the
// next slab's loads in flight (in registers) while the current one is multiplied;
// 4 waves in a 2 x 2 grid, each owning 2 x 2 tiles of v_mfma_f32_16x16x4f32 or
// v_mfma_f64_16x16x4f64.  Operands are converted to the arithmetic type while they
// are staged, so float32 data can feed float64 arithmetic (W = Y^T Y of a float32
// block is summed in float64).  Each thread loads 8 elements of each operand per
// slab, consecutive threads along the operand's contiguous dimension.
//
// Lane layouts (checked on gfx950): both instructions take A[m = lane%16]
// [k = lane/16] and B[k = lane/16][n = lane%16].  The float32 result holds
// D[4*(lane/16) + v][lane%16] in register v; the float64 result holds
// D[4*v + lane/16][lane%16].
#include <algorithm>
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int BM = 64, BN = 64, BK = 32;

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
  int sym;
  int batch, ksplit, kchunk;   // ksplit > 1: workgroup z takes K range z / batch of side z % batch
  double* part;                // and writes its partial product there (M x N each)
};

template <typename TA, typename TB, typename TC, typename ACC, bool TA_T, bool TB_T>
__global__ __launch_bounds__(256) void gemm_kernel(Args p) {
  __shared__ ACC As[BK][BM + 4];
  __shared__ ACC Bs[BK][BN + 4];
  const int z = blockIdx.z;
  const TA* A;
  const TB* B;
  TC* C;
  int K = p.K;
  long ldc = p.ldc;
  if (p.ksplit > 1) {
    const int side = z % p.batch, kc0 = (z / p.batch) * p.kchunk;
    K = min(p.kchunk, p.K - kc0);
    A = (const TA*)p.A + side * p.sA + (TA_T ? (long)kc0 * p.lda : (long)kc0);
    B = (const TB*)p.B + side * p.sB + (TB_T ? (long)kc0 : (long)kc0 * p.ldb);
    C = (TC*)(p.part + (long)z * p.M * p.N);
    ldc = p.N;
  } else {
    A = (const TA*)p.A + z * p.sA;
    B = (const TB*)p.B + z * p.sB;
    C = (TC*)p.C + z * p.sC;
  }
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  if (p.sym && n0 < m0) return;   // a tile below the diagonal: its mirror writes it
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  typename Mfma<ACC>::acc_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0;

  // Element q of this thread in a slab: A (m, k) and B (k, n), consecutive threads
  // along the stored contiguous dimension.
  auto a_mk = [&](int q, int& mm, int& kk) {
    if (TA_T) { mm = tid & 63; kk = (tid >> 6) + 4 * q; }   // A stored K x M: contiguous in m
    else      { kk = tid & 31; mm = (tid >> 5) + 8 * q; }   // A stored M x K: contiguous in k
  };
  auto b_kn = [&](int q, int& kk, int& nn) {
    if (TB_T) { kk = tid & 31; nn = (tid >> 5) + 8 * q; }   // B stored N x K: contiguous in k
    else      { nn = tid & 63; kk = (tid >> 6) + 4 * q; }   // B stored K x N: contiguous in n
  };
  ACC ra[8], rb[8];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      int mm, kk;
      a_mk(q, mm, kk);
      const int gm = m0 + mm, gk = k0 + kk;
      ra[q] = (gm < p.M && gk < K) ? (ACC)(TA_T ? A[(long)gk * p.lda + gm] : A[(long)gm * p.lda + gk]) : (ACC)0;
      int nn;
      b_kn(q, kk, nn);
      const int gn = n0 + nn, gk2 = k0 + kk;
      rb[q] = (gn < p.N && gk2 < K) ? (ACC)(TB_T ? B[(long)gn * p.ldb + gk2] : B[(long)gk2 * p.ldb + gn]) : (ACC)0;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      int mm, kk, nn;
      a_mk(q, mm, kk);
      As[kk][mm] = ra[q];
      b_kn(q, kk, nn);
      Bs[kk][nn] = rb[q];
    }
  };

  fetch(0);
  stage();
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) fetch(k0 + BK);   // in flight during the multiplies below
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
    if (more) {
      stage();
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gm = m0 + wm * 32 + i * 16 + Mfma<ACC>::row(lane, v);
        const int gn = n0 + wn * 32 + j * 16 + (lane & 15);
        if (gm < p.M && gn < p.N && !(p.sym && gn < gm)) {
          TC* dst = C + (long)gm * ldc + gn;
          double r = p.alpha * (double)acc[i][j][v];
          if (p.beta != 0.0) r += p.beta * (double)*dst;
          *dst = (TC)r;
          if (p.sym && gn != gm) C[(long)gn * ldc + gm] = (TC)r;
        }
      }
}

// Large products with both operands stored K-major (A as K x M, B as K x N), one type for
// operands, result and arithmetic, M a multiple of TM and N of TN (the float32 sweeps' C Q,
// with C read as its transpose): TM x TN output tiles, 4 waves in 2 x 2 of
// (TM/2) x (TN/2), K in 16-deep slabs double-buffered in LDS with one barrier per slab, the
// next slab's loads in flight in registers while the current one is multiplied.  Both
// operands are staged along their contiguous rows.
constexpr int TKS = 16;
template <typename T, int TM, int TN>
__global__ __launch_bounds__(256) void gemm_tn_kernel(Args p) {
  constexpr int FI = TM / 32, FJ = TN / 32;         // MFMA tiles per wave along M and N
  constexpr int QA = TKS * TM / 256, QB = TKS * TN / 256;   // elements per thread per slab
  __shared__ T As[2][TKS][TM + 4];
  __shared__ T Bs[2][TKS][TN + 4];
  const int z = blockIdx.z;
  const T* A = (const T*)p.A + z * p.sA;
  const T* B = (const T*)p.B + z * p.sB;
  T* C = (T*)p.C + z * p.sC;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  typename Mfma<T>::acc_t acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0;
  // element q of this thread in a slab: column tid % TM (TN) of row tid / TM (TN) + q 256 / TM (TN)
  T ra[QA], rb[QB];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int e = tid + 256 * q, gk = k0 + e / TM;
      ra[q] = gk < p.K ? A[(long)gk * p.lda + m0 + e % TM] : (T)0;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int e = tid + 256 * q, gk = k0 + e / TN;
      rb[q] = gk < p.K ? B[(long)gk * p.ldb + n0 + e % TN] : (T)0;
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int e = tid + 256 * q;
      As[buf][e / TM][e % TM] = ra[q];
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int e = tid + 256 * q;
      Bs[buf][e / TN][e % TN] = rb[q];
    }
  };
  fetch(0);
  stage(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < p.K; k0 += TKS) {
    const bool more = k0 + TKS < p.K;
    if (more) fetch(k0 + TKS);
#pragma unroll
    for (int ks = 0; ks < TKS; ks += 4) {
      T a[FI], b[FJ];
#pragma unroll
      for (int i = 0; i < FI; ++i) a[i] = As[buf][ks + (lane >> 4)][wm * (TM / 2) + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < FJ; ++j) b[j] = Bs[buf][ks + (lane >> 4)][wn * (TN / 2) + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = Mfma<T>::op(a[i], b[j], acc[i][j]);
    }
    if (more) stage(buf ^ 1);   // the other buffer was last read before the previous barrier
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gm = m0 + wm * (TM / 2) + i * 16 + Mfma<T>::row(lane, v);
        const int gn = n0 + wn * (TN / 2) + j * 16 + (lane & 15);
        T* dst = C + (long)gm * p.ldc + gn;
        double r = p.alpha * (double)acc[i][j][v];
        if (p.beta != 0.0) r += p.beta * (double)*dst;
        *dst = (T)r;
      }
}

template <typename T, int TM, int TN>
hipError_t run_tn(const GemmDesc& d, hipStream_t st) {
  Args p{d.M, d.N, d.K, d.A, d.lda, d.sA, d.B, d.ldb, d.sB, d.C, d.ldc, d.sC, d.alpha, d.beta, d.sym,
         d.batch, 1, d.K, nullptr};
  hipLaunchKernelGGL((gemm_tn_kernel<T, TM, TN>), dim3(d.N / TN, d.M / TM, d.batch), dim3(256), 0, st, p);
  return hipGetLastError();
}

// C[side] = the sum of the side's ksplit partial products, in the order of their K ranges.
__global__ __launch_bounds__(256) void sum_parts_kernel(const double* part, int ksplit, int batch, long mn, double* C,
                                                        long sC) {
  const int side = blockIdx.y;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < mn; e += (long)gridDim.x * 256) {
    double t = 0.0;
    for (int q = 0; q < ksplit; ++q) t += part[((long)q * batch + side) * mn + e];
    C[side * sC + e] = t;
  }
}

template <typename TA, typename TB, typename TC, typename ACC>
hipError_t run(const GemmDesc& d, hipStream_t st) {
  Args p{d.M, d.N, d.K, d.A, d.lda, d.sA, d.B, d.ldb, d.sB, d.C, d.ldc, d.sC, d.alpha, d.beta, d.sym,
         d.batch, 1, d.K, d.part};
  if (d.ksplit > 1 && d.part) {
    p.ksplit = d.ksplit;
    p.kchunk = (d.K + d.ksplit - 1) / d.ksplit;
  }
  dim3 grid((d.N + BN - 1) / BN, (d.M + BM - 1) / BM, d.batch * p.ksplit);
  if (d.ta && d.tb) hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, true, true>), grid, dim3(256), 0, st, p);
  else if (d.ta)    hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, true, false>), grid, dim3(256), 0, st, p);
  else if (d.tb)    hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, false, true>), grid, dim3(256), 0, st, p);
  else              hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, ACC, false, false>), grid, dim3(256), 0, st, p);
  if (p.ksplit > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long mn = (long)d.M * d.N;
    hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)std::min<long>((mn + 255) / 256, 1024), d.batch), dim3(256),
                       0, st, d.part, p.ksplit, d.batch, mn, (double*)d.C, d.sC);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t gemm(const GemmDesc& d, hipStream_t st) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  if (d.sym && (d.M != d.N || d.beta != 0.0)) return hipErrorInvalidValue;
  // split K: partial products of type double, packed M x N, summed into C (whose rows must be packed)
  if (d.ksplit > 1 && (!d.part || d.typeC != GF64 || d.ldc != d.N || d.alpha != 1.0 || d.beta != 0.0))
    return hipErrorInvalidValue;
  const int code = (d.typeA << 3) | (d.typeB << 2) | (d.typeC << 1) | d.acc;
  // float32 products with K-major operands on 128 x 128 tiles (2.19 ms for the 64k half's C Q
  // against 2.57 ms on 64 x 64).  Float64 stays on 64 x 64: with the K-major kernel its C Q took
  // 4.72 ms on 128 x 128 tiles (332 registers per lane, one wave per SIMD) and 4.33 ms on
  // 128 x 64, Y^T Y 1.53 and 1.14 ms, against 4.09 and 0.87 ms.
  if (d.ta && !d.tb && d.K > 0 && code == 0b0000 && d.M % 128 == 0 && d.N % 128 == 0 && !d.sym)
    return run_tn<float, 128, 128>(d, st);
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
