// Gram C = X^T X of one group side, X = [K_l1 | ... | K_lG] (never materialised).
//
// The uncentred covariance of the concatenated rows gives the right singular
// vectors of X (KV-CoRE, section 2.A); xKV factors the horizontally
// concatenated group once (xKV blog, section on what xKV does).
//
// bf16 path, one workgroup per 128 x 128 tile of the upper triangle (I <= J):
//   * a 64-token slab of the I and J column blocks is read from HBM with
//     16-byte loads, transposed 8x8 in registers and stored token-contiguous
//     in LDS (double buffered), so that every MFMA operand is one 16-byte LDS
//     read: v_mfma_f32_32x32x16_bf16 wants 8 consecutive tokens of one column
//     per lane for both operands;
//   * 4 waves in a 2 x 2 grid, 64 x 64 outputs per wave (2 x 2 MFMA tiles);
//   * float32 MFMA sums cover 256 tokens, then are added into float64
//     register totals, so rounding is relative to a 256-token partial rather
//     than to the full sum (the eigengap at the target rank is ~3e-3 relative,
//     which a float32 full-length sum does not resolve);
//   * the tile and its mirror are written in float64 (and float32 for the
//     float32 subspace iterations).
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int GT = 128;            // output tile edge
constexpr int SLAB = 64;           // tokens per LDS stage
constexpr int LDS_ROW = SLAB + 8;  // padded LDS row (uint16 elements): 144 bytes
constexpr int OUTER = 4;           // slabs per float32 partial (256 tokens)

struct GramArgs {
  PtrTable layers;
  int G, T, d_kv, n, nt, tiles_per_side;
  long ld;
  double* C;
  float* C32;
};

__device__ __forceinline__ void upper_tile(int idx, int nt, int* I, int* J) {
  int i = 0;
  while (idx >= nt - i) {
    idx -= nt - i;
    ++i;
  }
  *I = i;
  *J = i + idx;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

__global__ __launch_bounds__(256) void gram_bf16_kernel(GramArgs a) {
  extern __shared__ __align__(16) uint16_t lds_raw[];
  // lds[buf][operand][column][token]
  auto lds = [&](int buf, int op, int c, int t) -> uint16_t* {
    return lds_raw + (((buf * 2 + op) * GT + c) * LDS_ROW + t);
  };
  const int side = blockIdx.x / a.tiles_per_side;
  int I, J;
  upper_tile(blockIdx.x % a.tiles_per_side, a.nt, &I, &J);
  const bool diag = (I == J);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Loader role: 8 tokens x 8 columns of one operand per thread.
  const int op = tid >> 7;
  const int tg = (tid & 127) >> 4;
  const int cg = tid & 15;
  const bool loader = !(diag && op == 1);
  const int col = (op ? J : I) * GT + cg * 8;
  const uint16_t* src = nullptr;
  if (loader && col < a.n) {
    const int l = col / a.d_kv;
    src = (const uint16_t*)a.layers.p[side * a.G + l] + (col - l * a.d_kv);
  }
  uint4 rows[8];

  auto gload = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = t0 + tg * 8 + i;
      rows[i] = (src && t < a.T) ? *(const uint4*)(src + (long)t * a.ld) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    if (!loader) return;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int w = c >> 1;
      uint32_t q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = word_of(rows[2 * j], w), hi = word_of(rows[2 * j + 1], w);
        q[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *(uint4*)lds(buf, op, cg * 8 + c, tg * 8) = make_uint4(q[0], q[1], q[2], q[3]);
    }
  };

  f32x16_t acc[2][2];
  double tot[2][2][16];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc[mi][ni][j] = 0.f;
        tot[mi][ni][j] = 0.0;
      }

  const int n_slabs = (a.T + SLAB - 1) / SLAB;
  const int opB = diag ? 0 : 1;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < n_slabs; ++s) {
    const int buf = s & 1;
    if (s + 1 < n_slabs) gload((s + 1) * SLAB);
#pragma unroll
    for (int ks = 0; ks < SLAB / 16; ++ks) {
      const int t_off = ks * 16 + (lane >> 5) * 8;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = as_bf16x8(*(const uint4*)lds(buf, 0, wm * 64 + mi * 32 + (lane & 31), t_off));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = as_bf16x8(*(const uint4*)lds(buf, opB, wn * 64 + ni * 32 + (lane & 31), t_off));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (s + 1 < n_slabs) lstore(buf ^ 1);
    if ((s + 1) % OUTER == 0 || s + 1 == n_slabs) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            tot[mi][ni][j] += (double)acc[mi][ni][j];
            acc[mi][ni][j] = 0.f;
          }
    }
    __syncthreads();
  }

  const long nn = (long)a.n * a.n;
  double* C = a.C + side * nn;
  float* C32 = a.C32 ? a.C32 + side * nn : nullptr;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = I * GT + wm * 64 + mi * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
        const int c = J * GT + wn * 64 + ni * 32 + (lane & 31);
        if (m < a.n && c < a.n) {
          const double v = tot[mi][ni][j];
          C[(long)m * a.n + c] = v;
          if (!diag) C[(long)c * a.n + m] = v;
          if (C32) {
            C32[(long)m * a.n + c] = (float)v;
            if (!diag) C32[(long)c * a.n + m] = (float)v;
          }
        }
      }
}

// float32 layers (small workloads): 16 x 16 output tiles, float64 sums.
struct GramF32Args {
  PtrTable layers;
  int G, T, d_kv, n, nt16;
  long ld;
  double* C;
  float* C32;
};

__global__ __launch_bounds__(256) void gram_f32_kernel(GramF32Args a) {
  __shared__ float xi[16][17], xj[16][17];
  const int side = blockIdx.z;
  const int I = blockIdx.y, J = blockIdx.x;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  auto ptr = [&](int col) -> const float* {
    const int l = col / a.d_kv;
    return (const float*)a.layers.p[side * a.G + l] + (col - l * a.d_kv);
  };
  const int ci = I * 16 + tx, cj = J * 16 + tx;
  const float* pi = ci < a.n ? ptr(ci) : nullptr;
  const float* pj = cj < a.n ? ptr(cj) : nullptr;
  double s = 0.0;
  for (int t0 = 0; t0 < a.T; t0 += 16) {
    const int t = t0 + ty;
    xi[ty][tx] = (pi && t < a.T) ? pi[(long)t * a.ld] : 0.f;
    xj[ty][tx] = (pj && t < a.T) ? pj[(long)t * a.ld] : 0.f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) s += (double)xi[k][ty] * (double)xj[k][tx];
    __syncthreads();
  }
  const int m = I * 16 + ty, c = J * 16 + tx;
  if (m < a.n && c < a.n) {
    const long nn = (long)a.n * a.n;
    a.C[side * nn + (long)m * a.n + c] = s;
    if (a.C32) a.C32[side * nn + (long)m * a.n + c] = (float)s;
  }
}

}  // namespace

static constexpr size_t kGramLds = 2 * 2 * GT * LDS_ROW * sizeof(uint16_t);

hipError_t launch_gram_bf16(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                            double* C, float* C32, hipStream_t st) {
  GramArgs a;
  a.layers = layers;
  a.G = G;
  a.T = T;
  a.d_kv = d_kv;
  a.n = G * d_kv;
  a.nt = (a.n + GT - 1) / GT;
  a.tiles_per_side = a.nt * (a.nt + 1) / 2;
  a.ld = ld;
  a.C = C;
  a.C32 = C32;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gram_bf16_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGramLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(gram_bf16_kernel, dim3(a.tiles_per_side * n_sides), dim3(256), kGramLds, st, a);
  return hipGetLastError();
}

hipError_t launch_gram_f32(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                           double* C, float* C32, hipStream_t st) {
  GramF32Args a;
  a.layers = layers;
  a.G = G;
  a.T = T;
  a.d_kv = d_kv;
  a.n = G * d_kv;
  a.nt16 = (a.n + 15) / 16;
  a.ld = ld;
  a.C = C;
  a.C32 = C32;
  hipLaunchKernelGGL(gram_f32_kernel, dim3(a.nt16, a.nt16, n_sides), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace xkv
