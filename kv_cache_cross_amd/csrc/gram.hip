// Gram C = X^T X of one group side, X = [K_l1 | ... | K_lG] (never materialised).
//
// The uncentred covariance of the concatenated rows gives the right singular
// vectors of X (KV-CoRE, section 2.A); xKV factors the horizontally
// concatenated group once (xKV blog, section on what xKV does).
//
// bf16 path, one 512-thread workgroup per 256 x 256 tile of the upper triangle
// (I <= J; a diagonal tile reads its column block once):
//   * 32-token slabs of the I and J column blocks go from HBM straight into LDS
//     with direct-to-LDS loads (no registers), three slabs ahead of the math, in a
//     ring of four stages.  A stage is a set of 1 KiB blocks of 16 tokens x 32
//     columns, one load instruction each;
//   * the MFMA operands are read with the LDS transpose load ds_read_b64_tr_b16: in
//     each group of 16 lanes, lane i receives column i of four consecutive token rows
//     of a 4 x 16 block, so two such reads give a lane the 8 consecutive tokens of one
//     column that v_mfma_f32_32x32x16_bf16 takes for both operands;
//   * 8 waves in a 2 x 4 grid, 128 x 64 outputs per wave (4 x 2 MFMA tiles), so an
//     operand read from LDS feeds 2 or 4 MFMAs;
//   * float32 MFMA sums cover a segment of 1024 tokens; at each segment end they are
//     added into the float64 output tile in memory (the tile belongs to this
//     workgroup alone).  The segment is short because the matrix cores' float32
//     accumulation is biased toward zero: terms much smaller than the largest one of
//     an accumulation lose their low bits (a probe: the products 1 and 0.75 ulp(1) in
//     one instruction sum to 1, not 1 + ulp), so the relative error of a partial grows
//     in proportion to its length rather than its square root.  Measured at the 16k
//     Llama-shaped group (n = 4096, r = 512), the projector's distance to the float64
//     one is 2.7e-3 with 8192-token segments, 6.9e-4 with 2048, 3.3e-4 with 1024;
//   * the last segment also writes the mirror tile and the float32 copy used by the
//     float32 subspace iterations.
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int GT = 256;                      // output tile edge
constexpr int TS = 32;                       // tokens per slab
constexpr int NST = 4;                       // LDS stages
constexpr int STAGE = 2 * 8 * 2 * 1024;      // bytes per stage: [op][32-col block][16-token half][16][32]
constexpr int SEG = 1024;                    // tokens per float32 partial

typedef short v4s __attribute__((ext_vector_type(4)));

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

// Workgroup barrier without a memory fence: a fence would wait for every load into
// LDS in flight, the loads into later stages included.  The caller waits for what the
// barrier must cover (its own loads into the stage about to be read, with vmcnt; its
// LDS stores, with lgkmcnt); the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Two transpose reads (token rows r and r + 4 of a block) make one MFMA operand.
__device__ __forceinline__ bf16x8_t tr_operand(const unsigned char* p) {
  union {
    v4s h[2];
    bf16x8_t b;
  } u;
  u.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  u.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 4 * 64));
  return u.b;
}

__global__ __launch_bounds__(512) void gram_bf16_kernel(GramArgs a) {
  // The four stages are separate arrays, each named by a constant at every use, so
  // that a load into one stage is known not to touch the stage being read.
  __shared__ __align__(16) unsigned char st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
  // XCD-aware order: the dispatcher hands block b to XCD b % 8, so logical tile
  // (b % 8) q + b / 8 gives each XCD a contiguous range of the row-major upper-triangle
  // tile list (q = blocks / 8).  The tiles an XCD runs at once then share their row block
  // and most column blocks, and its L2 serves the repeats: the L2-miss traffic of the
  // 64k Gram halves (from 2 x 62.3 to about 2 x 35 GiB per launch).
  const int nblk = gridDim.x, q8 = nblk / 8, b = blockIdx.x;
  const int lt = b < 8 * q8 ? (b % 8) * q8 + b / 8 : b;
  const int side = lt / a.tiles_per_side;
  int I, J;
  upper_tile(lt % a.tiles_per_side, a.nt, &I, &J);
  const bool diag = (I == J);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;   // wave tile: rows wm*128.., cols wn*64..

  // Load role: wave w moves blocks 4w .. 4w+3 of a slab: operand w / 4, 32-column
  // blocks 2w % 8 and (2w + 1) % 8, both token halves.  Lane l fills 16-byte slot l of
  // the block: token row l / 4 of the half, column group (l % 4) ^ (row % 4), i.e.
  // columns 8 ((l % 4) ^ ((l / 4) % 4)) .. + 7 (the swizzle keeps the transpose reads
  // below free of bank conflicts).  Threads whose
  // column is past n read column 0 of the first layer (never used).  Every wave loads,
  // so that the number of loads in flight is the same on every path: the second
  // operand of a diagonal tile repeats the first (a cache hit, never read).
  const int dop = wave >> 2;
  const unsigned char* base[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int cb = (2 * wave + u) & 7;
    const int col = (dop && !diag ? J : I) * GT + 32 * cb + 8 * ((lane & 3) ^ ((lane >> 2) & 3));
    const unsigned char* p = (const unsigned char*)a.layers.p[side * a.G];
    if (col < a.n) {
      const int l = col / a.d_kv;
      p = (const unsigned char*)a.layers.p[side * a.G + l] + 2 * (col - l * a.d_kv);
    }
    base[u] = p;
  }
  const uint32_t ldb = (uint32_t)a.ld * 2u;   // byte offsets within a layer fit 32 bits (host check)
  // Every wave issues exactly four load instructions per slab, so the wait for slab s
  // is a fixed count; past the last slab the last one is read again.
  auto dma_slab = [&](int sl, unsigned char* stage) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = i >> 1, half = i & 1;
      const int cb = (2 * wave + u) & 7;
      const int t = min(sl * TS + 16 * half + (lane >> 2), a.T - 1);
      unsigned char* dst = stage + ((dop * 8 + cb) * 2 + half) * 1024;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base[u] + (uint32_t)t * ldb),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

  const long nn = (long)a.n * a.n;
  double* C = a.C + side * nn;
  float* C32 = a.C32 ? a.C32 + side * nn : nullptr;
  // Fold the float32 partial into the float64 tile (first segment: store).  Element j
  // of MFMA tile (mi, ni) of this lane is row m0 + 32 mi + 8 (j / 4) + j % 4, column
  // c0 + 32 ni.
  auto flush = [&](bool first, bool last) {
    // The row stride is made opaque here, so that no output address is computed ahead
    // of the slab loop and held in registers through it.
    long nrow = a.n;
    __asm__ volatile("" : "+s"(nrow));
    int m0 = I * GT + wm * 128 + (lane >> 5) * 4, c0 = J * GT + wn * 64 + (lane & 31);
    __asm__ volatile("" : "+v"(m0), "+v"(c0));
    double* Cb = C + (long)m0 * nrow + c0;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          // four elements at a time, so that few float64 values are live at once
          if ((j & 3) == 0) __asm__ volatile("" ::: "memory");
          const int m = m0 + mi * 32 + (j >> 2) * 8 + (j & 3), c = c0 + ni * 32;
          if (m < nrow && c < nrow) {
            double* p = Cb + (long)(mi * 32 + (j >> 2) * 8 + (j & 3)) * nrow + ni * 32;
            const double v = (first ? 0.0 : *p) + (double)acc[mi][ni][j];
            *p = v;
            if (last) {
              if (!diag) C[(long)c * nrow + m] = v;
              if (C32) {
                C32[(long)m * nrow + c] = (float)v;
                if (!diag) C32[(long)c * nrow + m] = (float)v;
              }
            }
          }
          acc[mi][ni][j] = 0.f;
        }
      }
  };

  // Operand reads.  Lane l (group q = l / 16, i = l % 16) points at token row
  // 8 (q / 2) + i / 4 and column 16 (q % 2) + 4 (i % 4) of a block (16-byte column
  // group 2 (q % 2) + (i % 4) / 2, placed at slot group ^ (row % 4), half i % 2); the
  // transpose read then hands it column 16 (q % 2) + i = l % 32 of token rows
  // 8 (q / 2) + 0..3.  In each 16-lane group the four rows' 32 bytes fall in distinct
  // quarters of 128 bytes.
  const int q16 = lane >> 4, i16 = lane & 15;
  const int lane_off = (8 * (q16 >> 1) + (i16 >> 2)) * 64 +
                       16 * ((2 * (q16 & 1) + ((i16 >> 1) & 1)) ^ ((i16 >> 2) & 3)) + 8 * (i16 & 1);
  const int opB = diag ? 0 : 1;
  auto compute = [&](const unsigned char* stage) {
    const unsigned char* sb = stage + lane_off;
#pragma unroll
    for (int ks = 0; ks < TS / 16; ++ks) {
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = tr_operand(sb + ((0 * 8 + 4 * wm + mi) * 2 + ks) * 1024);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bfr[ni] = tr_operand(sb + ((opB * 8 + 2 * wn + ni) * 2 + ks) * 1024);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);   // one k-step's operands live at a time
    }
  };

  const int n_slabs = (a.T + TS - 1) / TS;
  // One slab: wait for its loads, start the load three slabs ahead into the stage
  // read one slab ago, then the math.  vmcnt(8): of this wave's loads in flight
  // (slabs s, s+1, s+2, four each), slab s's have landed; the barrier extends that to
  // every wave and ends the reads of slab s - 1.  Loads are issued for every slab
  // position up to a multiple of four (past the end: the last slab again), so the
  // count never depends on a branch; only the math is skipped there.
  auto body = [&](int s, unsigned char* cur, unsigned char* ahead) {
    __builtin_amdgcn_s_waitcnt(0x0F78);
    lds_barrier();
    dma_slab(min(s + 3, n_slabs - 1), ahead);
    if (s < n_slabs) {
      if (s * TS + TS > a.T) {   // last, partial slab: zero the token rows past T
        const int op = tid >> 8, cb = (tid >> 5) & 7, tok = tid & 31;
        if (s * TS + tok >= a.T) {
          uint4* row = (uint4*)(cur + ((op * 8 + cb) * 2 + (tok >> 4)) * 1024 + (tok & 15) * 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) row[e] = make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the zero rows are written
        lds_barrier();
      }
      compute(cur);
      const int t_end = (s + 1) * TS;
      if (t_end % SEG == 0 || s + 1 == n_slabs) {
        flush(t_end <= SEG, s + 1 == n_slabs);
        __builtin_amdgcn_s_waitcnt(0);
      }
    }
  };
  dma_slab(0, st0);
  dma_slab(min(1, n_slabs - 1), st1);
  dma_slab(min(2, n_slabs - 1), st2);
  for (int s = 0; s < n_slabs; s += NST) {
    body(s, st0, st3);
    body(s + 1, st1, st0);
    body(s + 2, st2, st1);
    body(s + 3, st3, st2);
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the workgroup
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



hipError_t launch_gram_bf16(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                            double* C, float* C32, hipStream_t st) {
  if ((long)T * ld >= (1L << 31)) return hipErrorInvalidValue;   // 32-bit byte offsets per layer
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
  hipLaunchKernelGGL(gram_bf16_kernel, dim3(a.tiles_per_side * n_sides), dim3(512), 0, st, a);
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
