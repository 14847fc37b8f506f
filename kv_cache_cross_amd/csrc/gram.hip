// Gram C = X^T X of one group side, X = [K_l1 | ... | K_lG] (never materialised).
//
// The uncentred covariance of the concatenated rows gives the right singular
// vectors of X (KV-CoRE, section 2.A); xKV factors the horizontally
// concatenated group once (xKV blog, section on what xKV does).
//
// bf16 path, one 256-thread workgroup (four waves, one per SIMD, each with the
// whole register file of its lane) per 256 x 128 tile of the upper triangle
// (rows I*256.., columns J*128.., tiles with J >= 2 I; a tile that straddles the
// diagonal writes its elements on or above it):
//   * 32-token slabs of the tile's 256 + 128 columns go from HBM straight into LDS
//     with direct-to-LDS loads (no registers), three slabs ahead of the math, in a
//     ring of four stages.  A stage is 24 blocks of 16 tokens x 32 columns (1 KiB,
//     one load instruction each);
//   * the MFMA operands are read with the LDS transpose load ds_read_b64_tr_b16: in
//     each group of 16 lanes, lane i receives column i of four consecutive token rows
//     of a 4 x 16 block, so two such reads give a lane the 8 consecutive tokens of one
//     column that v_mfma_f32_32x32x16_bf16 takes for both operands;
//   * wave w computes the 128 x 64 outputs (4 x 2 MFMA tiles) at rows 128 (w / 2),
//     columns 64 (w % 2) of the tile, so an operand read from LDS feeds 2 or 4 MFMAs;
//   * two-level sums: the matrix cores accumulate 512 tokens at a time into float32
//     registers, which are then added on the vector ALU into a compensated (Kahan)
//     float32 pair of registers that holds the whole sum; the tile is written once,
//     as float64 (and the float32 copy the float32 iterations use).  The short
//     matrix-core span matters because their float32 accumulation is biased toward
//     zero: terms much smaller than the largest one of an accumulation lose their low
//     bits (a probe: the products 1 and 0.75 ulp(1) in one instruction sum to 1, not
//     1 + ulp), so a partial's relative error grows in proportion to its length.
//     Measured at the 16k Llama-shaped group (n = 4096, r = 512), the projector's
//     distance to the float64 one is 2.7e-3 with 8192-token partials, 3.3e-4 with
//     1024 and 1.7e-4 with 512.  The total needs more than float32: rounding the
//     exact 16k Gram to float32 alone moves that projector by 1.9e-4, and a plain
//     float32 running sum of the 512-token partials by ~6e-4.
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int TI = 256;                      // tile rows (the I column block)
constexpr int TJ = 128;                      // tile columns (the J column block)
constexpr int TS = 32;                       // tokens per slab
constexpr int NST = 4;                       // LDS stages
constexpr int NCB = (TI + TJ) / 32;          // 32-column blocks per slab: 8 of I, 4 of J
constexpr int STAGE = NCB * 2 * 1024;        // bytes per stage: [col block][16-token half][16][32]
constexpr int SUB = 16 * TS;                 // tokens per matrix-core partial of a tile (the fold period)

typedef short v4s __attribute__((ext_vector_type(4)));

struct GramArgs {
  PtrTable layers;
  int G, T, d_kv, n, nI, nJ, tiles_per_side;
  long ld;
  double* C;
  float* C32;
};

// Tile idx of one side's list (row-major over I, then J = 2 I ..).
__device__ __forceinline__ void upper_tile(int idx, int nI, int nJ, int* I, int* J) {
  int i = 0;
  while (i < nI && idx >= nJ - 2 * i) {
    idx -= nJ - 2 * i;
    ++i;
  }
  *I = i;
  *J = 2 * i + idx;
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

// s_waitcnt with vmcnt(n) and the other counters left alone.
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__global__ __launch_bounds__(256) void gram_bf16_kernel(GramArgs a) {
  // The four stages are separate arrays, each named by a constant at every use, so
  // that a load into one stage is known not to touch the stage being read.
  __shared__ __align__(16) unsigned char st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
  // XCD-aware order: the dispatcher hands block b to XCD b % 8, so logical tile
  // (b % 8) q + b / 8 gives each XCD a contiguous range of the row-major tile list
  // (q = blocks / 8).  The tiles an XCD runs at once then share their row block and
  // most column blocks, and its L2 serves the repeats.
  const int nblk = gridDim.x, q8 = nblk / 8, b = blockIdx.x;
  const int lt = b < 8 * q8 ? (b % 8) * q8 + b / 8 : b;
  const int side = lt / a.tiles_per_side;
  int I, J;
  upper_tile(lt % a.tiles_per_side, a.nI, a.nJ, &I, &J);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;   // wave tile: rows wm*128.., cols wn*64..

  // Load role: wave w moves column blocks 3w .. 3w+2 of the slab (blocks 0..7: the I
  // columns I*256 + 32 cb, blocks 8..11: the J columns J*128 + 32 (cb - 8)), both
  // token halves.  Lane l fills 16-byte slot l of a block: token row l / 4 of the
  // half, column group (l % 4) ^ (row % 4), i.e. columns 8 ((l % 4) ^ ((l / 4) % 4))
  // .. + 7 (the swizzle keeps the transpose reads below free of bank conflicts).
  // Threads whose column is past n read column 0 of the first layer (never used).
  const unsigned char* base[3];
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int cb = 3 * wave + u;
    const int cstart = cb < 8 ? I * TI + 32 * cb : J * TJ + 32 * (cb - 8);
    const int col = cstart + 8 * ((lane & 3) ^ ((lane >> 2) & 3));
    const unsigned char* p = (const unsigned char*)a.layers.p[side * a.G];
    if (col < a.n) {
      const int l = col / a.d_kv;
      p = (const unsigned char*)a.layers.p[side * a.G + l] + 2 * (col - l * a.d_kv);
    }
    base[u] = p;
  }
  const uint32_t ldb = (uint32_t)a.ld * 2u;   // byte offsets within a layer fit 32 bits (host check)
  // Every wave issues exactly six load instructions per slab, so the wait for slab s
  // is a fixed count; past the last slab the last one is read again.
  auto dma_slab = [&](int sl, unsigned char* stage) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int u = i >> 1, half = i & 1;
      const int cb = 3 * wave + u;
      const int t = min(sl * TS + 16 * half + (lane >> 2), a.T - 1);
      unsigned char* dst = stage + (cb * 2 + half) * 1024;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base[u] + (uint32_t)t * ldb),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };

  f32x16_t acc[4][2];
  float sum[4][2][16], cmp[4][2][16];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc[mi][ni][j] = 0.f;
        sum[mi][ni][j] = 0.f;
        cmp[mi][ni][j] = 0.f;
      }
  // The matrix-core partial into the register-resident total, compensated (Kahan):
  // cmp collects the rounding error of every addition, so the total keeps about twice
  // float32's precision (a plain float32 running sum would add a random walk of
  // roundings that alone moves the 16k group's projector by ~6e-4).
  // One MFMA tile (MI, NI), with constant indices so that every array stays in
  // registers; fold_tile dispatches a wave-uniform tile number t = 2 MI + NI.
#define XKV_GRAM_FOLD(MI, NI)                                   \
  _Pragma("unroll") for (int j = 0; j < 16; ++j) {              \
    const float y = acc[MI][NI][j] - cmp[MI][NI][j];            \
    const float z = sum[MI][NI][j] + y;                         \
    cmp[MI][NI][j] = (z - sum[MI][NI][j]) - y;                  \
    sum[MI][NI][j] = z;                                         \
    acc[MI][NI][j] = 0.f;                                       \
  }
  auto fold_tile = [&](int t) __attribute__((always_inline)) {
    switch (t) {
      case 0: XKV_GRAM_FOLD(0, 0) break;
      case 1: XKV_GRAM_FOLD(0, 1) break;
      case 2: XKV_GRAM_FOLD(1, 0) break;
      case 3: XKV_GRAM_FOLD(1, 1) break;
      case 4: XKV_GRAM_FOLD(2, 0) break;
      case 5: XKV_GRAM_FOLD(2, 1) break;
      case 6: XKV_GRAM_FOLD(3, 0) break;
      default: XKV_GRAM_FOLD(3, 1) break;
    }
  };
#undef XKV_GRAM_FOLD

  // Operand reads.  Lane l (group q = l / 16, i = l % 16) points at token row
  // 8 (q / 2) + i / 4 and column 16 (q % 2) + 4 (i % 4) of a block (16-byte column
  // group 2 (q % 2) + (i % 4) / 2, placed at slot group ^ (row % 4), half i % 2); the
  // transpose read then hands it column 16 (q % 2) + i = l % 32 of token rows
  // 8 (q / 2) + 0..3.  In each 16-lane group the four rows' 32 bytes fall in distinct
  // quarters of 128 bytes.
  const int q16 = lane >> 4, i16 = lane & 15;
  const int lane_off = (8 * (q16 >> 1) + (i16 >> 2)) * 64 +
                       16 * ((2 * (q16 & 1) + ((i16 >> 1) & 1)) ^ ((i16 >> 2) & 3)) + 8 * (i16 & 1);
  auto compute = [&](const unsigned char* stage) {
    const unsigned char* sb = stage + lane_off;
#pragma unroll
    for (int ks = 0; ks < TS / 16; ++ks) {
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = tr_operand(sb + ((4 * wm + mi) * 2 + ks) * 1024);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bfr[ni] = tr_operand(sb + ((8 + 2 * wn + ni) * 2 + ks) * 1024);
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
  // read one slab ago, then the math.  vmcnt(12): of this wave's loads in flight
  // (slabs s, s+1, s+2, six each), slab s's have landed; the barrier extends that to
  // every wave and ends the reads of slab s - 1.  Loads are issued for every slab
  // position up to a multiple of four (past the end: the last slab again), so the
  // count never depends on a branch; only the math is skipped there.
  // The eight MFMA tiles fold at different slabs of each 16-slab (512-token) period,
  // tile t after slab t, so that one tile's vector-ALU work runs while the matrix
  // cores still work through the other tiles of the slab.
  auto body = [&](int s, const int k, unsigned char* cur, unsigned char* ahead) {
    __builtin_amdgcn_s_waitcnt(vm_wait(12));
    lds_barrier();
    dma_slab(min(s + 3, n_slabs - 1), ahead);
    if (s < n_slabs) {
      if (s * TS + TS > a.T) {   // last, partial slab: zero the token rows past T
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
          const int idx = tid + 256 * rep;   // (column block, token) pairs: 12 x 32
          const int cb = idx >> 5, tok = idx & 31;
          if (idx < NCB * 32 && s * TS + tok >= a.T) {
            uint4* row = (uint4*)(cur + (cb * 2 + (tok >> 4)) * 1024 + (tok & 15) * 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) row[e] = make_uint4(0, 0, 0, 0);
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the zero rows are written
        lds_barrier();
      }
      compute(cur);
      if ((s & 8) == 0) fold_tile((s & 4) + k);
    }
  };
  dma_slab(0, st0);
  dma_slab(min(1, n_slabs - 1), st1);
  dma_slab(min(2, n_slabs - 1), st2);
  for (int s = 0; s < n_slabs; s += NST) {
    body(s, 0, st0, st3);
    body(s + 1, 1, st1, st0);
    body(s + 2, 2, st2, st1);
    body(s + 3, 3, st3, st2);
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the workgroup
#pragma unroll
  for (int t = 0; t < 8; ++t) fold_tile(t);

  // Write the tile: element j of MFMA tile (mi, ni) of this lane is row
  // m0 + 32 mi + 8 (j / 4) + j % 4, column c0 + 32 ni; only elements on or above the
  // diagonal, each also at its mirror position.
  const long nn = (long)a.n * a.n;
  double* C = a.C + side * nn;
  float* C32 = a.C32 ? a.C32 + side * nn : nullptr;
  const int nrow = a.n;
  const int m0 = I * TI + wm * 128 + (lane >> 5) * 4, c0 = J * TJ + wn * 64 + (lane & 31);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = m0 + mi * 32 + (j >> 2) * 8 + (j & 3), c = c0 + ni * 32;
        if (m < nrow && c < nrow && c >= m) {
          const double v = (double)sum[mi][ni][j] - (double)cmp[mi][ni][j];
          C[(long)m * nrow + c] = v;
          if (c != m) C[(long)c * nrow + m] = v;
          if (C32) {
            C32[(long)m * nrow + c] = (float)v;
            if (c != m) C32[(long)c * nrow + m] = (float)v;
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



hipError_t launch_gram_bf16(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                            double* C, float* C32, hipStream_t st) {
  if ((long)T * ld >= (1L << 31)) return hipErrorInvalidValue;   // 32-bit byte offsets per layer
  GramArgs a;
  a.layers = layers;
  a.G = G;
  a.T = T;
  a.d_kv = d_kv;
  a.n = G * d_kv;
  a.nI = (a.n + TI - 1) / TI;
  a.nJ = 2 * a.nI;
  a.tiles_per_side = 0;
  for (int i = 0; i < a.nI; ++i) a.tiles_per_side += a.nJ - 2 * i;
  a.ld = ld;
  a.C = C;
  a.C32 = C32;
  hipLaunchKernelGGL(gram_bf16_kernel, dim3(a.tiles_per_side * n_sides), dim3(256), 0, st, a);
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
