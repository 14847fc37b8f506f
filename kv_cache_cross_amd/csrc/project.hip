// Projection A = X V_r (the shared token basis, xKV blog section on what xKV
// does) and the per-chunk landmark means used by the top-k chunk selector
// (xKV blog, section on Selective Reconstruction).
//
// bf16 projection: both operands are contiguous along the contracted
// dimension (X rows along columns of the group, VrT rows along the group
// columns).  When d_kv is a multiple of 32 (every workload), project_tile_kernel
// computes 256 x 256 output tiles from 32-column slices loaded straight into LDS;
// otherwise a 128 x 128 output tile stages 128 x 64 slices of each through LDS
// with 16-byte loads (double buffered).  Both feed v_mfma_f32_32x32x16_bf16 with
// one 16-byte LDS read per operand, and in both the rank tile is the
// fastest-varying workgroup index, so the workgroups that read the same X rows
// run together and share them through L2.
//
// Landmarks: m[l, h, c] = mean over the chunk's tokens of RoPE(K_l[t, h], t),
// from the original keys, float32 sums, angle formed in float64.
#include "xkv_common.h"
#include "xkv_kernels.h"

namespace xkv {
namespace {

constexpr int PT = 128;            // output tile edge (tokens and rank)
constexpr int PK = 64;             // contraction slice per stage
constexpr int PROW = PK + 8;       // padded LDS row (uint16): 144 bytes

struct ProjArgs {
  PtrTable layers;
  PtrTable A_out;
  const uint16_t* VrT;
  long sVT;
  int G, T, d_kv, n, r;
  long ld;
};

__global__ __launch_bounds__(256) void project_bf16_kernel(ProjArgs a) {
  extern __shared__ __align__(16) uint16_t lds_raw[];
  auto xs = [&](int buf, int row, int k) -> uint16_t* { return lds_raw + ((buf * 2 + 0) * PT + row) * PROW + k; };
  auto vs = [&](int buf, int row, int k) -> uint16_t* { return lds_raw + ((buf * 2 + 1) * PT + row) * PROW + k; };
  const int side = blockIdx.z;
  const int j0 = blockIdx.x * PT;    // rank tile
  const int t0 = blockIdx.y * PT;    // token tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* VrT = a.VrT + side * a.sVT;

  // Loader: 4 rows x one 8-column group per operand per thread.
  const int lrow = tid >> 3;         // 0..31
  const int lcg = tid & 7;           // 0..7
  uint4 xr[4], vr[4];
  auto gload = [&](int k0) {
    const int col = k0 + lcg * 8;
    const uint16_t* xp = nullptr;
    if (col < a.n) {
      const int l = col / a.d_kv;
      xp = (const uint16_t*)a.layers.p[side * a.G + l] + (col - l * a.d_kv);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + lrow + 32 * i;
      xr[i] = (xp && t < a.T) ? *(const uint4*)(xp + (long)t * a.ld) : make_uint4(0, 0, 0, 0);
      const int j = j0 + lrow + 32 * i;
      vr[i] = (col < a.n && j < a.r) ? *(const uint4*)(VrT + (long)j * a.n + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(uint4*)xs(buf, lrow + 32 * i, lcg * 8) = xr[i];
      *(uint4*)vs(buf, lrow + 32 * i, lcg * 8) = vr[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

  const int nk = (a.n + PK - 1) / PK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) gload((s + 1) * PK);
#pragma unroll
    for (int ks = 0; ks < PK / 16; ++ks) {
      const int k_off = ks * 16 + (lane >> 5) * 8;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) af[mi] = as_bf16x8(*(const uint4*)xs(buf, wm * 64 + mi * 32 + (lane & 31), k_off));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bfr[ni] = as_bf16x8(*(const uint4*)vs(buf, wn * 64 + ni * 32 + (lane & 31), k_off));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (s + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  uint16_t* Aout = (uint16_t*)a.A_out.p[side];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + wm * 64 + mi * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
        const int c = j0 + wn * 64 + ni * 32 + (lane & 31);
        if (t < a.T && c < a.r) Aout[(long)t * a.r + c] = f32_to_bf16_bits(acc[mi][ni][j]);
      }
}

// bf16 projection, large tiles (d_kv a multiple of 32): one 512-thread workgroup per
// 256 (tokens) x 256 (ranks) output tile, eight waves of 128 x 64 (4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16).  32-column slices of the contraction (one layer's
// columns of the X rows, the same columns of VrT) go from memory straight into LDS
// with direct-to-LDS loads, three slices ahead of the math, in a ring of four stages
// of 32 blocks (16 rows x 32 columns, 1 KiB each).  In a block, 16-byte unit u holds
// row u / 4 and column chunk (u % 4) ^ ((row / 2) % 4), so that the operand reads (one
// 16-byte read per lane: a row's 8 consecutive columns) of any 8 consecutive lanes
// touch distinct banks.
constexpr int QT = 256;            // output tile edge (tokens and ranks)
constexpr int QK = 32;             // contraction slice per stage
constexpr int QSTAGE = 32 * 1024;  // bytes per stage: 16 blocks of X rows, 16 of VrT rows

__global__ __launch_bounds__(512) void project_tile_kernel(ProjArgs a) {
  __shared__ __align__(16) unsigned char st0[QSTAGE], st1[QSTAGE], st2[QSTAGE], st3[QSTAGE];
  const int side = blockIdx.z;
  const int j0 = blockIdx.x * QT;    // rank tile (fastest: the tiles that share X rows run together)
  const int t0 = blockIdx.y * QT;    // token tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;   // wave tile: tokens wm*128.., ranks wn*64..
  const uint16_t* VrT = a.VrT + side * a.sVT;

  // Load role: wave w fills blocks 4w .. 4w+3 of a stage (0..15: X rows t0 + 16 b ..,
  // 16..31: VrT rows j0 + 16 (b - 16) ..); lane l loads row l / 4 of its block, column
  // chunk (l % 4) ^ ((l / 4 / 2) % 4).  Rows past T or r re-read the last row (never stored).
  const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lrow >> 1) & 3);
  long roff[4];
  bool is_x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bidx = 4 * wave + i;
    is_x[i] = bidx < 16;
    if (is_x[i]) roff[i] = (long)min(t0 + 16 * bidx + lrow, a.T - 1) * a.ld;
    else roff[i] = (long)min(j0 + 16 * (bidx - 16) + lrow, a.r - 1) * a.n;
  }
  auto dma = [&](int ks, unsigned char* stage) {
    const int k0 = ks * QK;
    const int l = k0 / a.d_kv;
    const uint16_t* xl = (const uint16_t*)a.layers.p[side * a.G + l] + (k0 - l * a.d_kv) + 8 * lchunk;
    const uint16_t* vr = VrT + k0 + 8 * lchunk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)((is_x[i] ? xl : vr) + roff[i]),
          (__attribute__((address_space(3))) void*)(stage + (4 * wave + i) * 1024), 16, 0, 0);
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

  // Operand of lane l for k-step ks: row l % 32 of a 32-row tile (block (l % 32) / 16,
  // row l % 16), column chunk 2 ks + l / 32.
  const int rb = lane & 15;
  int off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    off[ks] = ((lane >> 4) & 1) * 1024 + (rb * 4 + ((2 * ks + (lane >> 5)) ^ ((rb >> 1) & 3))) * 16;
  auto compute = [&](const unsigned char* stage) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = as_bf16x8(*(const uint4*)(stage + (8 * wm + 2 * mi) * 1024 + off[ks]));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = as_bf16x8(*(const uint4*)(stage + (16 + 4 * wn + 2 * ni) * 1024 + off[ks]));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = a.n / QK;
  // Slice s: wait for its loads (vmcnt(8): this wave's loads of slices s+1, s+2 may still
  // be in flight), barrier (every wave's loads of s have landed and the reads of s - 1
  // are over), start slice s + 3 into the stage of s - 1, then the math.  Past the last
  // slice the last one is loaded again so that the count of loads never varies.
  auto body = [&](int s, unsigned char* cur, unsigned char* ahead) {
    __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    dma(min(s + 3, nk - 1), ahead);
    if (s < nk) compute(cur);
  };
  dma(0, st0);
  dma(min(1, nk - 1), st1);
  dma(min(2, nk - 1), st2);
  for (int s = 0; s < nk; s += 4) {
    body(s, st0, st3);
    body(s + 1, st1, st0);
    body(s + 2, st2, st1);
    body(s + 3, st3, st2);
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the workgroup

  uint16_t* Aout = (uint16_t*)a.A_out.p[side];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + wm * 128 + mi * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
        const int c = j0 + wn * 64 + ni * 32 + (lane & 31);
        if (t < a.T && c < a.r) Aout[(long)t * a.r + c] = f32_to_bf16_bits(acc[mi][ni][j]);
      }
}

struct ProjF32Args {
  PtrTable layers;
  PtrTable A_out;
  const float* VrT;
  long sVT;
  int G, T, d_kv, n, r;
  long ld;
};

// float32 path (small workloads): 16 x 16 tiles, float64 sums.
__global__ __launch_bounds__(256) void project_f32_kernel(ProjF32Args a) {
  __shared__ float xt[16][17], vt[16][17];
  const int side = blockIdx.z;
  const int t0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  const float* VrT = a.VrT + side * a.sVT;
  double s = 0.0;
  for (int k0 = 0; k0 < a.n; k0 += 16) {
    const int col = k0 + tx;
    const int t = t0 + ty;
    float xv = 0.f;
    if (col < a.n && t < a.T) {
      const int l = col / a.d_kv;
      xv = ((const float*)a.layers.p[side * a.G + l])[(long)t * a.ld + (col - l * a.d_kv)];
    }
    xt[ty][tx] = xv;
    const int j = j0 + ty;
    vt[ty][tx] = (col < a.n && j < a.r) ? VrT[(long)j * a.n + col] : 0.f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) s += (double)xt[ty][k] * (double)vt[tx][k];
    __syncthreads();
  }
  const int t = t0 + ty, j = j0 + tx;
  if (t < a.T && j < a.r) ((float*)a.A_out.p[side])[(long)t * a.r + j] = (float)s;
}

struct LmArgs {
  PtrTable layers;
  PtrTable out;
  int G, T, H, d, chunk, n_chunks, bf16;
  long ld;
  long pos0;   // position of row 0 (0 for a prefix; the old length when rows are appended)
  double theta;
};

// One thread per (chunk, rotation pair); blockIdx.y = head, blockIdx.z = side * G + layer.
__global__ __launch_bounds__(256) void landmarks_kernel(LmArgs a) {
  const int half = a.d >> 1;
  const int per_block = 256 / half;
  const int c = blockIdx.x * per_block + threadIdx.x / half;
  const int i = threadIdx.x % half;
  const int h = blockIdx.y, sl = blockIdx.z;
  if (c >= a.n_chunks) return;
  const double f = rope_freq(a.theta, i, a.d);
  const long col = (long)h * a.d + i;
  float lo = 0.f, hi = 0.f;
  for (int q = 0; q < a.chunk; ++q) {
    const long t = (long)c * a.chunk + q;
    float xl, xh;
    if (a.bf16) {
      const uint16_t* src = (const uint16_t*)a.layers.p[sl] + t * a.ld + col;
      xl = bf16_bits_to_f32(src[0]);
      xh = bf16_bits_to_f32(src[half]);
    } else {
      const float* src = (const float*)a.layers.p[sl] + t * a.ld + col;
      xl = src[0];
      xh = src[half];
    }
    float cs, sn;
    rope_cs(a.pos0 + t, f, &cs, &sn);
    lo += xl * cs - xh * sn;
    hi += xh * cs + xl * sn;
  }
  const float inv = 1.f / (float)a.chunk;
  const long o = ((long)h * a.n_chunks + c) * a.d + i;
  if (a.bf16) {
    uint16_t* dst = (uint16_t*)a.out.p[sl];
    dst[o] = f32_to_bf16_bits(lo * inv);
    dst[o + half] = f32_to_bf16_bits(hi * inv);
  } else {
    float* dst = (float*)a.out.p[sl];
    dst[o] = lo * inv;
    dst[o + half] = hi * inv;
  }
}

// VrT (r x n) = Bt^T (Bt: n x r, row stride ldb), 32 x 32 tiles through LDS.
template <typename ST>
__global__ __launch_bounds__(256) void transpose_kernel(const ST* Bt, long ldb, int n, int r, ST* VrT) {
  __shared__ ST tile[32][33];
  const int i0 = blockIdx.x * 32, j0 = blockIdx.y * 32, tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8) {
    const int i = i0 + k, j = j0 + tx;
    if (i < n && j < r) tile[k][tx] = Bt[(long)i * ldb + j];
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int j = j0 + k, i = i0 + tx;
    if (i < n && j < r) VrT[(long)j * n + i] = tile[tx][k];
  }
}

}  // namespace

hipError_t launch_transpose_basis(const void* Bt, long ldb, int n, int r, void* VrT, int bf16, hipStream_t st) {
  const dim3 grid((n + 31) / 32, (r + 31) / 32);
  if (bf16)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)Bt, ldb, n, r,
                       (uint16_t*)VrT);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, st, (const float*)Bt, ldb, n, r, (float*)VrT);
  return hipGetLastError();
}

static constexpr size_t kProjLds = 2 * 2 * PT * PROW * sizeof(uint16_t);

hipError_t launch_project_bf16(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                               const uint16_t* VrT, long sVT, int r, const PtrTable& A_out,
                               hipStream_t st) {
  ProjArgs a;
  a.layers = layers;
  a.A_out = A_out;
  a.VrT = VrT;
  a.sVT = sVT;
  a.G = G;
  a.T = T;
  a.d_kv = d_kv;
  a.n = G * d_kv;
  a.r = r;
  a.ld = ld;
  if (d_kv % QK == 0) {
    dim3 grid((r + QT - 1) / QT, (T + QT - 1) / QT, n_sides);
    hipLaunchKernelGGL(project_tile_kernel, grid, dim3(512), 0, st, a);
    return hipGetLastError();
  }
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)project_bf16_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kProjLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((r + PT - 1) / PT, (T + PT - 1) / PT, n_sides);
  hipLaunchKernelGGL(project_bf16_kernel, grid, dim3(256), kProjLds, st, a);
  return hipGetLastError();
}

hipError_t launch_project_f32(const PtrTable& layers, int n_sides, int G, long ld, int T, int d_kv,
                              const float* VrT, long sVT, int r, const PtrTable& A_out,
                              hipStream_t st) {
  ProjF32Args a;
  a.layers = layers;
  a.A_out = A_out;
  a.VrT = VrT;
  a.sVT = sVT;
  a.G = G;
  a.T = T;
  a.d_kv = d_kv;
  a.n = G * d_kv;
  a.r = r;
  a.ld = ld;
  dim3 grid((r + 15) / 16, (T + 15) / 16, n_sides);
  hipLaunchKernelGGL(project_f32_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_landmarks(const PtrTable& layers, int n_sides, int G, long ld, int T, int n_kv_heads,
                            int head_dim, int chunk, double theta, const PtrTable& lm_out, int bf16,
                            hipStream_t st, long pos0) {
  LmArgs a;
  a.pos0 = pos0;
  a.layers = layers;
  a.out = lm_out;
  a.G = G;
  a.T = T;
  a.H = n_kv_heads;
  a.d = head_dim;
  a.chunk = chunk;
  a.n_chunks = T / chunk;
  a.bf16 = bf16;
  a.ld = ld;
  a.theta = theta;
  const int per_block = 256 / (head_dim / 2);
  dim3 grid((a.n_chunks + per_block - 1) / per_block, n_kv_heads, n_sides * G);
  hipLaunchKernelGGL(landmarks_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace xkv
