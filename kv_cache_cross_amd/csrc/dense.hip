// Dense decode baseline: attention of one query position over every cached position
// (full attention, the reference point the SR decode is measured against: xKV blog,
// section on figures 5-7, attention latency against full attention), and the RoPE
// helper that turns pre-RoPE keys into the post-RoPE keys a standard cache holds.
//
// dense_attend_kernel (grid: KV heads x splits x batch, 256 threads, bf16, head dim
// 128): a block takes 256 cached rows of its head.  The keys go to registers (thread t
// holds dims [32(t%4), 32(t%4)+32) of rows t/4 + 64i), the values to LDS with direct-
// to-LDS loads, all requested before the queries are rotated.  Scores are quad-reduced
// with DPP, the softmax partial covers the block's rows, and the weighted value sum
// leaves one (max, denominator, sum) partial per query head.
// dense_merge_kernel (grid: KV heads x batch) merges the partials by their
// log-sum-exp weights.
#include <hip/hip_runtime.h>
#include <algorithm>
#include "xkv_common.h"
#include "dense_params.h"

namespace xkv {
namespace {

constexpr int DRB = 256;   // cached rows per attend block
constexpr int DD = 128;    // head dim
constexpr int DG = 8;      // largest query group

XKV_DEV float dwave_sum(float v) {
#define XKV_DPPF(old, x, ctrl, rm, bc) \
  __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), ctrl, rm, 0xF, bc))
  v += XKV_DPPF(0.f, v, 0x111, 0xF, true);
  v += XKV_DPPF(0.f, v, 0x112, 0xF, true);
  v += XKV_DPPF(0.f, v, 0x114, 0xF, true);
  v += XKV_DPPF(0.f, v, 0x118, 0xF, true);
  v += XKV_DPPF(0.f, v, 0x142, 0xA, false);
  v += XKV_DPPF(0.f, v, 0x143, 0xC, false);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
XKV_DEV float dwave_max(float v) {
  v = fmaxf(v, XKV_DPPF(-INFINITY, v, 0x111, 0xF, false));
  v = fmaxf(v, XKV_DPPF(-INFINITY, v, 0x112, 0xF, false));
  v = fmaxf(v, XKV_DPPF(-INFINITY, v, 0x114, 0xF, false));
  v = fmaxf(v, XKV_DPPF(-INFINITY, v, 0x118, 0xF, false));
  v = fmaxf(v, XKV_DPPF(-INFINITY, v, 0x142, 0xA, false));
  v = fmaxf(v, XKV_DPPF(-INFINITY, v, 0x143, 0xC, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Sum over the four lanes of a quad (quad_perm [1,0,3,2] then [2,3,0,1]).
XKV_DEV float quad_sum(float v) {
  v += XKV_DPPF(0.f, v, 0xB1, 0xF, false);
  v += XKV_DPPF(0.f, v, 0x4E, 0xF, false);
  return v;
}
#undef XKV_DPPF

__global__ __launch_bounds__(256, 2) void dense_attend_kernel(DenseParams P) {
  extern __shared__ __align__(16) uint16_t vs[];   // staged value rows, DRB x DD (64 KiB)
  __shared__ __align__(16) float qs[DG][DD];
  __shared__ __align__(16) float pw[DG][DRB];
  __shared__ float st_m[DG], st_l[DG];
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = P.grp;
  const long r0 = (long)s * DRB;
  const long last = P.n_ctx - 1;
  const uint16_t* Kg = (const uint16_t*)P.K + b * P.bs_kv + (long)h * DD;
  const uint16_t* Vg = (const uint16_t*)P.V + b * P.bs_kv + (long)h * DD;

  // Keys: rows rsub + 64 i, dims [32 qq, 32 qq + 32) (rows past the context re-read the
  // last row and are masked).
  const int qq = tid & 3, rsub = tid >> 2;
  uint4 kr[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long row = std::min(r0 + rsub + 64 * i, last);
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[i][u] = *(const uint4*)(Kg + row * P.ld_kv + 32 * qq + 8 * u);
  }
  // Values: each wave instruction moves four 256-byte rows into LDS.
#pragma unroll
  for (int i = 0; i < DRB / 16; ++i) {
    const int rl = (wave * (DRB / 16) + i) * 4 + (lane >> 4);
    const long row = std::min(r0 + rl, last);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Vg + row * P.ld_kv + (lane & 15) * 8),
                                     (__attribute__((address_space(3))) void*)(vs + (wave * (DRB / 16) + i) * 4 * DD), 16, 0, 0);
  }
  // Rotated, scaled queries (two pairs per thread at most).
  {
    const uint16_t* qg = (const uint16_t*)P.q + ((long)b * P.Hq + (long)h * grp) * DD;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      if (e < grp * 64) {
        const int j = e >> 6, i = e & 63;
        const float x = bf16_bits_to_f32(qg[j * DD + i]), y = bf16_bits_to_f32(qg[j * DD + i + 64]);
        float c, sn;
        rope_cs_turns(P.q_pos, P.turns[i], &c, &sn);
        qs[j][i] = (x * c - y * sn) * P.scale;
        qs[j][i + 64] = (y * c + x * sn) * P.scale;
      }
    }
  }
  __syncthreads();
  // Scores: partial dot products over the thread's 32 dims, summed across the quad.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float kf[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {kr[i][u].x, kr[i][u].y, kr[i][u].z, kr[i][u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[8 * u + 2 * e] = __uint_as_float(w[e] << 16);
        kf[8 * u + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
    const int rl = rsub + 64 * i;
    const bool valid = r0 + rl <= last;
#pragma unroll
    for (int j = 0; j < DG; ++j) {
      if (j < grp) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 32; e += 4) {
          const float4 q4 = *(const float4*)&qs[j][32 * qq + e];
          acc += q4.x * kf[e] + q4.y * kf[e + 1] + q4.z * kf[e + 2] + q4.w * kf[e + 3];
        }
        acc = quad_sum(acc);
        if (qq == 0) pw[j][rl] = valid ? acc : -INFINITY;
      }
    }
  }
  __syncthreads();
  // Softmax partial of each query head over the block's rows (4 per lane).
  for (int j = wave; j < grp; j += 4) {
    float v[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = pw[j][lane + 64 * i];
      mx = fmaxf(mx, v[i]);
    }
    mx = dwave_max(mx);
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = (v[i] == -INFINITY) ? 0.f : __expf(v[i] - mx);
      pw[j][lane + 64 * i] = p;
      l += p;
    }
    l = dwave_sum(l);
    if (lane == 0) {
      st_m[j] = mx;
      st_l[j] = l;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the direct-to-LDS value loads have landed
  __syncthreads();
  // Weighted value sum: thread t takes dims 2(t%64), +1 over rows [64(t/64), 64(t/64)+64).
  const int c = 2 * lane, rg = wave;
  float o0[DG], o1[DG];
#pragma unroll
  for (int j = 0; j < DG; ++j) o0[j] = o1[j] = 0.f;
#pragma unroll 4
  for (int i4 = 0; i4 < 64; i4 += 4) {
    const int rr = rg * 64 + i4;
    float a0[4], a1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w = *(const uint32_t*)(vs + (rr + u) * DD + c);
      a0[u] = __uint_as_float(w << 16);
      a1[u] = __uint_as_float(w & 0xffff0000u);
    }
    // Every one of the DG weight rows is read (rows past grp hold unused values), so that
    // no LDS read waits behind a branch.
#pragma unroll
    for (int j = 0; j < DG; ++j) {
      const float4 p4 = *(const float4*)&pw[j][rr];
      o0[j] += p4.x * a0[0] + p4.y * a0[1] + p4.z * a0[2] + p4.w * a0[3];
      o1[j] += p4.x * a1[0] + p4.y * a1[1] + p4.z * a1[2] + p4.w * a1[3];
    }
  }
  __syncthreads();   // every wave is done with the staged values
  float* red = (float*)vs;   // [4 row groups][DG][DD]
#pragma unroll
  for (int j = 0; j < DG; ++j)
    if (j < grp) *(float2*)&red[(rg * DG + j) * DD + c] = make_float2(o0[j], o1[j]);
  __syncthreads();
  float* part = P.part + (((long)b * P.Hkv + h) * P.n_splits + s) * (long)grp * (2 + DD);
  for (int e = tid; e < grp * DD; e += 256) {
    const int j = e / DD, i = e % DD;
    part[2 * grp + e] = (red[(0 * DG + j) * DD + i] + red[(1 * DG + j) * DD + i]) +
                        (red[(2 * DG + j) * DD + i] + red[(3 * DG + j) * DD + i]);
  }
  if (tid < grp) {
    part[tid] = st_m[tid];
    part[grp + tid] = st_l[tid];
  }
}

// Merge of (b, h)'s split partials by their log-sum-exp weights into the output.
__global__ __launch_bounds__(256) void dense_merge_kernel(DenseParams P) {
  __shared__ float wq[DMAXP][DG];
  __shared__ float lq[DMAXP][DG];
  __shared__ float run_l[DG];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int grp = P.grp, np = P.n_splits;
  const long stride = (long)grp * (2 + DD);
  const float* p0 = P.part + ((long)b * P.Hkv + h) * np * stride;
  for (int idx = tid; idx < np * grp; idx += 256) {
    const int q = idx / grp, j = idx % grp;
    wq[q][j] = p0[q * stride + j];
    lq[q][j] = p0[q * stride + grp + j];
  }
  __syncthreads();
  if (tid < grp) {
    const int j = tid;
    float M = -INFINITY;
    for (int q = 0; q < np; ++q) M = fmaxf(M, wq[q][j]);
    float L = 0.f;
    for (int q = 0; q < np; ++q) {
      const float w = (wq[q][j] == -INFINITY) ? 0.f : __expf(wq[q][j] - M);
      wq[q][j] = w;
      L += w * lq[q][j];
    }
    run_l[j] = L;
  }
  __syncthreads();
  constexpr int NB = 16;
  for (int e = tid; e < grp * DD; e += 256) {
    const int j = e / DD;
    float acc = 0.f;
    for (int q0 = 0; q0 < np; q0 += NB) {
      float v[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) v[u] = p0[(long)min(q0 + u, np - 1) * stride + 2 * grp + e];
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (q0 + u < np) acc += wq[q0 + u][j] * v[u];
    }
    P.out[((long)b * P.Hq + (long)h * grp) * DD + e] = acc / run_l[j];
  }
}

// y[row] = RoPE(x[row], pos0 + row) for rows of n_heads x head_dim (rotate-half pairs
// (i, i + d/2), angle (pos0 + row) * freq[i] reduced in float64); one thread per pair.
template <typename ST>
__global__ void rope_rows_kernel(const ST* x, long ldx, ST* y, long ldy, int rows, long pos0, int n_heads,
                                 int d, double theta) {
  const int half = d >> 1;
  const long total = (long)rows * n_heads * half;
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    const int i = (int)(e % half);
    const long rh = e / half;
    const int hh = (int)(rh % n_heads);
    const long row = rh / n_heads;
    float c, s;
    rope_cs(pos0 + row, rope_freq(theta, i, d), &c, &s);
    const ST* xr = x + row * ldx + (long)hh * d;
    ST* yr = y + row * ldy + (long)hh * d;
    const float lo = ld_elem(xr + i), hi = ld_elem(xr + i + half);
    st_elem(yr + i, lo * c - hi * s);
    st_elem(yr + i + half, hi * c + lo * s);
  }
}

}  // namespace

hipError_t launch_dense_decode(const DenseParams& P, hipStream_t st) {
  const size_t lds = (size_t)DRB * DD * sizeof(uint16_t);
  static bool granted = false;
  if (!granted) {
    hipError_t e = hipFuncSetAttribute((const void*)dense_attend_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    granted = true;
  }
  hipLaunchKernelGGL(dense_attend_kernel, dim3(P.Hkv, P.n_splits, P.batch), dim3(256), lds, st, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dense_merge_kernel, dim3(P.Hkv, P.batch), dim3(256), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_rope_rows(const void* x, long ldx, void* y, long ldy, int rows, long pos0, int n_heads, int d,
                            double theta, int bf16, hipStream_t st) {
  const long total = (long)rows * n_heads * (d / 2);
  const int blocks = (int)std::min<long>(4096, (total + 255) / 256);
  if (blocks <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(rope_rows_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t*)x, ldx,
                       (uint16_t*)y, ldy, rows, pos0, n_heads, d, theta);
  else
    hipLaunchKernelGGL(rope_rows_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)x, ldx, (float*)y,
                       ldy, rows, pos0, n_heads, d, theta);
  return hipGetLastError();
}

}  // namespace xkv
