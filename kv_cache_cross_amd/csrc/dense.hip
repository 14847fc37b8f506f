// Dense decode baseline: attention of one query position over every cached position
// (full attention, the reference point the SR decode is measured against: xKV blog,
// section on figures 5-7, attention latency against full attention), and the RoPE
// helper that turns pre-RoPE keys into the post-RoPE keys a standard cache holds.
//
// dense_attend_kernel<G> (grid: KV heads x splits x batch, 256 threads, bf16, head dim
// 128, G query heads per KV head): a block takes rows_per_block cached rows of its
// head and each of its four waves streams a quarter of them in 32-row tiles, with the
// next tile's keys and values in flight while the current one is used.
//   * scores: S^T (16 rows x 16 query slots) = K_tile Q^T on v_mfma_f32_16x16x32_bf16,
//     the keys loaded straight into the A-operand layout (lane l: row l % 16, dims
//     32 kk + 8 (l / 16) .. + 7), the rotated, scaled queries held as the B operand in
//     two bf16 parts (high and remainder), so the query keeps about 16 bits;
//   * an online softmax per wave (running max and denominator per query head);
//   * the weighted value sum on the vector ALUs, lane l owning dims 8 (l % 16) .. + 7
//     of a quarter of the tile's rows, the tile's weights passed through a per-wave
//     LDS slot;
//   * the four waves' states are combined once, into one (max, denominator, sum)
//     partial per query head.
// dense_merge_kernel (grid: query heads x batch) merges the partials of one query
// head by their log-sum-exp weights.
#include <hip/hip_runtime.h>
#include <algorithm>
#include "xkv_common.h"
#include "dense_params.h"

namespace xkv {
namespace {

constexpr int DD = 128;    // head dim
constexpr int DG = 8;      // largest query group
constexpr int PWS = 36;    // LDS row of one query head's tile weights: 32 rows, alpha, pad

XKV_DEV float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
XKV_DEV float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

// One tile's loads: keys of two 16-row MFMA tiles (A-operand layout) and the values of
// 32 rows, 16 bytes per lane (lane l: dims 8 (l % 16) .. + 7 of rows 8 (l / 16) + i),
// 16 instructions of 1 KiB per tile.  Rows past the context re-read the last row and
// are masked by the caller.
struct DenseTile {
  uint4 k[2][4];
  uint4 v[8];
  // Kb, Vb: the block's (sequence, head) base; byte offsets fit 32 bits (checked on the
  // host) and are added to the 64-bit base.
  XKV_DEV void load(const char* Kb, const char* Vb, uint32_t ld_bytes, int row0, int last, int lane) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int row = min(row0 + 16 * st + (lane & 15), last);
      const uint32_t off = (uint32_t)row * ld_bytes + 16u * (uint32_t)(lane >> 4);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) k[st][kk] = *(const uint4*)(Kb + (off + 64u * kk));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(row0 + 8 * (lane >> 4) + i, last);
      v[i] = *(const uint4*)(Vb + ((uint32_t)row * ld_bytes + 16u * (uint32_t)(lane & 15)));
    }
  }
};

template <int G>
__global__ __launch_bounds__(256, 2) void dense_attend_kernel(DenseParams P) {
  __shared__ __align__(16) float pw[4][DG][PWS];
  __shared__ __align__(16) float wo[4][G][DD];
  __shared__ float wm[4][DG], wl[4][DG];
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, j = lane & 15;       // score layout: rows 4 g4 + v, query slot j
  const int last = (int)P.n_ctx - 1;
  const int rpw = P.rows_per_block >> 2;
  const int w0 = s * P.rows_per_block + wave * rpw;
  const int ntile = rpw >> 5;
  const uint32_t ldb = (uint32_t)P.ld_kv * 2u;
  const char* Kg = (const char*)((const uint16_t*)P.K + b * P.bs_kv + (long)h * DD);
  const char* Vg = (const char*)((const uint16_t*)P.V + b * P.bs_kv + (long)h * DD);

  // Tile t covers rows w0 + 32 t ..; every load is unconditional: past the wave's last
  // tile the prefetch re-reads that tile (a cache hit), so no wait depends on a branch.
  DenseTile ta, tb;
  ta.load(Kg, Vg, ldb, w0, last, lane);

  // B operand: query slot j's rotated, scaled query, dims 32 kk + 8 g4 + e, split into
  // a bf16 high part and a bf16 remainder (q = hi + lo to about 16 significant bits),
  // both multiplied in: the scores keep near-float32 accuracy in the query.
  // RoPE pairs (i, i + 64) sit in slices kk and kk + 2 of the same lane.
  bf16x8_t qb[4], ql[4];
  {
    float qf[4][8];
    const uint16_t* qg = (const uint16_t*)P.q + ((long)b * P.Hq + (long)h * G + std::min(j, G - 1)) * DD;
    uint4 qr[4];   // unconditional 16-byte loads (slots past the group re-read the last head)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qr[kk] = *(const uint4*)(qg + 32 * kk + 8 * g4);
    const float keep = (j < G) ? 1.f : 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t w[4] = {qr[kk].x, qr[kk].y, qr[kk].z, qr[kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[kk][2 * e] = keep * __uint_as_float(w[e] << 16);
        qf[kk][2 * e + 1] = keep * __uint_as_float(w[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float c, sn;
        rope_cs_turns(P.q_pos, P.turns[32 * kk + 8 * g4 + e], &c, &sn);
        const float x = qf[kk][e], y = qf[kk + 2][e];
        qf[kk][e] = (x * c - y * sn) * P.scale;
        qf[kk + 2][e] = (y * c + x * sn) * P.scale;
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = f32_to_bf16_bits(qf[kk][e]);
        lo[e] = f32_to_bf16_bits(qf[kk][e] - __uint_as_float(hi[e] << 16));
      }
      qb[kk] = as_bf16x8(make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
                                    hi[6] | (hi[7] << 16)));
      ql[kk] = as_bf16x8(make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
                                    lo[6] | (lo[7] << 16)));
    }
  }

  float m_run = -INFINITY, l_run = 0.f;   // query slot j (the same in the four lane groups)
  float o[G][8];                          // query head jj, dims 8 (lane % 16) + e, rows of group g4
#pragma unroll
  for (int jj = 0; jj < G; ++jj)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[jj][e] = 0.f;
  float* my_pw = &pw[wave][0][0];

  auto process = [&](const DenseTile& cur, int row0) {
    f32x4_t sc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sc[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.k[st][kk]), qb[kk], sc[st], 0, 0, 0);
        sc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.k[st][kk]), ql[kk], sc[st], 0, 0, 0);
      }
    }
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool valid = row0 + 16 * st + 4 * g4 + v <= last;
        sv[4 * st + v] = valid ? sc[st][v] : -INFINITY;
        tmax = fmaxf(tmax, sv[4 * st + v]);
      }
    tmax = xor_max(xor_max(tmax, 16), 32);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sv[i] = (sv[i] == -INFINITY) ? 0.f : __expf(sv[i] - m_new);
      psum += sv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    __builtin_amdgcn_wave_barrier();
    if (j < G) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
        *(float4*)&my_pw[j * PWS + 16 * st + 4 * g4] = make_float4(sv[4 * st], sv[4 * st + 1], sv[4 * st + 2], sv[4 * st + 3]);
      if (g4 == 0) my_pw[j * PWS + 32] = alpha;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const float a = my_pw[jj * PWS + 32];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[jj][e] *= a;
    }
#pragma unroll
    for (int i0 = 0; i0 < 8; i0 += 4) {
      float vf[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w[4] = {cur.v[i0 + u].x, cur.v[i0 + u].y, cur.v[i0 + u].z, cur.v[i0 + u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[u][2 * e] = __uint_as_float(w[e] << 16);
          vf[u][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const float4 p4 = *(const float4*)&my_pw[jj * PWS + 8 * g4 + i0];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[jj][e] = fmaf(p4.w, vf[3][e], fmaf(p4.z, vf[2][e], fmaf(p4.y, vf[1][e], fmaf(p4.x, vf[0][e], o[jj][e]))));
      }
    }
  };
  for (int t = 0; t < ntile; t += 2) {
    tb.load(Kg, Vg, ldb, w0 + 32 * min(t + 1, ntile - 1), last, lane);
    process(ta, w0 + 32 * t);
    ta.load(Kg, Vg, ldb, w0 + 32 * min(t + 2, ntile - 1), last, lane);
    if (t + 1 < ntile) process(tb, w0 + 32 * (t + 1));
  }

  // Combine the four waves.
  l_run = xor_sum(xor_sum(l_run, 16), 32);
  if (j < G && g4 == 0) {
    wm[wave][j] = m_run;
    wl[wave][j] = l_run;
  }
  // Sum the four lane groups' rows; lanes 0-15 then hold the wave's sums.
#pragma unroll
  for (int jj = 0; jj < G; ++jj)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[jj][e] = xor_sum(xor_sum(o[jj][e], 16), 32);
  if (g4 == 0) {
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      *(float4*)&wo[wave][jj][8 * j] = make_float4(o[jj][0], o[jj][1], o[jj][2], o[jj][3]);
      *(float4*)&wo[wave][jj][8 * j + 4] = make_float4(o[jj][4], o[jj][5], o[jj][6], o[jj][7]);
    }
  }
  __syncthreads();
  float* part = P.part + (((long)b * P.Hkv + h) * P.n_splits + s) * (long)G * (2 + DD);
  for (int e = tid; e < G * DD; e += 256) {
    const int jj = e / DD, i = e % DD;
    const float M = fmaxf(fmaxf(wm[0][jj], wm[1][jj]), fmaxf(wm[2][jj], wm[3][jj]));
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (wm[w][jj] != -INFINITY) acc += __expf(wm[w][jj] - M) * wo[w][jj][i];
    part[2 * G + e] = acc;
  }
  if (tid < G) {
    const float M = fmaxf(fmaxf(wm[0][tid], wm[1][tid]), fmaxf(wm[2][tid], wm[3][tid]));
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (wm[w][tid] != -INFINITY) L += __expf(wm[w][tid] - M) * wl[w][tid];
    part[tid] = M;
    part[G + tid] = L;
  }
}

// Merge of one query head's split partials by their log-sum-exp weights.  Phase 1
// forms the weights exp(m_s - M) and the denominator; phase 2 sums the weighted
// partial outputs, eight groups of splits over 32 lanes of float4 dims each.
__global__ __launch_bounds__(256) void dense_merge_kernel(DenseParams P) {
  __shared__ float wq[DMAXP];
  __shared__ float red_m[4], red_l[4];
  __shared__ __align__(16) float4 acc_s[8][32];
  const int qh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = P.grp, h = qh / grp, j = qh % grp, np = P.n_splits;
  const long stride = (long)grp * (2 + DD);
  const float* p0 = P.part + ((long)b * P.Hkv + h) * np * stride;
  float m[2], l[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = tid + 256 * u;
    m[u] = (q < np) ? p0[q * stride + j] : -INFINITY;
    l[u] = (q < np) ? p0[q * stride + grp + j] : 0.f;
  }
  float mx = fmaxf(m[0], m[1]);
  for (int o = 32; o > 0; o >>= 1) mx = xor_max(mx, o);
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  float ls = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = tid + 256 * u;
    const float w = (m[u] == -INFINITY) ? 0.f : __expf(m[u] - M);
    if (q < np) wq[q] = w;
    ls += w * l[u];
  }
  for (int o = 32; o > 0; o >>= 1) ls = xor_sum(ls, o);
  if (lane == 0) red_l[wave] = ls;
  __syncthreads();
  const float L = (red_l[0] + red_l[1]) + (red_l[2] + red_l[3]);
  const int c4 = tid & 31, sg = tid >> 5;
  const float* ob = p0 + 2 * grp + (long)j * DD + 4 * c4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int NB = 8;
  for (int q0 = sg; q0 < np; q0 += 8 * NB) {
    float4 v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = *(const float4*)(ob + (long)std::min(q0 + 8 * u, np - 1) * stride);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (q0 + 8 * u < np) {
        const float w = wq[q0 + 8 * u];
        acc.x += w * v[u].x;
        acc.y += w * v[u].y;
        acc.z += w * v[u].z;
        acc.w += w * v[u].w;
      }
  }
  acc_s[sg][c4] = acc;
  __syncthreads();
  if (tid < 32) {
    float4 r = acc_s[0][tid];
#pragma unroll
    for (int g = 1; g < 8; ++g) {
      r.x += acc_s[g][tid].x;
      r.y += acc_s[g][tid].y;
      r.z += acc_s[g][tid].z;
      r.w += acc_s[g][tid].w;
    }
    const float inv = 1.f / L;
    *(float4*)(P.out + ((long)b * P.Hq + qh) * DD + 4 * tid) = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
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

template <int G>
hipError_t launch_attend_g(const DenseParams& P, hipStream_t st) {
  hipLaunchKernelGGL(dense_attend_kernel<G>, dim3(P.Hkv, P.n_splits, P.batch), dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_decode(const DenseParams& P, hipStream_t st) {
  hipError_t e;
  switch (P.grp) {
    case 1: e = launch_attend_g<1>(P, st); break;
    case 2: e = launch_attend_g<2>(P, st); break;
    case 3: e = launch_attend_g<3>(P, st); break;
    case 4: e = launch_attend_g<4>(P, st); break;
    case 5: e = launch_attend_g<5>(P, st); break;
    case 6: e = launch_attend_g<6>(P, st); break;
    case 7: e = launch_attend_g<7>(P, st); break;
    case 8: e = launch_attend_g<8>(P, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dense_merge_kernel, dim3(P.Hq, P.batch), dim3(256), 0, st, P);
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
