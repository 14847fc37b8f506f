// Selective Reconstruction decode for one layer and one step (xKV blog,
// section on Selective Reconstruction; decode attention as in KQ-SVD
// section 3.2).
//
// sr_select_kernel (grid: score blocks x KV heads x batch)
//   * block (0, 0, b) appends the new token's pre-RoPE k, v to the exact tail;
//   * every block forms the scaled, rotated query sum of its KV head's query
//     group and scores a slice of the candidate chunks against the landmarks
//     (a GEMV streaming the landmarks once);
//   * the last block of each (sequence, head) to finish, found with an atomic
//     counter, runs the top-k: an MSB-first radix select over order-preserving
//     keys, then an index-ordered compaction (ties go to the lower chunk id).
//
// sr_attend_kernel (grid: splits + 1 x KV heads x batch)
//   * split s < n_splits takes 64 rows: the selected chunks
//     [s*64/chunk, (s+1)*64/chunk) of its head, skipping rows that the exact
//     tail covers; it rebuilds k_t = A_k[t] B_k,l,h on the bf16 matrix cores
//     (A rows and Bt rows are both contiguous along r, read straight from
//     memory), rotates them, scores them against the group's queries and keeps
//     the softmax partial (max, denominator) and, for compressed values, the
//     weighted sum of A_v rows: sum_t p_t (a_t B) = (sum_t p_t a_t) B, so B_v
//     is applied once per query head after the merge instead of per row;
//   * split n_splits attends the exact rows (sink, local window, generated);
//   * the last block of each (sequence, head) merges the partials by their
//     log-sum-exp weights, applies B_v and writes the output.
#include "xkv_common.h"
#include "xkv_kernels.h"
#include "decode_params.h"

namespace xkv {
namespace {

constexpr int RB = 64;     // rows per attend split
constexpr int MAXG = 8;    // largest query group per KV head
constexpr int MAXD = 128;

XKV_DEV uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;   // -0.0 ranks equal to +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
XKV_DEV T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
XKV_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Inclusive prefix sum over the 256 threads of a block.
XKV_DEV int block_scan_incl(int v, int* tmp /* >= 4 ints */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += tmp[w];
  __syncthreads();
  return v + add;
}

// Ascending ids of the k largest of sc[0..n), ties to the lower id; -1 padding.
XKV_DEV void topk_block(const float* sc, int n, int k, int* out, int* hist, int* tmp, int* bcast) {
  const int tid = threadIdx.x;
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < k; i += 256) out[i] = (i < n) ? i : -1;
    return;
  }
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint32_t key = order_key(sc[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    const int v = hist[255 - tid];              // digits from the top
    const int incl = block_scan_incl(v, tmp);   // keys with digit >= 255 - tid
    const int excl = incl - v;                  // keys with digit >  255 - tid
    if (v > 0 && excl < remaining && remaining <= incl) {
      bcast[0] = 255 - tid;
      bcast[1] = remaining - excl;
    }
    __syncthreads();
    prefix |= (uint32_t)bcast[0] << shift;
    mask |= 0xffu << shift;
    remaining = bcast[1];
    __syncthreads();
  }
  // Keys above the threshold, then the first `remaining` equal keys in id order.
  const int seg = (n + 255) / 256;
  const int s0 = min(n, tid * seg), s1 = min(n, s0 + seg);
  int gt = 0, eq = 0;
  for (int i = s0; i < s1; ++i) {
    const uint32_t key = order_key(sc[i]);
    gt += key > prefix;
    eq += key == prefix;
  }
  const int eq_before = block_scan_incl(eq, tmp) - eq;
  const int take_eq = max(0, min(eq, remaining - eq_before));
  const int mine = gt + take_eq;
  int pos = block_scan_incl(mine, tmp) - mine;
  int seen = 0;
  for (int i = s0; i < s1; ++i) {
    const uint32_t key = order_key(sc[i]);
    if (key > prefix) {
      out[pos++] = i;
    } else if (key == prefix) {
      if (seen < take_eq) out[pos++] = i;
      ++seen;
    }
  }
}

template <typename ST>
XKV_DEV void load8(const ST* p, float* v);
template <>
XKV_DEV void load8<uint16_t>(const uint16_t* p, float* v) {
  const uint4 u = *(const uint4*)p;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
XKV_DEV void load8<float>(const float* p, float* v) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Rotated, scaled queries of KV head h's group into qs[j][0..d).
template <typename ST>
XKV_DEV void load_group_queries(const SrParams& P, int b, int h, float (*qs)[MAXD]) {
  const int half = P.d >> 1;
  const ST* q = (const ST*)P.q + ((long)b * P.Hq + (long)h * P.grp) * P.d;
  for (int e = threadIdx.x; e < P.grp * half; e += 256) {
    const int j = e / half, i = e % half;
    float c, s;
    rope_cs(P.q_pos, rope_freq(P.theta, i, P.d), &c, &s);
    const float x = ld_elem(q + j * P.d + i), y = ld_elem(q + j * P.d + i + half);
    qs[j][i] = (x * c - y * s) * P.scale;
    qs[j][i + half] = (y * c + x * s) * P.scale;
  }
}

template <typename ST>
__global__ __launch_bounds__(256) void sr_select_kernel(SrParams P) {
  __shared__ float qs[MAXG][MAXD];
  __shared__ float qsum[MAXD];
  __shared__ int hist[256];
  __shared__ int tmp[8];
  __shared__ int bcast[2];
  __shared__ int is_last;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;

  if (blk == 0 && h == 0 && P.k_new != nullptr && P.n_gen > 0) {
    const long row = P.n_sink + P.n_local + P.n_gen - 1;
    ST* kt = (ST*)P.k_tail + b * P.bs_tail + row * P.ld_tail;
    ST* vt = (ST*)P.v_tail + b * P.bs_tail + row * P.ld_tail;
    const ST* kn = (const ST*)P.k_new + b * P.bs_new;
    const ST* vn = (const ST*)P.v_new + b * P.bs_new;
    for (int i = tid; i < P.Hkv * P.d; i += 256) {
      kt[i] = kn[i];
      vt[i] = vn[i];
    }
  }

  load_group_queries<ST>(P, b, h, qs);
  __syncthreads();
  for (int i = tid; i < P.d; i += 256) {
    float s = 0.f;
    for (int j = 0; j < P.grp; ++j) s += qs[j][i];
    qsum[i] = s;
  }
  __syncthreads();

  const int per_blk = (P.n_cand + P.score_blocks - 1) / P.score_blocks;
  const int c0 = blk * per_blk, c1 = min(P.n_cand, c0 + per_blk);
  const int lpc = P.d >> 3;           // lanes per chunk, 8 elements each
  const int cpi = 256 / lpc;          // chunks per pass
  const int sub = tid % lpc, slot = tid / lpc;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qsum[sub * 8 + e];
  const ST* lm = (const ST*)P.lm + b * P.bs_lm + (long)h * P.n_chunks * P.d;
  float* scores = P.scores + ((long)b * P.Hkv + h) * P.n_cand;
  const int iters = (c1 - c0 + cpi - 1) / cpi;
  for (int it = 0; it < max(iters, 0); ++it) {
    const int c = c0 + it * cpi + slot;
    float dot = 0.f;
    if (c < c1) {
      float v[8];
      load8<ST>(lm + (long)c * P.d + sub * 8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += qv[e] * v[e];
    }
    for (int o = lpc >> 1; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    if (c < c1 && sub == 0) scores[c] = dot;
  }

  __threadfence();
  __syncthreads();
  int* counter = P.counters + ((long)b * P.Hkv + h) * 2;
  if (tid == 0) is_last = (atomicAdd(counter, 1) == P.score_blocks - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  topk_block(scores, P.n_cand, P.top_k, P.sel + ((long)b * P.Hkv + h) * P.top_k, hist, tmp, bcast);
  if (tid == 0) *counter = 0;
}

template <typename ST>
__global__ __launch_bounds__(256) void sr_attend_kernel(SrParams P) {
  __shared__ float qs[MAXG][MAXD];
  __shared__ float kh[RB][MAXD + 1];
  __shared__ float pw[MAXG][RB];
  __shared__ int rows_t[RB];
  __shared__ float st_m[MAXG], st_l[MAXG];
  __shared__ float run_m[MAXG], run_l[MAXG], run_a[MAXG], run_b[MAXG];
  __shared__ int is_last;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int d = P.d, half = d >> 1, grp = P.grp;
  const bool exact_split = (s == P.n_splits);
  const long bh = (long)b * P.Hkv + h;

  load_group_queries<ST>(P, b, h, qs);

  if (!exact_split) {
    // ---- rows of this split ----
    if (tid < RB) {
      const int ci = s * P.cps + tid / P.chunk;
      const int c = (ci < P.k_eff) ? P.sel[bh * P.top_k + ci] : -1;
      const int t = c * P.chunk + tid % P.chunk;
      rows_t[tid] = (c >= 0 && t >= P.n_sink && t < P.T - P.n_local) ? t : -1;
    }
    __syncthreads();

    // ---- rebuild keys of the rows, then RoPE ----
    const ST* A = (const ST*)P.A_k + b * P.bs_A_k;
    const ST* Bt = (const ST*)P.Bt_k + b * P.bs_Bt_k + (long)h * d * P.ld_Bt_k;
    bool done = false;
    if constexpr (sizeof(ST) == 2) {
      if (d == 128 && (P.r_k & 63) == 0) {
        const int rh = wave >> 1, cp = wave & 1;
        const int row_l = rh * 32 + (lane & 31);
        const int t_row = rows_t[row_l];
        const uint16_t* arow = (const uint16_t*)A + (long)(t_row >= 0 ? t_row : 0) * P.ld_A_k;
        const uint16_t* b0 = (const uint16_t*)Bt + (long)(cp * 32 + (lane & 31)) * P.ld_Bt_k;
        const uint16_t* b1 = b0 + 64L * P.ld_Bt_k;
        f32x16_t acc0, acc1;
#pragma unroll
        for (int j = 0; j < 16; ++j) { acc0[j] = 0.f; acc1[j] = 0.f; }
        for (int k0 = 0; k0 < P.r_k; k0 += 64) {
          const int kb = k0 + (lane >> 5) * 32;
          uint4 av[4], bv0[4], bv1[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            av[i] = *(const uint4*)(arow + kb + 8 * i);
            bv0[i] = *(const uint4*)(b0 + kb + 8 * i);
            bv1[i] = *(const uint4*)(b1 + kb + 8 * i);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[i]), as_bf16x8(bv0[i]), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[i]), as_bf16x8(bv1[i]), acc1, 0, 0, 0);
          }
        }
        const int i = cp * 32 + (lane & 31);
        const double f = rope_freq(P.theta, i, 128);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = rh * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
          const int t = rows_t[row];
          float c = 1.f, sn = 0.f;
          if (t >= 0) rope_cs(t, f, &c, &sn);
          const float lo = acc0[j], hi = acc1[j];
          kh[row][i] = lo * c - hi * sn;
          kh[row][i + 64] = hi * c + lo * sn;
        }
        done = true;
      }
    }
    if (!done) {
      for (int e = tid; e < RB * half; e += 256) {
        const int row = e / half, i = e % half;
        const int t = rows_t[row];
        float lo = 0.f, hi = 0.f;
        if (t >= 0) {
          const ST* ar = A + (long)t * P.ld_A_k;
          const ST* bl = Bt + (long)i * P.ld_Bt_k;
          const ST* bh2 = Bt + (long)(i + half) * P.ld_Bt_k;
          for (int k = 0; k < P.r_k; ++k) {
            const float a = ld_elem(ar + k);
            lo += a * ld_elem(bl + k);
            hi += a * ld_elem(bh2 + k);
          }
        }
        float c = 1.f, sn = 0.f;
        if (t >= 0) rope_cs(t, rope_freq(P.theta, i, d), &c, &sn);
        kh[row][i] = lo * c - hi * sn;
        kh[row][i + half] = hi * c + lo * sn;
      }
    }
    __syncthreads();

    // ---- scores and softmax partials ----
    for (int e = tid; e < grp * RB; e += 256) {
      const int j = e / RB, row = e % RB;
      float v = -INFINITY;
      if (rows_t[row] >= 0) {
        v = 0.f;
        for (int i = 0; i < d; ++i) v += qs[j][i] * kh[row][i];
      }
      pw[j][row] = v;
    }
    __syncthreads();
    for (int j = wave; j < grp; j += 4) {
      const float v = pw[j][lane];
      const float mx = wave_max(v);
      const float p = (v == -INFINITY) ? 0.f : __expf(v - mx);
      const float l = wave_sum(p);
      pw[j][lane] = p;
      if (lane == 0) { st_m[j] = mx; st_l[j] = l; }
    }
    __syncthreads();

    // ---- value partial ----
    const int R = P.vec_len;
    float* part = P.part + (bh * P.n_splits + s) * (long)grp * (2 + R);
    if (tid < grp) { part[tid] = st_m[tid]; part[grp + tid] = st_l[tid]; }
    float* vec = part + 2 * grp;
    if (P.r_v > 0) {
      const ST* Av = (const ST*)P.A_v + b * P.bs_A_v;
      for (int kp = tid; kp < (P.r_v >> 1); kp += 256) {
        float acc[MAXG][2];
#pragma unroll
        for (int j = 0; j < MAXG; ++j) { acc[j][0] = 0.f; acc[j][1] = 0.f; }
        for (int row = 0; row < RB; ++row) {
          const int t = rows_t[row];
          if (t < 0) continue;
          const ST* ap = Av + (long)t * P.ld_A_v + 2 * kp;
          const float a0 = ld_elem(ap), a1 = ld_elem(ap + 1);
#pragma unroll
          for (int j = 0; j < MAXG; ++j) {
            if (j < grp) {
              const float p = pw[j][row];
              acc[j][0] += p * a0;
              acc[j][1] += p * a1;
            }
          }
        }
#pragma unroll
        for (int j = 0; j < MAXG; ++j)
          if (j < grp) { vec[j * R + 2 * kp] = acc[j][0]; vec[j * R + 2 * kp + 1] = acc[j][1]; }
      }
    } else {
      const ST* V = (const ST*)P.V_full + b * P.bs_V + (long)h * d;
      for (int e = tid; e < grp * d; e += 256) {
        const int j = e / d, i = e % d;
        float acc = 0.f;
        for (int row = 0; row < RB; ++row) {
          const int t = rows_t[row];
          if (t >= 0) acc += pw[j][row] * ld_elem(V + (long)t * P.ld_V + i);
        }
        vec[j * R + i] = acc;
      }
    }
  } else {
    // ---- exact rows: sink, local window, generated ----
    const int n_tail = P.n_sink + P.n_local + P.n_gen;
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = 0.f;
    if (tid < MAXG) { run_m[tid] = -INFINITY; run_l[tid] = 0.f; }
    const ST* kt = (const ST*)P.k_tail + b * P.bs_tail + (long)h * d;
    const ST* vt = (const ST*)P.v_tail + b * P.bs_tail + (long)h * d;
    for (int r0 = 0; r0 < n_tail; r0 += RB) {
      __syncthreads();
      if (tid < RB) {
        const int row = r0 + tid;
        int pos = -1;
        if (row < P.n_sink) pos = row;
        else if (row < P.n_sink + P.n_local) pos = P.T - P.n_local + (row - P.n_sink);
        else if (row < n_tail) pos = P.T + (row - P.n_sink - P.n_local);
        rows_t[tid] = pos;
      }
      __syncthreads();
      for (int e = tid; e < RB * half; e += 256) {
        const int rl = e / half, i = e % half;
        const int pos = rows_t[rl];
        float lo = 0.f, hi = 0.f, c = 1.f, sn = 0.f;
        if (pos >= 0) {
          const ST* kr = kt + (long)(r0 + rl) * P.ld_tail;
          lo = ld_elem(kr + i);
          hi = ld_elem(kr + i + half);
          rope_cs(pos, rope_freq(P.theta, i, d), &c, &sn);
        }
        kh[rl][i] = lo * c - hi * sn;
        kh[rl][i + half] = hi * c + lo * sn;
      }
      __syncthreads();
      for (int e = tid; e < grp * RB; e += 256) {
        const int j = e / RB, rl = e % RB;
        float v = -INFINITY;
        if (rows_t[rl] >= 0) {
          v = 0.f;
          for (int i = 0; i < d; ++i) v += qs[j][i] * kh[rl][i];
        }
        pw[j][rl] = v;
      }
      __syncthreads();
      for (int j = wave; j < grp; j += 4) {
        const float v = pw[j][lane];
        const float mt = wave_max(v);
        const float mnew = fmaxf(run_m[j], mt);
        const float p = (v == -INFINITY) ? 0.f : __expf(v - mnew);
        const float lt = wave_sum(p);
        pw[j][lane] = p;
        if (lane == 0) {
          const float alpha = (run_m[j] == -INFINITY) ? 0.f : __expf(run_m[j] - mnew);
          run_a[j] = alpha;
          run_l[j] = run_l[j] * alpha + lt;
          run_m[j] = mnew;
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = tid + 256 * q;
        if (e < grp * d) {
          const int j = e / d, i = e % d;
          float acc = o[q] * run_a[j];
          for (int rl = 0; rl < RB; ++rl)
            if (rows_t[rl] >= 0) acc += pw[j][rl] * ld_elem(vt + (long)(r0 + rl) * P.ld_tail + i);
          o[q] = acc;
        }
      }
    }
    __syncthreads();
    float* part = P.part_ex + bh * (long)grp * (2 + d);
    if (tid < grp) { part[tid] = run_m[tid]; part[grp + tid] = run_l[tid]; }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      if (e < grp * d) part[2 * grp + e] = o[q];
    }
  }

  // ---- the last block of (b, h) merges ----
  __threadfence();
  __syncthreads();
  int* counter = P.counters + bh * 2 + 1;
  if (tid == 0) is_last = (atomicAdd(counter, 1) == P.n_splits);
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  const int R = P.vec_len;
  const float* pex = P.part_ex + bh * (long)grp * (2 + d);
  if (tid < grp) {
    const int j = tid;
    float M = pex[j];
    for (int q = 0; q < P.n_splits; ++q) M = fmaxf(M, P.part[(bh * P.n_splits + q) * (long)grp * (2 + R) + j]);
    float L = (pex[j] == -INFINITY) ? 0.f : pex[grp + j] * __expf(pex[j] - M);
    for (int q = 0; q < P.n_splits; ++q) {
      const float* pq = P.part + (bh * P.n_splits + q) * (long)grp * (2 + R);
      if (pq[j] != -INFINITY) L += pq[grp + j] * __expf(pq[j] - M);
    }
    run_m[j] = M;
    run_l[j] = L;
  }
  __syncthreads();
  // Weighted sum of the split vectors into LDS (reusing kh as scratch: grp x R floats).
  float* vsum = &kh[0][0];
  for (int e = tid; e < grp * R; e += 256) {
    const int j = e / R;
    float acc = 0.f;
    for (int q = 0; q < P.n_splits; ++q) {
      const float* pq = P.part + (bh * P.n_splits + q) * (long)grp * (2 + R);
      if (pq[j] != -INFINITY) acc += __expf(pq[j] - run_m[j]) * pq[2 * grp + e];
    }
    vsum[e] = acc;
  }
  __syncthreads();
  const ST* Btv = (P.r_v > 0) ? (const ST*)P.Bt_v + b * P.bs_Bt_v + (long)h * d * P.ld_Bt_v : nullptr;
  for (int e = tid; e < grp * d; e += 256) {
    const int j = e / d, i = e % d;
    float acc = 0.f;
    if (P.r_v > 0) {
      const ST* brow = Btv + (long)i * P.ld_Bt_v;
      const float* vj = vsum + j * R;
      for (int k = 0; k < P.r_v; ++k) acc += vj[k] * ld_elem(brow + k);
    } else {
      acc = vsum[j * R + i];
    }
    if (pex[j] != -INFINITY) acc += __expf(pex[j] - run_m[j]) * pex[2 * grp + e];
    P.out[((long)b * P.Hq + (long)h * grp + j) * d + i] = acc / run_l[j];
  }
  if (tid == 0) *counter = 0;
}

__global__ __launch_bounds__(256) void topk_rows_kernel(const float* scores, int n_cand, long ld, int k, int* sel) {
  __shared__ int hist[256];
  __shared__ int tmp[8];
  __shared__ int bcast[2];
  topk_block(scores + blockIdx.x * ld, n_cand, k, sel + (long)blockIdx.x * k, hist, tmp, bcast);
}

}  // namespace

hipError_t launch_sr_select(const SrParams& P, int bf16, hipStream_t st) {
  dim3 grid(P.score_blocks, P.Hkv, P.batch);
  if (bf16) hipLaunchKernelGGL(sr_select_kernel<uint16_t>, grid, dim3(256), 0, st, P);
  else hipLaunchKernelGGL(sr_select_kernel<float>, grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_sr_attend(const SrParams& P, int bf16, hipStream_t st) {
  dim3 grid(P.n_splits + 1, P.Hkv, P.batch);
  if (bf16) hipLaunchKernelGGL(sr_attend_kernel<uint16_t>, grid, dim3(256), 0, st, P);
  else hipLaunchKernelGGL(sr_attend_kernel<float>, grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int rows, int n_cand, long ld, int k, int* sel, hipStream_t st) {
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(256), 0, st, scores, n_cand, ld, k, sel);
  return hipGetLastError();
}

}  // namespace xkv
