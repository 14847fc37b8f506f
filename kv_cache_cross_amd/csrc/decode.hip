// Selective Reconstruction decode for one layer and one step (xKV blog,
// section on Selective Reconstruction; decode attention as in KQ-SVD
// section 3.2).  Four kernels, ordered by the stream (no device-scope fences
// inside any of them: on this GPU such a fence writes back the XCD's L2):
//
// sr_score_kernel (grid: score_blocks + 1 x KV heads x batch)
//   * block (0, 0, b) appends the new token's pre-RoPE k, v to the exact tail;
//   * blocks x < score_blocks form the scaled, rotated query sum of the KV
//     head's query group and score a slice of the candidate chunks against the
//     landmarks (a GEMV that streams the landmarks once, each thread's loads
//     issued before its arithmetic);
//   * block x == score_blocks attends the exact rows (sink, local window,
//     generated tokens), which do not depend on the selection, and leaves a
//     softmax partial (max, denominator, weighted value sum) per query head.
// sr_topk_kernel (grid: KV heads x batch): the head's scores go to LDS as
//   order-preserving keys; an MSB-first radix select finds the k-th key and an
//   index-ordered compaction writes the k chunk ids (ties to the lower id).
// sr_attend_mfma_kernel (bf16, head_dim 128, r % 64 == 0; grid: KV heads x
// splits x batch, so one head's blocks share an XCD and its B slices in L2)
//   * a block takes 64 rows: the selected chunks [s*64/chunk, (s+1)*64/chunk)
//     of its head, minus rows the exact tail covers;
//   * the gathered rows of A_k and A_v are staged into LDS with every load in
//     flight at once (16 bytes per lane, a wave per row);
//   * waves 0-1 rebuild k_t = A_k[t] B_k,l,h and waves 2-3 v_t = A_v[t] B_v,l,h
//     on v_mfma_f32_32x32x16_bf16; B rows are contiguous along r and stream
//     from L2 two k-steps ahead of the MFMAs; the key waves apply RoPE;
//   * scores, a softmax partial and the partial output sum_t p_t v_t per query
//     head.
// sr_attend_generic_kernel covers every other shape (float32, other head
// dims, exact values) with the same partials.
// sr_merge_kernel (grid: KV heads x batch) merges the split partials and the
//   exact-row partial by their log-sum-exp weights into the output.
#include "xkv_common.h"
#include "xkv_kernels.h"
#include "decode_params.h"

namespace xkv {
namespace {

constexpr int RB = 64;        // rows per attend block
constexpr int MAXG = 8;       // largest query group per KV head
constexpr int MAXD = 128;     // largest head dim
constexpr int KCH = 512;      // rank columns staged per pass (MFMA path)
constexpr int AROW = KCH + 8; // padded LDS row of staged A rows (bf16 elements)
constexpr int HROW = MAXD + 1;
constexpr int MAXP = 129;     // splits + 1 that the merge supports

XKV_DEV uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;   // -0.0 ranks equal to +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

XKV_DEV float wave_sum(float v) {
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

XKV_DEV uint32_t block_reduce_minmax(uint32_t v, bool is_max, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t u = __shfl_xor(v, o);
    v = is_max ? max(v, u) : min(v, u);
  }
  if (lane == 0) tmp[wave] = v;
  __syncthreads();
  uint32_t r = tmp[0];
  for (int w = 1; w < 4; ++w) r = is_max ? max(r, tmp[w]) : min(r, tmp[w]);
  __syncthreads();
  return r;
}

// Ascending ids of the k largest keys[0..n) (order-preserving keys in LDS), ties to
// the lower id; -1 padding when k > n.
//
// MSB-first radix select with 8-bit digits, starting below the bits that every key
// shares (found from the minimum and maximum key), with four privatised histograms
// to spread LDS atomics, and stopping as soon as the bin holding the k-th key is
// taken whole.  `hist` holds 4 x 256 ints, `bcast` 3 ints.
XKV_DEV void topk_keys(const uint32_t* keys, int n, int k, int* out, int* hist, int* tmp, int* bcast) {
  const int tid = threadIdx.x;
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < k; i += 256) out[i] = (i < n) ? i : -1;
    return;
  }
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = tid; i < n; i += 256) {
    lo = min(lo, keys[i]);
    hi = max(hi, keys[i]);
  }
  lo = block_reduce_minmax(lo, false, (uint32_t*)tmp);
  hi = block_reduce_minmax(hi, true, (uint32_t*)tmp);
  const int common = (lo == hi) ? 32 : __clz(lo ^ hi);   // leading bits every key shares
  uint32_t mask = common >= 32 ? 0xffffffffu : ~(0xffffffffu >> common);
  uint32_t prefix = lo & mask;
  int remaining = k;
  int bit = 32 - common;                                  // bits still to resolve
  while (bit > 0) {
    const int w = bit >= 8 ? 8 : bit;
    const int shift = bit - w;
    const uint32_t dmask = (1u << w) - 1u;
    for (int i = tid; i < 1024; i += 256) hist[i] = 0;
    __syncthreads();
    int* h4 = hist + ((tid & 3) << 8);
    for (int i = tid; i < n; i += 256) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&h4[(key >> shift) & dmask], 1);
    }
    __syncthreads();
    const int v = hist[255 - tid] + hist[256 + 255 - tid] + hist[512 + 255 - tid] + hist[768 + 255 - tid];
    const int incl = block_scan_incl(v, tmp);   // keys with digit >= 255 - tid
    const int excl = incl - v;                  // keys with digit >  255 - tid
    if (v > 0 && excl < remaining && remaining <= incl) {
      bcast[0] = 255 - tid;
      bcast[1] = remaining - excl;
      bcast[2] = v;
    }
    __syncthreads();
    prefix |= (uint32_t)bcast[0] << shift;
    mask |= dmask << shift;
    remaining = bcast[1];
    const bool whole = bcast[1] == bcast[2];   // the k-th key's bin is taken entirely
    __syncthreads();
    bit = shift;
    if (whole) break;
  }
  // Keys above the threshold prefix, then the first `remaining` keys equal to it in id order.
  const int seg = (n + 255) / 256;
  const int s0 = min(n, tid * seg), s1 = min(n, s0 + seg);
  int gt = 0, eq = 0;
  for (int i = s0; i < s1; ++i) {
    const uint32_t key = keys[i] & mask;
    gt += key > prefix;
    eq += key == prefix;
  }
  const int eq_before = block_scan_incl(eq, tmp) - eq;
  const int take_eq = max(0, min(eq, remaining - eq_before));
  const int mine = gt + take_eq;
  int pos = block_scan_incl(mine, tmp) - mine;
  int seen = 0;
  for (int i = s0; i < s1; ++i) {
    const uint32_t key = keys[i] & mask;
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
    rope_cs_turns(P.q_pos, P.turns[i], &c, &s);
    const float x = ld_elem(q + j * P.d + i), y = ld_elem(q + j * P.d + i + half);
    qs[j][i] = (x * c - y * s) * P.scale;
    qs[j][i + half] = (y * c + x * s) * P.scale;
  }
}

// Softmax partial of `grp` query heads over RB rows whose scores are in pw
// (-inf for absent rows): pw becomes exp(score - max); st_m, st_l get max and sum.
XKV_DEV void softmax_partial(int grp, float (*pw)[RB], float* st_m, float* st_l) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = wave; j < grp; j += 4) {
    const float v = pw[j][lane];
    const float mx = wave_max(v);
    const float p = (v == -INFINITY) ? 0.f : __expf(v - mx);
    const float l = wave_sum(p);
    pw[j][lane] = p;
    if (lane == 0) {
      st_m[j] = mx;
      st_l[j] = l;
    }
  }
}

// Exact rows of one (sequence, head): sink, local window, generated tokens, 64 per
// block (tile e_blk), each tile leaving its own partial.  The newest generated row is
// read from k_new / v_new when given, since block (0, 0, b) of the same launch is
// what copies it into the tail.
template <typename ST>
XKV_DEV void exact_rows(const SrParams& P, int b, int h, int e_blk, float (*qs)[MAXD], float* smem) {
  float (*kh)[HROW] = (float (*)[HROW])smem;
  float (*vh)[HROW] = (float (*)[HROW])(smem + RB * HROW);
  __shared__ float pw[MAXG][RB];
  __shared__ int pos_t[RB];
  __shared__ float run_m[MAXG], run_l[MAXG], run_a[MAXG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = P.d, half = d >> 1, grp = P.grp;
  const int n_tail = P.n_sink + P.n_local + P.n_gen;
  const ST* kt = (const ST*)P.k_tail + b * P.bs_tail + (long)h * d;
  const ST* vt = (const ST*)P.v_tail + b * P.bs_tail + (long)h * d;
  const ST* kn = P.k_new ? (const ST*)P.k_new + b * P.bs_new + (long)h * d : nullptr;
  const ST* vn = P.v_new ? (const ST*)P.v_new + b * P.bs_new + (long)h * d : nullptr;
  auto krow = [&](int row) -> const ST* { return (kn && row == n_tail - 1) ? kn : kt + (long)row * P.ld_tail; };
  auto vrow = [&](int row) -> const ST* { return (vn && row == n_tail - 1) ? vn : vt + (long)row * P.ld_tail; };
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  if (tid < MAXG) {
    run_m[tid] = -INFINITY;
    run_l[tid] = 0.f;
  }
  {
    const int r0 = e_blk * RB;   // this block's tile of the tail
    __syncthreads();
    if (tid < RB) {
      const int row = r0 + tid;
      int pos = -1;
      if (row < P.n_sink) pos = row;
      else if (row < P.n_sink + P.n_local) pos = P.T - P.n_local + (row - P.n_sink);
      else if (row < n_tail) pos = P.T + (row - P.n_sink - P.n_local);
      pos_t[tid] = pos;
    }
    __syncthreads();
    // Stage the tile's key and value rows (8 elements per load, every load issued first).
    {
      const int per_row = d >> 3;
      constexpr int U = 4;
      for (int e0 = tid; e0 < RB * per_row; e0 += 256 * U) {
        float kv[U][8], vv[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + 256 * u;
          const int rl = e / per_row, c8 = (e % per_row) * 8;
          if (e < RB * per_row && pos_t[rl] >= 0) {
            load8<ST>(krow(r0 + rl) + c8, kv[u]);
            load8<ST>(vrow(r0 + rl) + c8, vv[u]);
          } else {
#pragma unroll
            for (int x = 0; x < 8; ++x) kv[u][x] = vv[u][x] = 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + 256 * u;
          if (e < RB * per_row) {
            const int rl = e / per_row, c8 = (e % per_row) * 8;
#pragma unroll
            for (int x = 0; x < 8; ++x) {
              kh[rl][c8 + x] = kv[u][x];
              vh[rl][c8 + x] = vv[u][x];
            }
          }
        }
      }
    }
    __syncthreads();
    for (int e = tid; e < RB * half; e += 256) {
      const int rl = e / half, i = e % half;
      const int pos = pos_t[rl];
      if (pos >= 0) {
        float c, sn;
        rope_cs_turns(pos, P.turns[i], &c, &sn);
        const float lo = kh[rl][i], hi = kh[rl][i + half];
        kh[rl][i] = lo * c - hi * sn;
        kh[rl][i + half] = hi * c + lo * sn;
      }
    }
    __syncthreads();
    for (int e = tid; e < grp * RB; e += 256) {
      const int j = e / RB, rl = e % RB;
      float v = -INFINITY;
      if (pos_t[rl] >= 0) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < d; i += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) s4[u] += qs[j][i + u] * kh[rl][i + u];
        }
        v = (s4[0] + s4[1]) + (s4[2] + s4[3]);
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
#pragma unroll 8
        for (int rl = 0; rl < RB; ++rl) acc += pw[j][rl] * vh[rl][i];
        o[q] = acc;
      }
    }
  }
  __syncthreads();
  float* part = P.part_ex + (((long)b * P.Hkv + h) * P.n_exact + e_blk) * (long)grp * (2 + d);
  if (tid < grp) {
    part[tid] = run_m[tid];
    part[grp + tid] = run_l[tid];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q;
    if (e < grp * d) part[2 * grp + e] = o[q];
  }
}

template <typename ST>
__global__ __launch_bounds__(256) void sr_score_kernel(SrParams P) {
  extern __shared__ __align__(16) float smem_f[];
  __shared__ float qs[MAXG][MAXD];
  __shared__ float qsum[MAXD];
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
  if (blk >= P.score_blocks) {
    exact_rows<ST>(P, b, h, blk - P.score_blocks, qs, smem_f);
    return;
  }
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
  constexpr int BATCH = 8;
  for (int it0 = 0; it0 < iters; it0 += BATCH) {
    float v[BATCH][8];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = c0 + (it0 + u) * cpi + slot;
      if (it0 + u < iters && c < c1) {
        load8<ST>(lm + (long)c * P.d + sub * 8, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += qv[e] * v[u][e];
      for (int o = lpc >> 1; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
      const int c = c0 + (it0 + u) * cpi + slot;
      if (it0 + u < iters && c < c1 && sub == 0) scores[c] = dot;
    }
  }
}

__global__ __launch_bounds__(256) void sr_topk_kernel(SrParams P) {
  extern __shared__ __align__(16) uint32_t keys[];
  __shared__ int hist[1024];
  __shared__ int tmp[8];
  __shared__ int bcast[4];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const long bh = (long)b * P.Hkv + h;
  const float* scores = P.scores + bh * P.n_cand;
  // Rows of the score array are 16-byte aligned only when n_cand is a multiple of 4.
  const int n4 = (P.n_cand & 3) ? 0 : P.n_cand;
  for (int i = tid * 4; i < n4; i += 1024) {
    const float4 f = *(const float4*)(scores + i);
    keys[i] = order_key(f.x);
    keys[i + 1] = order_key(f.y);
    keys[i + 2] = order_key(f.z);
    keys[i + 3] = order_key(f.w);
  }
  for (int i = n4 + tid; i < P.n_cand; i += 256) keys[i] = order_key(scores[i]);
  __syncthreads();
  topk_keys(keys, P.n_cand, P.top_k, P.sel + bh * P.top_k, hist, tmp, bcast);
}

// Rows of split s: selected chunks [s*cps, (s+1)*cps) minus the exact-tail positions.
XKV_DEV void split_rows(const SrParams& P, long bh, int s, int* rows_t) {
  const int tid = threadIdx.x;
  if (tid < RB) {
    const int ci = s * P.cps + tid / P.chunk;
    const int c = (ci < P.k_eff) ? P.sel[bh * P.top_k + ci] : -1;
    const int t = c * P.chunk + tid % P.chunk;
    rows_t[tid] = (c >= 0 && t >= P.n_sink && t < P.T - P.n_local) ? t : -1;
  }
}

// The block's partial: max, sum and output sum of each query head of the group.
XKV_DEV void write_partial(const SrParams& P, int b, int h, int s, float (*pw)[RB], float (*vh)[HROW],
                           const float* st_m, const float* st_l) {
  const int tid = threadIdx.x, grp = P.grp, d = P.d;
  const long bh = (long)b * P.Hkv + h;
  float* part = P.part + (bh * P.n_splits + s) * (long)grp * (2 + d);
  if (tid < grp) {
    part[tid] = st_m[tid];
    part[grp + tid] = st_l[tid];
  }
  for (int e = tid; e < grp * d; e += 256) {
    const int j = e / d, i = e % d;
    float acc = 0.f;
#pragma unroll 8
    for (int row = 0; row < RB; ++row) acc += pw[j][row] * vh[row][i];
    part[2 * grp + e] = acc;
  }
}

__global__ __launch_bounds__(256) void sr_attend_mfma_kernel(SrParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* Ak = (uint16_t*)smem;              // [RB][AROW] staged A_k rows
  uint16_t* Av = Ak + RB * AROW;               // [RB][AROW] staged A_v rows
  float (*kh)[HROW] = (float (*)[HROW])smem;   // rotated keys, after the MFMA phase (aliases Ak)
  float (*vh)[HROW] = (float (*)[HROW])(smem + RB * AROW * 2);  // values (aliases Av)
  __shared__ float qs[MAXG][MAXD];
  __shared__ float pw[MAXG][RB];
  __shared__ int rows_t[RB];
  __shared__ float st_m[MAXG], st_l[MAXG];
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const long bh = (long)b * P.Hkv + h;
  const int r = P.r_k;

  split_rows(P, bh, s, rows_t);
  load_group_queries<uint16_t>(P, b, h, qs);
  __syncthreads();

  const bool kside = wave < 2;
  const int cp = wave & 1;
  const uint16_t* Ag_k = (const uint16_t*)P.A_k + b * P.bs_A_k;
  const uint16_t* Ag_v = (const uint16_t*)P.A_v + b * P.bs_A_v;
  const uint16_t* Bt = kside ? (const uint16_t*)P.Bt_k + b * P.bs_Bt_k + (long)h * 128 * P.ld_Bt_k
                             : (const uint16_t*)P.Bt_v + b * P.bs_Bt_v + (long)h * 128 * P.ld_Bt_v;
  const long ldB = kside ? P.ld_Bt_k : P.ld_Bt_v;
  const uint16_t* b0 = Bt + (long)(cp * 32 + (lane & 31)) * ldB;
  const uint16_t* b1 = b0 + 64L * ldB;
  const uint16_t* As = kside ? Ak : Av;
  const int half_off = (lane >> 5) * 32;

  f32x16_t acc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[rt][ct][j] = 0.f;

  for (int kc = 0; kc < r; kc += KCH) {
    const int kw = min(KCH, r - kc);
    // Stage the gathered rows: wave w takes rows 16w..16w+15, lane l bytes [16l, 16l+16).
    uint4 sk[16], sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = rows_t[wave * 16 + i];
      const bool ok = t >= 0 && lane * 8 < kw;
      sk[i] = ok ? *(const uint4*)(Ag_k + (long)t * P.ld_A_k + kc + lane * 8) : make_uint4(0, 0, 0, 0);
      sv[i] = ok ? *(const uint4*)(Ag_v + (long)t * P.ld_A_v + kc + lane * 8) : make_uint4(0, 0, 0, 0);
    }
    // B slices of the first two k-steps, in flight together with the row loads.
    uint4 bq[3][2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st * 64 < kw) {
        const int kb = kc + st * 64 + half_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bq[st][0][i] = *(const uint4*)(b0 + kb + 8 * i);
          bq[st][1][i] = *(const uint4*)(b1 + kb + 8 * i);
        }
      }
    }
    if (lane * 8 < kw) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        *(uint4*)(Ak + (wave * 16 + i) * AROW + lane * 8) = sk[i];
        *(uint4*)(Av + (wave * 16 + i) * AROW + lane * 8) = sv[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < KCH / 64; ++st) {
      if (st * 64 < kw) {
        if ((st + 2) * 64 < kw) {
          const int kb = kc + (st + 2) * 64 + half_off;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bq[(st + 2) % 3][0][i] = *(const uint4*)(b0 + kb + 8 * i);
            bq[(st + 2) % 3][1][i] = *(const uint4*)(b1 + kb + 8 * i);
          }
        }
        const int kl = st * 64 + half_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const bf16x8_t a = as_bf16x8(*(const uint4*)(As + (rt * 32 + (lane & 31)) * AROW + kl + 8 * i));
            acc[rt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(bq[st % 3][0][i]), acc[rt][0], 0, 0, 0);
            acc[rt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(bq[st % 3][1][i]), acc[rt][1], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }

  // Epilogue: keys get RoPE (pairs (i, i+64) sit in tiles cp and cp+2 of the same lane).
  const int i_lo = cp * 32 + (lane & 31);
  if (kside) {
    const double turns = P.turns[i_lo];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = rt * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
        const int t = rows_t[row];
        float c = 1.f, sn = 0.f;
        if (t >= 0) rope_cs_turns(t, turns, &c, &sn);
        const float lo = acc[rt][0][j], hi = acc[rt][1][j];
        kh[row][i_lo] = lo * c - hi * sn;
        kh[row][i_lo + 64] = hi * c + lo * sn;
      }
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = rt * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
        vh[row][i_lo] = acc[rt][0][j];
        vh[row][i_lo + 64] = acc[rt][1][j];
      }
  }
  __syncthreads();
  for (int e = tid; e < P.grp * RB; e += 256) {
    const int j = e / RB, row = e % RB;
    float v = -INFINITY;
    if (rows_t[row] >= 0) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
      for (int i = 0; i < 128; i += 4) {
        a0 += qs[j][i] * kh[row][i];
        a1 += qs[j][i + 1] * kh[row][i + 1];
        a2 += qs[j][i + 2] * kh[row][i + 2];
        a3 += qs[j][i + 3] * kh[row][i + 3];
      }
      v = (a0 + a1) + (a2 + a3);
    }
    pw[j][row] = v;
  }
  __syncthreads();
  softmax_partial(P.grp, pw, st_m, st_l);
  __syncthreads();
  write_partial(P, b, h, s, pw, vh, st_m, st_l);
}

template <typename ST>
__global__ __launch_bounds__(256) void sr_attend_generic_kernel(SrParams P) {
  __shared__ float qs[MAXG][MAXD];
  __shared__ float kh[RB][HROW];
  __shared__ float vh[RB][HROW];
  __shared__ float pw[MAXG][RB];
  __shared__ int rows_t[RB];
  __shared__ float st_m[MAXG], st_l[MAXG];
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = P.d, half = d >> 1;
  const long bh = (long)b * P.Hkv + h;

  split_rows(P, bh, s, rows_t);
  load_group_queries<ST>(P, b, h, qs);
  __syncthreads();
  const ST* A = (const ST*)P.A_k + b * P.bs_A_k;
  const ST* Bt = (const ST*)P.Bt_k + b * P.bs_Bt_k + (long)h * d * P.ld_Bt_k;
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
    if (t >= 0) rope_cs_turns(t, P.turns[i], &c, &sn);
    kh[row][i] = lo * c - hi * sn;
    kh[row][i + half] = hi * c + lo * sn;
  }
  if (P.r_v > 0) {
    const ST* Av = (const ST*)P.A_v + b * P.bs_A_v;
    const ST* Btv = (const ST*)P.Bt_v + b * P.bs_Bt_v + (long)h * d * P.ld_Bt_v;
    for (int e = tid; e < RB * d; e += 256) {
      const int row = e / d, i = e % d;
      const int t = rows_t[row];
      float v = 0.f;
      if (t >= 0) {
        const ST* ar = Av + (long)t * P.ld_A_v;
        const ST* br = Btv + (long)i * P.ld_Bt_v;
        for (int k = 0; k < P.r_v; ++k) v += ld_elem(ar + k) * ld_elem(br + k);
      }
      vh[row][i] = v;
    }
  } else {
    const ST* V = (const ST*)P.V_full + b * P.bs_V + (long)h * d;
    for (int e = tid; e < RB * d; e += 256) {
      const int row = e / d, i = e % d;
      const int t = rows_t[row];
      vh[row][i] = (t >= 0) ? ld_elem(V + (long)t * P.ld_V + i) : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < P.grp * RB; e += 256) {
    const int j = e / RB, row = e % RB;
    float v = -INFINITY;
    if (rows_t[row] >= 0) {
      v = 0.f;
      for (int i = 0; i < d; ++i) v += qs[j][i] * kh[row][i];
    }
    pw[j][row] = v;
  }
  __syncthreads();
  softmax_partial(P.grp, pw, st_m, st_l);
  __syncthreads();
  write_partial(P, b, h, s, pw, vh, st_m, st_l);
}

// Merge of the split partials and the exact-row partial of (b, h).  Partial q <
// n_splits is a split, partial n_splits the exact rows.  The headers are read in one
// parallel round into LDS; every output element then sums its partials with the
// loads of a batch issued together.
__global__ __launch_bounds__(256) void sr_merge_kernel(SrParams P) {
  __shared__ float wq[MAXP][MAXG];
  __shared__ float lq[MAXP][MAXG];
  __shared__ float run_l[MAXG];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int grp = P.grp, d = P.d;
  const int np = P.n_splits + P.n_exact;
  const long bh = (long)b * P.Hkv + h;
  const long stride = (long)grp * (2 + d);
  const float* pex = P.part_ex + bh * P.n_exact * stride;
  const float* p0 = P.part + bh * P.n_splits * stride;
  auto part = [&](int q) -> const float* {
    return q < P.n_splits ? p0 + q * stride : pex + (q - P.n_splits) * stride;
  };
  for (int idx = tid; idx < np * grp; idx += 256) {
    const int q = idx / grp, j = idx % grp;
    wq[q][j] = part(q)[j];
    lq[q][j] = part(q)[grp + j];
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
  constexpr int NB = 8;
  for (int e = tid; e < grp * d; e += 256) {
    const int j = e / d;
    float acc = 0.f;
    for (int q0 = 0; q0 < np; q0 += NB) {
      float v[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) v[u] = (q0 + u < np) ? part(q0 + u)[2 * grp + e] : 0.f;
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (q0 + u < np) acc += wq[q0 + u][j] * v[u];
    }
    P.out[((long)b * P.Hq + (long)h * grp) * d + e] = acc / run_l[j];
  }
}

__global__ __launch_bounds__(256) void topk_rows_kernel(const float* scores, int n_cand, long ld, int k, int* sel) {
  extern __shared__ __align__(16) uint32_t keys[];
  __shared__ int hist[1024];
  __shared__ int tmp[8];
  __shared__ int bcast[4];
  const float* sc = scores + blockIdx.x * ld;
  for (int i = threadIdx.x; i < n_cand; i += 256) keys[i] = order_key(sc[i]);
  __syncthreads();
  topk_keys(keys, n_cand, k, sel + (long)blockIdx.x * k, hist, tmp, bcast);
}

bool use_mfma(const SrParams& P, int bf16) {
  return bf16 && P.d == 128 && P.r_v > 0 && P.r_k == P.r_v && P.r_k % 64 == 0;
}

// Raise a kernel's dynamic-LDS limit once per process and kernel (to the largest size
// asked so far); `Tag` keeps one record per kernel.
template <int Tag, typename K>
hipError_t set_lds(K kernel, size_t bytes) {
  static size_t granted = 65536;
  if (bytes <= granted) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) granted = bytes;
  return e;
}

}  // namespace

hipError_t launch_sr_score(const SrParams& P, int bf16, hipStream_t st) {
  dim3 grid(P.score_blocks + P.n_exact, P.Hkv, P.batch);
  const size_t lds = (size_t)2 * RB * HROW * 4;   // the exact block's staged rows
  hipError_t e;
  if (bf16) {
    if ((e = set_lds<1>(sr_score_kernel<uint16_t>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(sr_score_kernel<uint16_t>, grid, dim3(256), lds, st, P);
  } else {
    if ((e = set_lds<2>(sr_score_kernel<float>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(sr_score_kernel<float>, grid, dim3(256), lds, st, P);
  }
  return hipGetLastError();
}

hipError_t launch_sr_topk(const SrParams& P, hipStream_t st) {
  if (P.top_k <= 0) return hipSuccess;
  const size_t lds = (size_t)(P.n_cand > 0 ? P.n_cand : 1) * 4;
  hipError_t e = set_lds<3>(sr_topk_kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sr_topk_kernel, dim3(P.Hkv, P.batch), dim3(256), lds, st, P);
  return hipGetLastError();
}

hipError_t launch_sr_attend(const SrParams& P, int bf16, hipStream_t st) {
  if (P.n_splits == 0) return hipSuccess;
  dim3 grid(P.Hkv, P.n_splits, P.batch);
  if (use_mfma(P, bf16)) {
    const size_t lds = (size_t)2 * RB * AROW * sizeof(uint16_t);
    hipError_t e = set_lds<4>(sr_attend_mfma_kernel, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sr_attend_mfma_kernel, grid, dim3(256), lds, st, P);
  } else if (bf16) {
    hipLaunchKernelGGL(sr_attend_generic_kernel<uint16_t>, grid, dim3(256), 0, st, P);
  } else {
    hipLaunchKernelGGL(sr_attend_generic_kernel<float>, grid, dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

hipError_t launch_sr_merge(const SrParams& P, hipStream_t st) {
  hipLaunchKernelGGL(sr_merge_kernel, dim3(P.Hkv, P.batch), dim3(256), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int rows, int n_cand, long ld, int k, int* sel, hipStream_t st) {
  const size_t lds = (size_t)n_cand * 4;
  hipError_t e = set_lds<5>(topk_rows_kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(256), lds, st, scores, n_cand, ld, k, sel);
  return hipGetLastError();
}

}  // namespace xkv
