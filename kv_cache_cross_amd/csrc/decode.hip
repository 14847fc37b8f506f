// Selective Reconstruction decode for one layer and one step (xKV blog,
// section on Selective Reconstruction; decode attention as in KQ-SVD
// section 3.2).  Three kernels on the matrix-core path, four otherwise, ordered by
// the stream (no device-scope fences inside any of them: on this GPU such a fence
// writes back the XCD's L2):
//
// sr_score_kernel (grid: KV heads x (exact tiles + score_blocks) x batch)
//   * the first blocks of each (head, sequence) attend one 64-row tile each of the
//     exact rows (sink, local window, generated tokens), which do not depend on the
//     selection, and leave a softmax partial (max, denominator, weighted value sum) per
//     query head;
//   * the first score block of head 0 appends the new token's pre-RoPE k, v to the
//     exact tail;
//   * every score block forms the scaled, rotated query sum of the KV head's query
//     group and scores a slice of the candidate chunks against the landmarks
//     (a GEMV that streams the landmarks once, each thread's loads issued
//     before its arithmetic).
// top-k selection (topk_keys): a head's scores become order-preserving keys in
//   registers; a histogram over value buckets and a radix select inside the k-th key's
//   bucket find the k-th key, and an index-ordered compaction yields the k chunk ids
//   (ties to the lower id).  On the matrix-core path (up to 16384 candidates per head)
//   every attend block runs it for its
//   head (the scores come from L2) and keeps its own split's ids; otherwise
//   sr_topk_kernel (one 1024-thread block per head and sequence) writes them all.
// sr_attend_mfma_kernel (bf16, head_dim 128, r_k % 128 == 0 and r_v == r_k, or r_v == 0
// with exact values (xK-SR); grid: KV heads x splits x batch, so one head's blocks
// share an XCD and its B slices in L2; 512 threads, one block per CU)
//   * a block takes 64 rows: the selected chunks [s*64/chunk, (s+1)*64/chunk) of its
//     head, minus rows the exact tail covers;
//   * the gathered rows of A_k and the block's B_k,l,h slice reach LDS with
//     direct-to-LDS loads; the value rows (A_v rank chunk, or exact V rows) follow
//     once the A_k rows have landed and arrive while the keys are formed;
//   * the eight waves rebuild k_t = A_k[t] B_k,l,h on v_mfma_f32_16x16x32_bf16, the
//     dims ordered so that RoPE pairs meet in one lane; scores (on the MFMA, bf16 hi + lo
//     parts) and a softmax partial follow;
//   * values are never rebuilt: since v_t = A_v[t] B_v,l,h, the block's weighted value
//     sum is (sum_t p_t A_v[t]) B_v,l,h, and it leaves the rank-r vector
//     sum_t p_t A_v[t] per query head.
// sr_attend_generic_kernel covers every other shape (float32, other head
// dims, exact values, ranks that differ) with value-space partials.
// sr_merge_kernel (grid: query heads x batch) and, for the matrix-core path,
//   sr_merge_rank_kernel (grid: KV heads x query heads per group x 4 dim slices x batch) merge
//   the split partials and the exact-row partials by their log-sum-exp weights
//   into the output; the latter applies B_v,l,h to the merged rank-r sum.
#include <hip/hip_ext.h>
#include <algorithm>
#include <mutex>
#include "xkv_common.h"
#include "xkv_kernels.h"
#include "decode_params.h"

namespace xkv {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int RB = 64;        // rows per attend block (generic path) and per exact-row tile
constexpr int RBM = 64;       // rows per matrix-core attend block
constexpr int ETR = 16;       // rows per exact-row tile
constexpr int MAXG = 8;       // largest query group per KV head
constexpr int MAXD = 128;     // largest head dim
constexpr int EROW = MAXD + 4;   // LDS row of a staged exact row (16-byte aligned rows)
constexpr int KCH = 512;      // rank columns staged per pass (MFMA path)
constexpr int AROW = KCH + 8; // padded LDS row of staged A rows (bf16 elements)
constexpr int HROW = MAXD + 1;
constexpr int MAXP = 257;     // splits + exact tiles that the value-space merge supports
constexpr int MAXP_RANK = 1088;   // ... and the rank-space merge (every chunk selected at 64k)

XKV_DEV uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;   // -0.0 ranks equal to +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide float sum / max with DPP moves (the pattern of wave_scan_add below, on
// float bit patterns), the result read from lane 63 and shared by every lane.
#define XKV_DPP_F(old, v, ctrl, rm, bc) \
  __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), ctrl, rm, 0xF, bc))
XKV_DEV float wave_sum(float v) {
  v += XKV_DPP_F(0.f, v, 0x111, 0xF, true);
  v += XKV_DPP_F(0.f, v, 0x112, 0xF, true);
  v += XKV_DPP_F(0.f, v, 0x114, 0xF, true);
  v += XKV_DPP_F(0.f, v, 0x118, 0xF, true);
  v += XKV_DPP_F(0.f, v, 0x142, 0xA, false);
  v += XKV_DPP_F(0.f, v, 0x143, 0xC, false);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
XKV_DEV float wave_max(float v) {
  v = fmaxf(v, XKV_DPP_F(-INFINITY, v, 0x111, 0xF, false));
  v = fmaxf(v, XKV_DPP_F(-INFINITY, v, 0x112, 0xF, false));
  v = fmaxf(v, XKV_DPP_F(-INFINITY, v, 0x114, 0xF, false));
  v = fmaxf(v, XKV_DPP_F(-INFINITY, v, 0x118, 0xF, false));
  v = fmaxf(v, XKV_DPP_F(-INFINITY, v, 0x142, 0xA, false));
  v = fmaxf(v, XKV_DPP_F(-INFINITY, v, 0x143, 0xC, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over aligned groups of `lanes` (8 or 16) lanes, the result in every lane of the
// group: quad_perm [1,0,3,2] then [2,3,0,1] sum each quad, row_half_mirror adds the
// mirrored quad of each 8-lane half, row_mirror the mirrored half of each 16-lane row.
XKV_DEV float lane_group_sum(float v, int lanes) {
  v += XKV_DPP_F(0.f, v, 0xB1, 0xF, false);
  v += XKV_DPP_F(0.f, v, 0x4E, 0xF, false);
  v += XKV_DPP_F(0.f, v, 0x141, 0xF, false);
  if (lanes == 16) v += XKV_DPP_F(0.f, v, 0x140, 0xF, false);
  return v;
}

// Barrier for LDS hand-offs: this wave's LDS stores have completed (lgkmcnt(0)), then
// s_barrier.  No memory fence: a workgroup fence would also wait for every global load
// and direct-to-LDS load in flight, which the attend kernel keeps going across barriers.
// The empty asm statements keep the compiler from moving memory accesses across it.
XKV_DEV void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt not waited for
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

constexpr int TKT = 1024;      // threads of a top-k block

// Wave-wide prefix sum / min / max with DPP moves (no LDS round trips): Hillis-Steele
// steps of 1, 2, 4 and 8 lanes inside each row of 16, then the row totals carried across
// rows with the row broadcasts of lanes 15 and 31.  Lanes a shift reaches past the row
// start take the operation's identity.
XKV_DEV int wave_scan_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}
XKV_DEV uint32_t wave_min_u32(uint32_t v) {
  const int id = -1;
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
XKV_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The top-k helpers below run in blocks of NT threads (NT / 64 waves, NT >= 256) and
// hand data over through LDS only, so their barriers are lds_sync(): global and
// direct-to-LDS loads a caller has in flight keep going across them.

// Inclusive prefix sum over the NT threads of a block (`tmp` >= NT / 64 ints).  No
// barrier after the reads of tmp: the caller passes one before tmp is written again.
template <int NT>
XKV_DEV int tk_scan_incl(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_add(v);
  if (lane == 63) tmp[wave] = v;
  lds_sync();
  int add = 0;
#pragma unroll
  for (int w = 0; w < NT / 64 - 1; ++w) add += (w < wave) ? tmp[w] : 0;   // independent reads
  return v + add;
}

// Block-wide minimum of lo and maximum of hi (`tmp` >= 2 NT / 64 ints).  As above, the
// caller passes a barrier before tmp is written again.
template <int NT>
XKV_DEV void tk_minmax(uint32_t& lo, uint32_t& hi, uint32_t* tmp) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    tmp[wave] = lo;
    tmp[NW + wave] = hi;
  }
  lds_sync();
  lo = tmp[0];
  hi = tmp[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = min(lo, tmp[w]);
    hi = max(hi, tmp[NW + w]);
  }
}

// Value of an order-preserving key (inverse of order_key, -0.0 read as +0.0).
XKV_DEV float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

constexpr int NBK = 2048;   // linear value buckets of the first top-k pass

// Ascending ids of the k largest of n order-preserving keys, ties to the lower id;
// -1 padding when k > n.  Only positions [lo_out, hi_out) of that list are written, to
// out[pos - lo_out] (a caller that needs the whole list passes 0, k).  A block of NT
// threads; thread t holds keys t*KPT .. t*KPT + KPT - 1 in registers (n <= NT * KPT,
// KPT <= 32).
//
// Pass 1 spreads the keys over NBK buckets linear in value between the minimum and
// the maximum (a monotone map, so every key of a higher bucket is larger than every
// key of a lower one) and finds the bucket b* that holds the k-th largest key; with
// scores spread over a range, LDS atomics rarely collide.  When b* holds at most 64
// keys one wave ranks them directly; otherwise an MSB-first radix select with 8-bit
// digits, starting below the bits that b*'s keys share, resolves the k-th key exactly,
// stopping as soon as the bin holding it is taken whole.  Non-finite extremes put every key in one bucket and leave the radix
// select to do all the work.  `hist` holds NBK ints, `tmp` 2 NT / 64, `bcast` 4.  The
// block's barriers are the ones the data hand-offs need (seven on the usual path); the
// function ends without one, so a caller that reuses the buffers passes a barrier first.
template <int KPT, int NT>
XKV_DEV void topk_keys(const uint32_t (&kr)[KPT], const float (&fv)[KPT], int n, int k, int lo_out, int hi_out,
                       int* out, int* hist, int* tmp, int* bcast) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int base = tid * KPT;
  if (k <= 0) return;
  hi_out = min(hi_out, k);
  auto emit = [&](int pos, int id) {
    if (pos >= lo_out && pos < hi_out) out[pos - lo_out] = id;
  };
  if (k >= n) {
    for (int i = lo_out + tid; i < hi_out; i += NT) out[i - lo_out] = (i < n) ? i : -1;
    return;
  }
  for (int i = tid; i < NBK; i += NT) hist[i] = 0;   // made visible by tk_minmax's barrier
  if (tid == 0) bcast[3] = 0;                           // gather count of the few-keys path
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (base + u < n) {
      lo = min(lo, kr[u]);
      hi = max(hi, kr[u]);
    }
  tk_minmax<NT>(lo, hi, (uint32_t*)tmp);
  const float fmin = key_value(lo), fmax = key_value(hi);
  float inv = 0.f;
  if (__builtin_isfinite(fmin) && __builtin_isfinite(fmax) && fmax > fmin) {
    inv = (float)NBK / (fmax - fmin);
    if (!__builtin_isfinite(inv)) inv = 0.f;
  }
  // Bucket of each key, -1 past n (a monotone map of the value; -0.0 falls with +0.0, a
  // NaN maximum leaves inv = 0).
  int bk[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    bk[u] = (base + u >= n) ? -1 : (inv == 0.f) ? 0 : (int)fminf((fv[u] - fmin) * inv, (float)(NBK - 1));

  // Pass 1: bucket histogram (keys past n add 0 to bucket 0, so that no atomic sits in a
  // branch), then the bucket b* holding the k-th largest key.
#pragma unroll
  for (int u = 0; u < KPT; ++u) atomicAdd(&hist[max(bk[u], 0)], bk[u] >= 0 ? 1 : 0);
  lds_sync();
  {
    constexpr int BPT = NBK / NT;        // buckets per thread
    const int top = NBK - 1 - BPT * tid; // this thread's buckets top, top-1, ...
    int v = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) v += hist[top - u];
    const int incl = tk_scan_incl<NT>(v, tmp);   // keys in buckets >= top - BPT + 1
    int c = incl - v;                         // keys in buckets > top
    if (c < k && k <= incl) {
      for (int u = 0; u < BPT; ++u) {
        const int hb = hist[top - u];
        if (c + hb >= k) {
          bcast[0] = top - u;
          bcast[1] = c;
          bcast[2] = hb;
          break;
        }
        c += hb;
      }
    }
  }
  lds_sync();
  // hist, tmp and bcast[0..2] are rewritten only after at least one more barrier
  const int bstar = bcast[0];
  int remaining = k - bcast[1];   // keys still to take from b*, 1..|b*|
  const int m_b = bcast[2];

  // Few keys in b* (the usual case): gather them; each thread then ranks its own keys of
  // b* among them by (key descending, id ascending) and keeps those ranked below
  // `remaining`; every key of a higher bucket is kept.
  if (m_b <= 64) {
    uint32_t selm = 0u;
#pragma unroll
    for (int u = 0; u < KPT; ++u) selm |= (uint32_t)(bk[u] > bstar) << u;
    if (remaining < m_b) {
      uint32_t* lkey = (uint32_t*)hist;   // the bucket histogram is no longer needed
      int* lid = hist + 64;
      int* lcount = bcast + 3;            // zeroed before the first barrier
      uint32_t inb = 0u;
#pragma unroll
      for (int u = 0; u < KPT; ++u) inb |= (uint32_t)(bk[u] == bstar) << u;
      for (uint32_t m = inb; m; m &= m - 1u) {
        const int u = __ffs(m) - 1;
        const int at = atomicAdd(lcount, 1);
        lkey[at] = kr[u];
        lid[at] = base + u;
      }
      lds_sync();
      for (uint32_t m = inb; m; m &= m - 1u) {
        const int u = __ffs(m) - 1;
        const uint32_t key = kr[u];
        const int id = base + u;
        int rank = 0;
        for (int j = 0; j < m_b; ++j) rank += lkey[j] > key || (lkey[j] == key && lid[j] < id);
        selm |= (uint32_t)(rank < remaining) << u;
      }
    } else {
#pragma unroll
      for (int u = 0; u < KPT; ++u) selm |= (uint32_t)(bk[u] == bstar) << u;
    }
    const int mine = __popc(selm);
    int pos = tk_scan_incl<NT>(mine, tmp) - mine;
    while (selm) {
      emit(pos++, base + __ffs(selm) - 1);
      selm &= selm - 1u;
    }
    return;
  }

  // Pass 2: radix select of the remaining-th largest key inside b*.
  uint32_t mask = 0u, prefix = 0u;
  if (remaining < m_b) {
    uint32_t lo2 = 0xffffffffu, hi2 = 0u;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (bk[u] == bstar) {
        lo2 = min(lo2, kr[u]);
        hi2 = max(hi2, kr[u]);
      }
    tk_minmax<NT>(lo2, hi2, (uint32_t*)tmp);
    const int common = (lo2 == hi2) ? 32 : __clz(lo2 ^ hi2);   // leading bits b*'s keys share
    mask = common >= 32 ? 0xffffffffu : ~(0xffffffffu >> common);
    prefix = lo2 & mask;
    int bit = 32 - common;                                     // bits still to resolve
    while (bit > 0) {
      const int w = bit >= 8 ? 8 : bit;
      const int shift = bit - w;
      const uint32_t dmask = (1u << w) - 1u;
      for (int i = tid; i < 256; i += NT) hist[i] = 0;
      lds_sync();
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (bk[u] == bstar && (kr[u] & mask) == prefix) atomicAdd(&hist[(kr[u] >> shift) & dmask], 1);
      lds_sync();
      const int v = tid < 256 ? hist[255 - tid] : 0;
      const int incl = tk_scan_incl<NT>(v, tmp);   // keys with digit >= 255 - tid
      const int excl = incl - v;               // keys with digit >  255 - tid
      if (v > 0 && excl < remaining && remaining <= incl) {
        bcast[0] = 255 - tid;
        bcast[1] = remaining - excl;
        bcast[2] = v;
      }
      lds_sync();
      prefix |= (uint32_t)bcast[0] << shift;
      mask |= dmask << shift;
      remaining = bcast[1];
      const bool whole = bcast[1] == bcast[2];   // the k-th key's bin is taken entirely
      bit = shift;
      if (whole) break;
    }
  }
  lds_sync();   // the reads of tmp and bcast above are done
  // Keys of higher buckets and keys of b* above the threshold prefix, then the first
  // `remaining` keys of b* equal to it in id order.
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    gtm |= (uint32_t)(bk[u] > bstar || (bk[u] == bstar && (kr[u] & mask) > prefix)) << u;
    eqm |= (uint32_t)(bk[u] == bstar && (kr[u] & mask) == prefix) << u;
  }
  const int eq = __popc(eqm);
  const int eq_before = tk_scan_incl<NT>(eq, tmp) - eq;
  int take = max(0, min(eq, remaining - eq_before));
  uint32_t sel = gtm;
  while (take-- > 0) {
    sel |= eqm & (0u - eqm);   // lowest remaining equal key
    eqm &= eqm - 1u;
  }
  const int mine = __popc(sel);
  int pos = tk_scan_incl<NT>(mine, tmp + NW) - mine;   // the other half: tmp may still be read
  while (sel) {
    emit(pos++, base + __ffs(sel) - 1);
    sel &= sel - 1u;
  }
}

// Order-preserving keys of scores[0..n) for thread t's slice t*KPT .. t*KPT + KPT - 1
// (16-byte loads when the slice is 16-byte aligned).
template <int KPT>
XKV_DEV void load_keys(const float* scores, int n, uint32_t (&kr)[KPT]) {
  const int base = threadIdx.x * KPT;
  if (KPT % 4 == 0 && (((uintptr_t)scores) & 15) == 0 && base + KPT <= n) {
#pragma unroll
    for (int u = 0; u < KPT; u += 4) {
      const float4 f = *(const float4*)(scores + base + u);
      kr[u] = order_key(f.x);
      kr[u + 1] = order_key(f.y);
      kr[u + 2] = order_key(f.z);
      kr[u + 3] = order_key(f.w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < KPT; ++u) kr[u] = (base + u < n) ? order_key(scores[base + u]) : 0u;
  }
}

// Eight storage elements held raw in registers (the load issued now, the conversion
// to float done where the values are used).
template <typename ST>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  uint4 u;
  XKV_DEV void load(const uint16_t* p) { u = *(const uint4*)p; }
  XKV_DEV void get(float* v) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Raw8<float> {
  float4 a, b;
  XKV_DEV void load(const float* p) {
    a = *(const float4*)p;
    b = *(const float4*)(p + 4);
  }
  XKV_DEV void get(float* v) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

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

// Exact rows of one (sequence, head): sink, local window, generated tokens, ETR per
// block of NT threads (tile e_blk), each tile leaving its own softmax partial.  These
// blocks ride in the score launch, ahead of its score blocks: they depend on nothing
// the step computes, and small tiles keep each block's work well inside the scoring
// blocks' time.  The tile's rows are requested before the queries, so the two
// latencies overlap.  The newest generated row is read from k_new / v_new when given,
// since the score launch copies it into the tail in this same step.
template <typename ST, int NT>
XKV_DEV void exact_tile(const SrParams& P, int b, int h, int e_blk, float* smem) {
  static_assert(NT == 256 && ETR * (MAXD / 8) <= NT && MAXG * ETR * 2 <= NT, "exact tile layout");
  // One staging buffer holds the tile's keys, then (once the scores are formed) its
  // values; the value rows wait in registers meanwhile.
  float (*kh)[EROW] = (float (*)[EROW])smem;
  float (*vh)[EROW] = kh;
  float (*qs)[MAXD] = (float (*)[MAXD])(smem + ETR * EROW);
  float (*pw)[ETR] = (float (*)[ETR])(smem + ETR * EROW + MAXG * MAXD);
  float* st_m = smem + ETR * EROW + MAXG * MAXD + MAXG * ETR;
  float* st_l = st_m + MAXG;
  double* turns_s = (double*)(st_l + MAXG);   // RoPE frequencies, read from LDS after the first barrier
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = P.d, half = d >> 1, grp = P.grp;
  const int lh = d == 128 ? 6 : 5;   // log2(half): head_dim is 64 or 128
  const int n_tail = P.n_sink + P.n_local + P.n_gen;
  const int r0 = e_blk * ETR;   // this block's tile of the tail
  auto pos_of = [&](int row) -> int {
    if (row < P.n_sink) return row;
    if (row < P.n_sink + P.n_local) return P.T - P.n_local + (row - P.n_sink);
    if (row < n_tail) return P.T + (row - P.n_sink - P.n_local);
    return -1;
  };
  const ST* kt = (const ST*)P.k_tail + b * P.bs_tail + (long)h * d;
  const ST* vt = (const ST*)P.v_tail + b * P.bs_tail + (long)h * d;
  const ST* kn = P.k_new ? (const ST*)P.k_new + b * P.bs_new + (long)h * d : nullptr;
  const ST* vn = P.v_new ? (const ST*)P.v_new + b * P.bs_new + (long)h * d : nullptr;
  // Thread t loads 8-element group t of the tile's keys and values (row t / (d/8)), raw.
  const int per_row = d >> 3;
  const int rl = tid / per_row, c8 = (tid % per_row) * 8;
  const bool ld_mine = tid < ETR * per_row && r0 + rl < n_tail;
  Raw8<ST> rk, rv;
  if (ld_mine) {
    const int row = r0 + rl;
    const bool newest = kn && row == n_tail - 1;
    rk.load((newest ? kn : kt + (long)row * P.ld_tail) + c8);
    rv.load((newest ? vn : vt + (long)row * P.ld_tail) + c8);
  }
  // The group's raw query pairs (pair e = j half + i for e = tid, tid + NT) and the RoPE
  // frequencies are requested with the rows; they are rotated after the first barrier.
  constexpr int QPT = MAXG * (MAXD / 2) / NT;
  float qx[QPT], qy[QPT];
  {
    const ST* q = (const ST*)P.q + ((long)b * P.Hq + (long)h * grp) * d;
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = tid + NT * u, j = e >> lh, i = e & (half - 1);
      qx[u] = e < grp * half ? ld_elem(q + j * d + i) : 0.f;
      qy[u] = e < grp * half ? ld_elem(q + j * d + i + half) : 0.f;
    }
    if (tid < half) turns_s[tid] = P.turns[tid];
  }
  // Staged rows past the tail are zero.
  auto stage = [&](const Raw8<ST>& raw) {
    if (tid < ETR * per_row) {
      float x8[8];
      const bool mine = r0 + rl < n_tail;
      if (mine) raw.get(x8);
#pragma unroll
      for (int x = 0; x < 8; ++x) kh[rl][c8 + x] = mine ? x8[x] : 0.f;
    }
  };
  stage(rk);
  __syncthreads();
  // Rotated, scaled queries, and RoPE on the staged keys (pair i of row r for
  // e = r half + i).
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int e = tid + NT * u, j = e >> lh, i = e & (half - 1);
    if (e < grp * half) {
      float c, s;
      rope_cs_turns(P.q_pos, turns_s[i], &c, &s);
      qs[j][i] = (qx[u] * c - qy[u] * s) * P.scale;
      qs[j][i + half] = (qy[u] * c + qx[u] * s) * P.scale;
    }
  }
  for (int e = tid; e < ETR * half; e += NT) {
    const int r = e >> lh, i = e & (half - 1);
    float c, sn;   // rows past the tail rotate by angle 0; their scores are masked
    rope_cs_turns(max(pos_of(r0 + r), 0), turns_s[i], &c, &sn);
    const float lo = kh[r][i], hi = kh[r][i + half];
    kh[r][i] = lo * c - hi * sn;
    kh[r][i + half] = hi * c + lo * sn;
  }
  __syncthreads();
  {
    // Score (j, r) by the lane pair 2 (j ETR + r) + {0, 1}, one half of the dims each,
    // the halves added across the pair.
    const int pr = tid >> 1, hs = tid & 1;
    const int j = pr / ETR, r = pr % ETR;
    const int jq = min(j, grp - 1);
    const int i0 = hs * half;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = i0; i < i0 + half; i += 4) {
      const float4 qv = *(const float4*)&qs[jq][i];
      const float4 kv = *(const float4*)&kh[r][i];
      a[0] += qv.x * kv.x;
      a[1] += qv.y * kv.y;
      a[2] += qv.z * kv.z;
      a[3] += qv.w * kv.w;
    }
    float v = (a[0] + a[1]) + (a[2] + a[3]);
    v += XKV_DPP_F(0.f, v, 0xB1, 0xF, false);   // quad_perm [1, 0, 3, 2]: the pair's other half
    if (hs == 0 && j < grp) pw[j][r] = (r0 + r < n_tail) ? v : -INFINITY;
  }
  __syncthreads();
  for (int j = wave; j < grp; j += NT / 64) {
    const float v = lane < ETR ? pw[j][lane] : -INFINITY;
    const float mx = wave_max(v);
    const float p = (v == -INFINITY) ? 0.f : __expf(v - mx);
    const float l = wave_sum(p);
    if (lane < ETR) pw[j][lane] = p;
    if (lane == 0) {
      st_m[j] = mx;
      st_l[j] = l;
    }
  }
  stage(rv);   // the keys are no longer read: the buffer takes the values
  __syncthreads();
  float* part = P.part_ex + (((long)b * P.Hkv + h) * P.n_exact + e_blk) * (long)grp * (2 + d);
  if (tid < grp) {
    part[tid] = st_m[tid];
    part[grp + tid] = st_l[tid];
  }
  {
    // Thread (dim i, head group jg): heads jg hpt .. + hpt of dim i over the tile's rows,
    // each value read once for its heads, the weights wave-uniform (broadcast).
    const int ngrp = NT / d;              // head groups: 2 (d = 128) or 4 (d = 64)
    const int hpt = MAXG / ngrp;
    const int i = tid % d, jg = tid / d;
    const int jb = jg * hpt;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < ETR; ++r) {
      const float v = vh[r][i];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += pw[min(jb + u, MAXG - 1)][r] * v;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < hpt && jb + u < grp) part[2 * grp + (long)(jb + u) * d + i] = acc[u];
  }
}

// Blocks y < n_exact of the grid attend exact-row tile y of their (head, sequence); the
// rest score a slice of the candidate chunks each.
template <typename ST>
__global__ __launch_bounds__(256) void sr_score_kernel(SrParams P) {
  extern __shared__ __align__(16) float smem_x[];
  __shared__ float qs[MAXG][MAXD];
  __shared__ float qsum[MAXD];
  const int h = blockIdx.x, b = blockIdx.z, tid = threadIdx.x;
  if ((int)blockIdx.y < P.n_exact) {
    exact_tile<ST, 256>(P, b, h, blockIdx.y, smem_x);
    return;
  }
  const int blk = blockIdx.y - P.n_exact;

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

  const int per_blk = (P.n_cand + P.score_blocks - 1) / P.score_blocks;
  const int c0 = blk * per_blk, c1 = min(P.n_cand, c0 + per_blk);
  if (c0 >= c1) return;
  // The raw queries and their RoPE frequencies are requested first, then the landmarks
  // of the first BATCH passes: the queries arrive first (loads return in order), and
  // their rotation and sum proceed while the landmarks are in flight.  Thread t takes
  // (head, pair) = (e / half, e % half) for e = t and t + 256.
  const int half = P.d >> 1;
  const ST* qg = (const ST*)P.q + ((long)b * P.Hq + (long)h * P.grp) * P.d;
  float qx[2] = {0.f, 0.f}, qy[2] = {0.f, 0.f};
  double qt[2] = {0.0, 0.0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + 256 * u;
    if (e < P.grp * half) {
      const int j = e / half, i = e % half;
      qx[u] = ld_elem(qg + j * P.d + i);
      qy[u] = ld_elem(qg + j * P.d + i + half);
      qt[u] = P.turns[i];
    }
  }
  // Past-the-end slots re-read the block's last chunk (in bounds) and are not stored.
  const int lpc = P.d >> 3;           // lanes per chunk, 8 elements each
  const int cpi = 256 / lpc;          // chunks per pass
  const int sub = tid % lpc, slot = tid / lpc;
  const ST* lm = (const ST*)P.lm + b * P.bs_lm + (long)h * P.n_chunks * P.d + sub * 8;
  float* scores = P.scores + ((long)b * P.Hkv + h) * P.ld_sc;
  const int iters = (c1 - c0 + cpi - 1) / cpi;
  constexpr int BATCH = 8;
  Raw8<ST> raw[BATCH];
  // unconditional (slots past the block re-read its last chunk), so that the wait for the
  // queries above is an exact count of the loads behind them
#pragma unroll
  for (int u = 0; u < BATCH; ++u) raw[u].load(lm + (long)min(c0 + u * cpi + slot, c1 - 1) * P.d);

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + 256 * u;
    if (e < P.grp * half) {
      const int j = e / half, i = e % half;
      float c, sn;
      rope_cs_turns(P.q_pos, qt[u], &c, &sn);
      qs[j][i] = (qx[u] * c - qy[u] * sn) * P.scale;
      qs[j][i + half] = (qy[u] * c + qx[u] * sn) * P.scale;
    }
  }
  __syncthreads();
  for (int i = tid; i < P.d; i += 256) {
    float s = 0.f;
    for (int j = 0; j < P.grp; ++j) s += qs[j][i];
    qsum[i] = s;
  }
  __syncthreads();
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qsum[sub * 8 + e];
  for (int it0 = 0; it0 < iters; it0 += BATCH) {
    if (it0 > 0) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (it0 + u < iters) raw[u].load(lm + (long)min(c0 + (it0 + u) * cpi + slot, c1 - 1) * P.d);
    }
    // All BATCH slots are reduced together (slots past `iters` hold unused values), so
    // the lane-group sums of different chunks overlap instead of waiting on each other.
    float dots[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      float v[8];
      raw[u].get(v);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += qv[e] * v[e];
      dots[u] = dot;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) dots[u] = lane_group_sum(dots[u], lpc);
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = c0 + (it0 + u) * cpi + slot;
      if (it0 + u < iters && c < c1 && sub == 0) scores[c] = dots[u];
    }
  }
}

// One block per (head, sequence) selects its top-k chunks (the paths whose attend
// kernel does not select them itself).
template <int KPT>
__global__ __launch_bounds__(TKT) void sr_topk_kernel(SrParams P) {
  __shared__ int hist[NBK];
  __shared__ int tmp[2 * (TKT / 64)];
  __shared__ int bcast[4];
  const int h = blockIdx.x % P.Hkv, b = blockIdx.x / P.Hkv;
  const long bh = (long)b * P.Hkv + h;
  uint32_t kr[KPT];
  float fv[KPT];
  load_keys<KPT>(P.scores + bh * P.ld_sc, P.n_cand, kr);
#pragma unroll
  for (int u = 0; u < KPT; ++u) fv[u] = key_value(kr[u]);
  topk_keys<KPT, TKT>(kr, fv, P.n_cand, P.top_k, 0, P.top_k, P.sel + bh * P.top_k, hist, tmp, bcast);
}

// Rows of split s: selected chunks [s*cps, (s+1)*cps) minus the exact-tail positions.
XKV_DEV void split_rows(const SrParams& P, long bh, int s, int nrows, int* rows_t) {
  const int tid = threadIdx.x;
  if (tid < nrows) {
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

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): two bf16 MFMA operands whose
// products carry about 16 significant bits of x.
XKV_DEV void split_bf16x8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 b = (__bf16)x[e];
    hi[e] = b;
    lo[e] = (__bf16)(x[e] - (float)b);
  }
}

constexpr int VROW_MAX = KCH + 16;   // LDS row of the value rows written for the weighted sum
constexpr int QSLOT = 8 * VROW_MAX * 2;   // bytes of one wave's share of region V

// EXACT_V: values are exact rows of V_full (xK-SR); the partial holds the value-space
// sum sum_t p_t v_t per query head instead of the rank-space sum.
//
// Work split of one block (64 gathered rows of one KV head, eight waves):
//  * keys: wave w = (dim group dg = w % 4, rank half kh = w / 4) rebuilds key dims
//    16 dg + m and 64 + 16 dg + m (m < 16) of all 64 rows over half of each rank chunk,
//    as K^T tiles D[dim][row] = B_k[dim] . A_k[row] (the B_k slice is the MFMA A
//    operand, from registers; the staged A_k rows are the B operand, from LDS).  A lane
//    then holds dims 4(l/16) + v of both halves of a RoPE pair for one row;
//  * the B_k slice reaches registers through LDS: direct-to-LDS loads of whole rows
//    (1 KB per instruction), 16-byte chunks XOR-swizzled by row so that the fragment
//    reads are free of bank conflicts.  Row-gathering fragment loads straight from
//    memory (16 rows x 64 bytes per instruction) cost several times more;
//  * the two rank halves of a tile meet in LDS: wave (dg, kh) finishes row tiles
//    2 kh, 2 kh + 1, rotates them (RoPE in the lane, no exchange) and scores them
//    against the query group on the MFMA (query and keys split into bf16 hi + lo parts,
//    three products); the four dim groups' partial scores of a row are added in LDS in
//    a fixed order;
//  * value rows (A_v rank chunk, or V_full dims with exact values) go to LDS with
//    direct-to-LDS loads once the A_k rows have landed, 16-byte chunks XOR-swizzled by
//    row so that the transposing reads below are free of bank conflicts;
//  * weighted value sum: P (query heads x 64 rows, hi + lo) times the 64 value rows on
//    the MFMA, the value rows read from LDS with transposing reads; wave w owns columns
//    [w W / 8, (w + 1) W / 8) of the W-wide sum, so no cross-wave reduction is needed.
// MULTI: r spans several rank chunks (the single-chunk instantiation issues every
// direct-to-LDS load outside any branch, which keeps the compiler's own waits for them
// exact).
// KPTF > 0: the block selects the head's top-k chunks itself from the scores (KPTF keys
// per thread, n_cand <= 512 KPTF), keeps the ids of its own split and writes them to
// `sel`; the selection runs while the first B_k staging is in flight.
template <bool EXACT_V, bool MULTI, int KPTF>
__global__ __launch_bounds__(512) void sr_attend_mfma_kernel(SrParams P) {
  // Region A: staged A_k rows (stride AROW); before them the B_k staging of dt = 1, after
  // them the partial-key exchange, partial scores, softmax weights and statistics.
  __shared__ __align__(16) uint16_t Ak[RBM * AROW];
  // Region V: the B_k staging of dt = 0, then the value rows (W columns each, no padding,
  // swizzled).
  __shared__ __align__(16) uint16_t Vr[RBM * VROW_MAX];
  __shared__ int rows_t[RBM];
  __shared__ int sel_s[64];                       // the split's chunk ids (KPTF > 0)
  __shared__ int tk_hist[KPTF > 0 ? NBK : 1];     // top-k scratch (KPTF > 0)
  __shared__ int tk_tmp[16];
  __shared__ int tk_bcast[4];
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int dg = wave & 3, kh = wave >> 2;
  const long bh = (long)b * P.Hkv + h;
  const int r = P.r_k, grp = P.grp;
  // Rank chunk: the largest of 512, 256, 128 that divides r.  A staged half-row of B_k
  // holds KC/2 ranks = 2^lcr chunks of 16 bytes; a rank half is nks MFMA k-steps.
  const int KC = (r & 511) == 0 ? 512 : (r & 255) == 0 ? 256 : 128;
  const int lcr = KC == 512 ? 5 : KC == 256 ? 4 : 3;
  const int nks = KC >> 6;
  // Value chunk: W columns, 2^lcv chunks of 16 bytes per row.
  const int W = EXACT_V ? 128 : KC;
  const int lcv = EXACT_V ? 4 : lcr + 1;
  const int Wtot = EXACT_V ? 128 : r;

  // ---- prologue ----
  // The single-chunk path: lane l of wave w reads the id of row 8w + (l & 7) itself
  // (unconditionally, clamped to a valid entry), so that no barrier stands between the
  // ids and the wave's A_k gathers.  The multi-chunk path reads them for the block.
  int csel = -1;
  float4 sraw[KPTF > 0 ? KPTF / 4 : 1];   // this thread's scores, raw (KPTF > 0)
  if constexpr (KPTF > 0) {
    // Past the row's end: the last 16 bytes of the row's padded stride again (ignored).
    const float* sc = P.scores + bh * P.ld_sc;
#pragma unroll
    for (int u = 0; u < KPTF / 4; ++u) sraw[u] = *(const float4*)(sc + min(tid * KPTF + 4 * u, P.ld_sc - 4));
  } else if constexpr (!MULTI) {
    const int ci = s * P.cps + (wave * 8 + (lane & 7)) / P.chunk;
    csel = P.sel[bh * P.top_k + min(ci, P.k_eff - 1)];
    if (ci >= P.k_eff) csel = -1;
  } else if (tid < RBM) {
    const int ci = s * P.cps + tid / P.chunk;
    if (ci < P.k_eff) csel = P.sel[bh * P.top_k + ci];
  }
  // Query fragment of this lane: head j = n (zero past the group), dims 16 dg + 4 g + v
  // and their RoPE partners 64 + 16 dg + 4 g + v.
  const int jq = min(n, grp - 1);
  const uint16_t* qg = (const uint16_t*)P.q + ((long)b * P.Hq + (long)h * grp + jq) * 128 + 16 * dg + 4 * g;
  uint16_t qraw[8];
  double turns[4];   // RoPE frequencies (turns per position) of this lane's dims, for q and k
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    qraw[v] = qg[v];
    qraw[4 + v] = qg[64 + v];
    turns[v] = P.turns[16 * dg + 4 * g + v];
  }
  // B_k fragments: (dt, ks) of lane (n, g) holds row 64 dt + n of the wave's 16-dim group,
  // ranks kc + kh KC/2 + 8 (4 ks + g) .. + 8.  On the selecting path those of rank chunk 0
  // are loaded straight from memory here, behind the scores, and arrive while the
  // selection runs (with a direct-to-LDS load in flight the compiler would make every LDS
  // atomic of the selection wait for it); otherwise they come through LDS below.
  const uint16_t* bk = (const uint16_t*)P.Bt_k + b * P.bs_Bt_k + (long)(h * 128 + 16 * dg) * P.ld_Bt_k;
  uint4 bq[2][8];
  if constexpr (KPTF > 0) {
#pragma unroll
    for (int dt = 0; dt < (MULTI ? 2 : 1); ++dt)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        bq[dt][ks] = *(const uint4*)(bk + (long)(64 * dt + n) * P.ld_Bt_k + kh * (KC >> 1) +
                                     8 * (4 * min(ks, nks - 1) + g));
  }
  // The keys are formed (and pinned by the empty asm statements) after those loads are
  // issued: the wait for the scores (issued first) is then a wait for them alone.
  uint32_t kr[KPTF > 0 ? KPTF : 1];
  float fv[KPTF > 0 ? KPTF : 1];
  if constexpr (KPTF > 0) {
#pragma unroll
    for (int u = 0; u < KPTF / 4; ++u) {
      fv[4 * u] = sraw[u].x;
      fv[4 * u + 1] = sraw[u].y;
      fv[4 * u + 2] = sraw[u].z;
      fv[4 * u + 3] = sraw[u].w;
    }
#pragma unroll
    for (int u = 0; u < KPTF; ++u) {
      __asm__ volatile("" : "+v"(fv[u]));
      kr[u] = order_key(fv[u]);
    }
  }
  // Selection positions [s cps, (s + 1) cps) into sel_s, the block's share of `sel`
  // written out (the last split also pads positions past its range with -1), and this
  // thread's chunk id: row 8 wave + (lane & 7) (single chunk) or row tid (multi-chunk).
  auto fused_select = [&]() __attribute__((always_inline)) {
    if constexpr (KPTF > 0) {
      const int lo = s * P.cps;
      topk_keys<KPTF, 512>(kr, fv, P.n_cand, P.top_k, lo, lo + P.cps, sel_s, tk_hist, tk_tmp, tk_bcast);
      lds_sync();
      int* sel_out = P.sel + bh * P.top_k;
      if (tid < P.cps && lo + tid < P.top_k) sel_out[lo + tid] = sel_s[tid];
      if (s == P.n_splits - 1)
        for (int ci = lo + P.cps + tid; ci < P.top_k; ci += 512) sel_out[ci] = -1;
      const int r = MULTI ? tid : wave * 8 + (lane & 7);
      const int ci = lo + min(r, RBM - 1) / P.chunk;
      csel = ci < P.k_eff ? sel_s[ci - lo] : -1;
    }
  };
  // B_k staging: half-rows (dims 16 dg + 64 dt + m, ranks kc + kh KC/2 + [0, KC/2)) of
  // this wave.  Multi-chunk: dt = 0 into its slot of region V, dt = 1 into its slot of
  // region A, together.  Single chunk: both into the region V slot in turn, so that region
  // A takes the A_k rows while the staging is under way.
  // 16-byte unit p of a slot holds row m = p >> lcr, chunk c = (p & (2^lcr - 1)) ^ (m & 7).
  // One half-row set (dt) into one slot; called with each slot's own array so that every
  // direct-to-LDS load names a single LDS array (which lets the compiler keep the loads
  // into one array from delaying reads of the other).
  auto stage_half = [&](unsigned char* slot, int dt, int kc) {
    const int ni = 1 << (lcr - 2);   // 1 KB instructions per half-row set
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = 64 * min(i, ni - 1) + lane;   // past the set: the last instruction again
      const int m = p >> lcr, c = (p & ((1 << lcr) - 1)) ^ (m & 7);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(bk + (long)(64 * dt + m) * P.ld_Bt_k + kc +
                                                           kh * (KC >> 1) + 8 * c),
          (__attribute__((address_space(3))) void*)(slot + 1024 * min(i, ni - 1)), 16, 0, 0);
    }
  };
  auto stage_b = [&](int kc) {
    stage_half((unsigned char*)Vr + wave * QSLOT, 0, kc);
    stage_half((unsigned char*)Ak + wave * 8192, 1, kc);
  };
  // Fragment (dt, ks) of lane (n, g): row n, chunk 4 ks + g (bq, declared above).
  auto read_half = [&](const unsigned char* slot, int dt) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int unit = (n << lcr) + ((4 * min(ks, nks - 1) + g) ^ (n & 7));
      bq[dt][ks] = *(const uint4*)(slot + 16 * unit);
    }
  };
  auto read_b = [&]() {
    read_half((const unsigned char*)Vr + wave * QSLOT, 0);
    read_half((const unsigned char*)Ak + wave * 8192, 1);
  };
  const int lcv_ni = 1 << (lcv - 3);   // 1 KB instructions for a wave's 8 value rows
  int tr[8], tv[8];   // A_k row of instruction i; value row of this lane in value instruction i
  unsigned char* const vslot = (unsigned char*)Vr + wave * QSLOT;
  if constexpr (!MULTI) {
    // Half the B_k staging (dt = 0) lands with the row ids; then the A_k gathers and the
    // other half (into the same slot) are in flight together.
    if constexpr (KPTF > 0) {
      fused_select();
    } else {
      stage_half(vslot, 0, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): ids, query and dt = 0 half have landed
      read_half(vslot, 0);
    }
    const int rl = wave * 8 + (lane & 7);
    const int t = csel * P.chunk + rl % P.chunk;
    const int trow = (csel >= 0 && t >= P.n_sink && t < P.T - P.n_local) ? t : -1;
    if (lane < 8) rows_t[rl] = trow;   // visible to the block after the barrier below
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tr[i] = __builtin_amdgcn_readlane(trow, i);
      tv[i] = __builtin_amdgcn_ds_bpermute(((64 * min(i, lcv_ni - 1) + lane) >> lcv) << 2, trow);
    }
  } else {
    if constexpr (KPTF > 0) {
      fused_select();
    } else {
      stage_b(0);
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the B_k slice has landed
      read_b();
    }
    if (tid < RBM) {
      const int t = csel * P.chunk + tid % P.chunk;
      rows_t[tid] = (csel >= 0 && t >= P.n_sink && t < P.T - P.n_local) ? t : -1;
    }
    lds_sync();   // the row ids are visible and every wave has read its B_k staging
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tr[i] = rows_t[wave * 8 + i];
      tv[i] = rows_t[wave * 8 + ((64 * min(i, lcv_ni - 1) + lane) >> lcv)];
    }
  }

  // Wave w gathers rows 8w .. 8w+7.  A_k rows: one row per instruction, lane l bytes
  // [16l, 16l + 16) (lanes past a narrow chunk re-read its last 16 bytes into columns
  // never read).  Value rows: 2^lcv units per row, row rho's chunk c at unit
  // rho 2^lcv + (c ^ 2 (rho & 3)), one 1 KB instruction per 64 units (repeated past the
  // wave's rows: the same bytes to the same place).  Absent rows (-1) load row 0 and are
  // masked later, so that every load is unconditional.
  const uint16_t* Ag_k = (const uint16_t*)P.A_k + b * P.bs_A_k;
  auto load_rows = [&](int kc) {
    const int col = min(lane * 8, KC - 8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(Ag_k + (long)max(tr[i], 0) * P.ld_A_k + kc + col),
          (__attribute__((address_space(3))) void*)(Ak + (wave * 8 + i) * AROW), 16, 0, 0);
  };
  auto load_vrows = [&](int kc) {
    const uint16_t* src;
    long ld;
    if constexpr (EXACT_V) {
      src = (const uint16_t*)P.V_full + b * P.bs_V + (long)h * 128;
      ld = P.ld_V;
    } else {
      src = (const uint16_t*)P.A_v + b * P.bs_A_v + kc;
      ld = P.ld_A_v;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = 64 * min(i, lcv_ni - 1) + lane;   // unit within the wave's rows
      const int rho = wave * 8 + (p >> lcv);
      const int c = (p & ((1 << lcv) - 1)) ^ (2 * (rho & 3));
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src + (long)max(tv[i], 0) * ld + 8 * c),
          (__attribute__((address_space(3))) void*)((unsigned char*)Vr + (wave * 8 << (lcv + 4)) +
                                                     1024 * min(i, lcv_ni - 1)),
          16, 0, 0);
    }
  };
  if constexpr (!MULTI) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the slot has been read
    stage_half(vslot, 1, 0);              // the dt = 1 half into the same slot
  }
  load_rows(0);

  // While the rows stream in: rotate the query fragment at the query position, scale it
  // and split it into bf16 hi + lo operands (zero for lanes past the group).
  bf16x8_t qhi, qlo;
  {
    float qf[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float c, sn;
      rope_cs_turns(P.q_pos, turns[v], &c, &sn);
      const float x = bf16_bits_to_f32(qraw[v]), y = bf16_bits_to_f32(qraw[4 + v]);
      const float keep = n < grp ? P.scale : 0.f;
      qf[v] = (x * c - y * sn) * keep;
      qf[4 + v] = (y * c + x * sn) * keep;
    }
    split_bf16x8(qf, qhi, qlo);
  }

  // ---- keys: K^T tiles over the rank chunks ----
  f32x4_t acc[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) acc[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // The staged rows' fragments are read one k-step ahead of the MFMAs that use them.
  auto kphase = [&]() {
    const uint16_t* abase = Ak + n * AROW + kh * (KC >> 1) + 8 * g;
    uint4 an[4], ac[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) an[rt] = *(const uint4*)(abase + rt * 16 * AROW);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < nks) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) ac[rt] = an[rt];
        if (ks + 1 < nks) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) an[rt] = *(const uint4*)(abase + rt * 16 * AROW + 32 * (ks + 1));
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          acc[rt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bq[0][ks]), as_bf16x8(ac[rt]), acc[rt][0], 0, 0, 0);
          acc[rt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bq[1][ks]), as_bf16x8(ac[rt]), acc[rt][1], 0, 0, 0);
        }
      }
    }
  };
  if constexpr (!MULTI) {
    // The value rows go out once the A_k rows have landed: with both gathers in flight
    // together the A_k rows land no earlier than the value rows; this way they have the
    // memory system first, and the value rows land while the keys and scores are formed.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the A_k rows and the dt = 1 half have landed
    read_half(vslot, 1);
    lds_sync();   // the row ids are visible and every wave has read its B_k staging
    load_vrows(0);
    kphase();
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_sync();
    kphase();
    for (int kc = KC; kc < r; kc += KC) {
      lds_sync();   // every wave is done with the previous chunk's rows
      stage_b(kc);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      read_b();
      lds_sync();   // the B_k staging has been read by every wave
      load_rows(kc);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_sync();
      kphase();
    }
    lds_sync();   // region V is free: the value rows of the first chunk
    load_vrows(0);
  }
  lds_sync();   // every wave is done reading the A_k rows

  // ---- the two rank halves meet: wave (dg, kh) takes row tiles 2 kh and 2 kh + 1 ----
  // (tiles picked with selects on the wave-uniform kh, so that the accumulators stay in
  // registers)
  f32x4_t mine[2][2];
  {
    float4* X = (float4*)Ak;   // [sender wave][tile u][dt][lane], 32 KB
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const f32x4_t a = kh ? acc[u][dt] : acc[2 + u][dt];
        mine[u][dt] = kh ? acc[2 + u][dt] : acc[u][dt];
        X[((wave * 2 + u) * 2 + dt) * 64 + lane] = make_float4(a[0], a[1], a[2], a[3]);
      }
    lds_sync();
    const int partner = wave ^ 4;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const float4 o = X[((partner * 2 + u) * 2 + dt) * 64 + lane];
        mine[u][dt][0] += o.x;
        mine[u][dt][1] += o.y;
        mine[u][dt][2] += o.z;
        mine[u][dt][3] += o.w;
      }
  }

  // ---- RoPE on the keys of this wave's tiles, then partial scores on the MFMA ----
  // Lane (n, g) holds row rt*16 + n (rt = 2 kh + u), dims i = 16 dg + 4 g + v
  // (mine[u][0][v]) and i + 64 (mine[u][1][v]).  Behind the exchange in region A:
  // sp[dg][j][row] (partial scores), pw[j][row] (weights), the statistics.  The score
  // stores are unconditional (heads past the group land in unused slots), which keeps
  // them free of waits for the value rows in flight.
  float* sp = (float*)Ak + 8192;      // [4 dim groups][16 heads][64 rows] (heads past the group unused)
  float* pw = sp + 4 * 16 * RBM;
  float* st_m = pw + MAXG * RBM;
  float* st_l = st_m + MAXG;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int rt = 2 * kh + u;
    const int t = max(rows_t[rt * 16 + n], 0);   // absent rows: angle 0, masked below
    float kf[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float c, sn;
      rope_cs_turns(t, turns[v], &c, &sn);
      const float x = mine[u][0][v], y = mine[u][1][v];
      kf[v] = x * c - y * sn;
      kf[4 + v] = y * c + x * sn;
    }
    bf16x8_t khi, klo;
    split_bf16x8(kf, khi, klo);
    f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, khi, sc, 0, 0, 0);
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, klo, sc, 0, 0, 0);
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo, khi, sc, 0, 0, 0);
    // sc[v] = partial score of query head 4g + v for row rt*16 + n
#pragma unroll
    for (int v = 0; v < 4; ++v) sp[(dg * 16 + 4 * g + v) * RBM + rt * 16 + n] = sc[v];   // unconditional
  }
  lds_sync();   // partial scores visible

  // ---- softmax of the summed scores (wave j < group size: query head j) ----
  if (wave < grp) {
    float v = -INFINITY;
    if (rows_t[lane] >= 0) v = ((sp[(0 * 16 + wave) * RBM + lane] + sp[(1 * 16 + wave) * RBM + lane]) +
                                sp[(2 * 16 + wave) * RBM + lane]) + sp[(3 * 16 + wave) * RBM + lane];
    const float mx = wave_max(v);
    const float p = (v == -INFINITY) ? 0.f : __expf(v - mx);
    const float l = wave_sum(p);
    // absent rows: weight 0 (their value rows hold row 0's values)
    pw[wave * RBM + lane] = p;
    if (lane == 0) {
      st_m[wave] = mx;
      st_l[wave] = l;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's value rows have landed
  lds_sync();

  // ---- weighted value sum: O[j][col] = sum_row P[j][row] V[row][col] ----
  // A operand: P (head j = n, rows 32 ks + 8 g .. + 8), hi + lo; B operand: value rows
  // 32 ks + 8 g .. + 8 at column col0 + n, two transposing reads of 4 rows each.
  bf16x8_t phi[2], plo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float pf[8];
    const float4 p0 = *(const float4*)&pw[jq * RBM + 32 * ks + 8 * g];
    const float4 p1 = *(const float4*)&pw[jq * RBM + 32 * ks + 8 * g + 4];
    const float keep = n < grp ? 1.f : 0.f;
    pf[0] = p0.x * keep; pf[1] = p0.y * keep; pf[2] = p0.z * keep; pf[3] = p0.w * keep;
    pf[4] = p1.x * keep; pf[5] = p1.y * keep; pf[6] = p1.z * keep; pf[7] = p1.w * keep;
    split_bf16x8(pf, phi[ks], plo[ks]);
  }
  float* part = P.part + (bh * P.n_splits + s) * (long)grp * (2 + Wtot);
  const int cw = W >> 3;   // columns per wave, a multiple of 16
  for (int kc = 0; kc < Wtot; kc += W) {
    if constexpr (MULTI) {
      if (kc > 0) {   // a further rank chunk of A_v (ranks above the first chunk)
        lds_sync();   // the previous chunk's value rows are read
        load_vrows(kc);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_sync();
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (16 * ct < cw) {
        const int col0 = wave * cw + 16 * ct;
        f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // lane (n, g) reads row rho = 32 ks + 8 g + (n >> 2) (and rho + 4), columns
          // col0 + 4 (n & 3) .. + 4: chunk cc, half n & 1
          const int rho = 32 * ks + 8 * g + (n >> 2);
          const int cc = (col0 >> 3) + ((n & 3) >> 1);
          const unsigned char* src =
              (const unsigned char*)Vr + ((rho << lcv) + (cc ^ (2 * (rho & 3)))) * 16 + 8 * (n & 1);
          union {
            v4s hv[2];
            bf16x8_t bv;
          } u;
          u.hv[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)src);
          u.hv[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(src + (4 << (lcv + 4))));
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[ks], u.bv, o, 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[ks], u.bv, o, 0, 0, 0);
        }
        // o[v] = O[4g + v][col0 + n]
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (4 * g + v < grp) part[2 * grp + (long)(4 * g + v) * Wtot + kc + col0 + n] = o[v];
      }
    }
  }
  if (tid < grp) {
    part[tid] = st_m[tid];
    part[grp + tid] = st_l[tid];
  }
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

  split_rows(P, bh, s, RB, rows_t);
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

// Merge of (b, h)'s split partials and exact-row partials by their log-sum-exp
// weights.  Partial q < n_splits is a split, the rest are exact-row tiles.  The
// headers are read in one parallel round into LDS; every output element then sums
// its partials with the loads of a batch issued together.
// Value-space merge, one block per (query head, sequence): phase 1 forms the weights
// exp(m_q - M) of the split and exact-tile partials and the denominator; phase 2 sums
// the weighted partial outputs, groups of partials over lanes of float4 dims.
__global__ __launch_bounds__(256) void sr_merge_kernel(SrParams P) {
  __shared__ float wq[MAXP];
  __shared__ float red_m[4], red_l[4];
  __shared__ __align__(16) float4 acc_s[16][32];
  const int qh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = P.grp, d = P.d, h = qh / grp, j = qh % grp;
  const int np = P.n_splits + P.n_exact;
  const long bh = (long)b * P.Hkv + h;
  const long stride = (long)grp * (2 + d);
  const float* p0 = P.part + bh * P.n_splits * stride;
  const float* pex = P.part_ex + bh * P.n_exact * stride;
  auto part = [&](int q) -> const float* { return q < P.n_splits ? p0 + q * stride : pex + (q - P.n_splits) * stride; };
  float m[2], l[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = min(tid + 256 * u, np - 1);   // past np: the last partial again, not used
    m[u] = part(q)[j];
    l[u] = part(q)[grp + j];
    if (tid + 256 * u >= np) {
      m[u] = -INFINITY;
      l[u] = 0.f;
    }
  }
  float mx = wave_max(fmaxf(m[0], m[1]));
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  float ls = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float w = (m[u] == -INFINITY) ? 0.f : __expf(m[u] - M);
    if (tid + 256 * u < np) wq[tid + 256 * u] = w;
    ls += w * l[u];
  }
  ls = wave_sum(ls);
  if (lane == 0) red_l[wave] = ls;
  __syncthreads();
  const float L = (red_l[0] + red_l[1]) + (red_l[2] + red_l[3]);
  const int nc4 = d >> 2, nsg = 256 / nc4;   // float4 columns, partial groups
  const int c4 = tid % nc4, sg = tid / nc4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int NB = 8;
  for (int q0 = sg; q0 < np; q0 += nsg * NB) {
    float4 v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = *(const float4*)(part(min(q0 + nsg * u, np - 1)) + 2 * grp + (long)j * d + 4 * c4);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (q0 + nsg * u < np) {
        const float w = wq[q0 + nsg * u];
        acc.x += w * v[u].x;
        acc.y += w * v[u].y;
        acc.z += w * v[u].z;
        acc.w += w * v[u].w;
      }
  }
  acc_s[sg][c4] = acc;
  __syncthreads();
  if (tid < nc4) {
    float4 r = acc_s[0][tid];
    for (int g = 1; g < nsg; ++g) {
      r.x += acc_s[g][tid].x;
      r.y += acc_s[g][tid].y;
      r.z += acc_s[g][tid].z;
      r.w += acc_s[g][tid].w;
    }
    const float inv = 1.f / L;
    float* o = P.out + ((long)b * P.Hq + qh) * d + 4 * tid;
    o[0] = r.x * inv;
    o[1] = r.y * inv;
    o[2] = r.z * inv;
    o[3] = r.w * inv;
  }
}

// Merge for the matrix-core path, one block per (KV head h, query head j of its group,
// sequence b): split partials carry sum_t p_t A_v[t] (rank space), exact-row tiles carry
// sum_t p_t v_t.  out = (sum_s w_s o_s) B_v,l,h + sum_e w_e o_e, over the weighted sum
// of denominators.  The headers, the first 32 split partials of the thread's two rank
// columns and the first 512 rank columns of the wave's 32 rows of B_v are all in flight
// before anything waits.
// Grid: KV heads x (query heads per group x MQ dim slices) x batch.  Block (h, j, q)
// merges query head j's partials into the rank-space sum and writes output dims
// [q d/MQ, (q + 1) d/MQ): more, smaller blocks than one per query head, so that the
// partial and B_v reads of a layer spread over MQ times more compute units.
constexpr int MQ = 4;
__global__ __launch_bounds__(256) void sr_merge_rank_kernel(SrParams P) {
  __shared__ float wq[MAXP_RANK];
  __shared__ float lq[MAXP_RANK];
  __shared__ float run_l;
  __shared__ __align__(16) float orank[MAX_RANK_MFMA];
  __shared__ float oval[MAXD / MQ];
  const int h = blockIdx.x, j = blockIdx.y / MQ, dq = blockIdx.y % MQ, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = P.grp, d = P.d, r = P.r_v;
  const int dd = d / MQ;           // output dims of this block
  const int ns = P.n_splits, np = ns + P.n_exact;
  const long bh = (long)b * P.Hkv + h;
  const long sstride = (long)grp * (2 + r), estride = (long)grp * (2 + d);
  const float* p0 = P.part + bh * ns * sstride + 2 * grp + (long)j * r;   // split q: p0[q * sstride + c]
  const float* pex = P.part_ex + bh * P.n_exact * estride;
  // Wave w takes output dims dq*dd + w*dd/4 + u (u < dd/4 <= 8), lane l rank columns
  // [8l, 8l + 8) of every 512.
  const int dw = dd / 4;
  const uint16_t* Bt = (const uint16_t*)P.Bt_v + b * P.bs_Bt_v + (long)(h * d + dq * dd + wave * dw) * P.ld_Bt_v;

  constexpr int HU = (MAXP_RANK + 255) / 256;
  float hw[HU], hl[HU];
#pragma unroll
  for (int u = 0; u < HU; ++u) {
    const int q = tid + 256 * u;
    if (q < np) {
      const float* pq = q < ns ? P.part + (bh * ns + q) * sstride : pex + (q - ns) * estride;
      hw[u] = pq[j];
      hl[u] = pq[grp + j];
    }
  }
  constexpr int PF = 32;
  const int c0 = min(2 * tid, r - 2);   // threads past r duplicate the last pair (unused)
  float2 pv[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) pv[u] = *(const float2*)(p0 + (long)max(0, min(u, ns - 1)) * sstride + c0);
  // The exact-row tiles' weighted value sums of this block's output dim tid (up to 16
  // tiles, 256 exact rows, in flight).
  constexpr int PE = 16;
  float ev[PE];
#pragma unroll
  for (int e = 0; e < PE; ++e)
    ev[e] = (tid < dd && e < P.n_exact) ? pex[e * estride + 2 * grp + (long)j * d + dq * dd + tid] : 0.f;
  uint4 bw[8];
  const int cb = min(lane * 8, r - 8);
#pragma unroll
  for (int u = 0; u < 8; ++u) bw[u] = *(const uint4*)(Bt + (long)min(u, dw - 1) * P.ld_Bt_v + cb);
#pragma unroll
  for (int u = 0; u < HU; ++u) {
    const int q = tid + 256 * u;
    if (q < np) {
      wq[q] = hw[u];
      lq[q] = hl[u];
    }
  }
  __syncthreads();
  if (wave == 0) {
    float M = -INFINITY;
    for (int q = lane; q < np; q += 64) M = fmaxf(M, wq[q]);
    M = wave_max(M);
    float L = 0.f;
    for (int q = lane; q < np; q += 64) {
      const float w = (wq[q] == -INFINITY) ? 0.f : __expf(wq[q] - M);
      wq[q] = w;
      L += w * lq[q];
    }
    L = wave_sum(L);
    if (lane == 0) run_l = L;
  }
  __syncthreads();
  // Combined rank-space sum of columns c0, c0 + 1 (and, for r > 512, further pairs),
  // the splits added in order.
  {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (u < ns) {
        a0 += wq[u] * pv[u].x;
        a1 += wq[u] * pv[u].y;
      }
    for (int q = PF; q < ns; ++q) {
      const float2 v = *(const float2*)(p0 + (long)q * sstride + c0);
      a0 += wq[q] * v.x;
      a1 += wq[q] * v.y;
    }
    if (2 * tid < r) {
      orank[c0] = a0;
      orank[c0 + 1] = a1;
    }
  }
  for (int c = 2 * tid + 512; c < r; c += 512) {
    float a0 = 0.f, a1 = 0.f;
    for (int q = 0; q < ns; ++q) {
      const float2 v = *(const float2*)(p0 + (long)q * sstride + c);
      a0 += wq[q] * v.x;
      a1 += wq[q] * v.y;
    }
    orank[c] = a0;
    orank[c + 1] = a1;
  }
  if (tid < dd) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < PE; ++e)
      if (e < P.n_exact) acc += wq[ns + e] * ev[e];
    for (int e = PE; e < P.n_exact; ++e) acc += wq[ns + e] * pex[e * estride + 2 * grp + (long)j * d + dq * dd + tid];
    oval[tid] = acc;
  }
  __syncthreads();
  // out[i] = orank . Bt_v[h*d + i] + oval[i]: each lane's partial over its rank columns,
  // then a wave-wide sum per output dim.
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  for (int c = lane * 8; c < r; c += 512) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = orank[c + e];
    if (c >= 512) {
#pragma unroll
      for (int u = 0; u < 8; ++u) bw[u] = *(const uint4*)(Bt + (long)min(u, dw - 1) * P.ld_Bt_v + c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t w[4] = {bw[u].x, bw[u].y, bw[u].z, bw[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[u] += o[2 * e] * __uint_as_float(w[e] << 16);
        acc[u] += o[2 * e + 1] * __uint_as_float(w[e] & 0xffff0000u);
      }
    }
  }
  // lanes past r (r < 512) hold partials of re-read columns: left out of the sum
  const bool live = lane * 8 < r;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float sum = wave_sum(live ? acc[u] : 0.f);
    if (u < dw && lane == 0) {
      const int i = wave * dw + u;
      P.out[((long)b * P.Hq + (long)h * grp + j) * d + dq * dd + i] = (sum + oval[i]) / run_l;
    }
  }
}

template <int KPT>
__global__ __launch_bounds__(TKT) void topk_rows_kernel(const float* scores, int n_cand, long ld, int k, int* sel) {
  __shared__ int hist[NBK];
  __shared__ int tmp[2 * (TKT / 64)];
  __shared__ int bcast[4];
  uint32_t kr[KPT];
  float fv[KPT];
  load_keys<KPT>(scores + blockIdx.x * ld, n_cand, kr);
#pragma unroll
  for (int u = 0; u < KPT; ++u) fv[u] = key_value(kr[u]);
  topk_keys<KPT, TKT>(kr, fv, n_cand, k, 0, k, sel + (long)blockIdx.x * k, hist, tmp, bcast);
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

// KV head fastest in the grid: consecutive blocks go to different XCDs, so with 8 KV
// heads one head's score blocks share an XCD, and the blocks that select the head's
// top-k find its scores in that XCD's L2.  The exact-row tiles come first in the grid.
template <typename ST>
hipError_t launch_score_st(const SrParams& P, hipStream_t st) {
  // the exact tiles' staged rows (keys, then values), queries, weights, softmax stats and
  // RoPE frequencies
  const size_t lds = sizeof(float) * (ETR * EROW + MAXG * MAXD + MAXG * ETR + 2 * MAXG) + sizeof(double) * (MAXD / 2);
  hipError_t e = set_lds<1 + (int)sizeof(ST)>(sr_score_kernel<ST>, lds);
  if (e != hipSuccess) return e;
  const dim3 grid(P.Hkv, P.n_exact + P.score_blocks, P.batch);
  hipLaunchKernelGGL(sr_score_kernel<ST>, grid, dim3(256), lds, st, P);
  return hipGetLastError();
}

hipError_t launch_sr_score(const SrParams& P, int bf16, hipStream_t st) {
  return bf16 ? launch_score_st<uint16_t>(P, st) : launch_score_st<float>(P, st);
}

// Top-k selection, one block per (head, sequence), unless the attend kernel selects
// (or nothing is selected).
hipError_t launch_sr_topk(const SrParams& P, int bf16, hipStream_t st) {
  (void)bf16;
  if (P.fuse_topk || P.k_eff == 0) return hipSuccess;
  const dim3 grid(P.Hkv * P.batch);
  if (P.n_cand <= TKT * 2)
    hipLaunchKernelGGL(sr_topk_kernel<2>, grid, dim3(TKT), 0, st, P);
  else if (P.n_cand <= TKT * 8)
    hipLaunchKernelGGL(sr_topk_kernel<8>, grid, dim3(TKT), 0, st, P);
  else
    hipLaunchKernelGGL(sr_topk_kernel<32>, grid, dim3(TKT), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_sr_attend(const SrParams& P, int bf16, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (P.n_splits == 0) {
    if (ev_start) {
      hipError_t e = hipEventRecord(ev_start, st);
      if (e == hipSuccess) e = hipEventRecord(ev_stop, st);
      return e;
    }
    return hipSuccess;
  }
  dim3 grid(P.Hkv, P.n_splits, P.batch);
  if (P.mfma) {
    // The timing events, when given, are stamped by the dispatch itself at the
    // kernel's start and end.
    const bool multi = (P.r_k & 511) ? P.r_k > ((P.r_k & 255) ? 128 : 256) : P.r_k > 512;
    const int kptf = !P.fuse_topk ? 0 : P.n_cand <= 512 * 16 ? 16 : 32;
#define XKV_ATTEND(EV, MU, KP) \
  hipExtLaunchKernelGGL(sr_attend_mfma_kernel<EV, MU, KP>, grid, dim3(512), 0, st, ev_start, ev_stop, 0, P)
#define XKV_ATTEND_K(EV, MU) \
  do {                                   \
    if (kptf == 16)                      \
      XKV_ATTEND(EV, MU, 16);            \
    else if (kptf == 32)                 \
      XKV_ATTEND(EV, MU, 32);            \
    else                                 \
      XKV_ATTEND(EV, MU, 0);             \
  } while (0)
    if (P.exact_v) {
      if (multi)
        XKV_ATTEND_K(true, true);
      else
        XKV_ATTEND_K(true, false);
    } else {
      if (multi)
        XKV_ATTEND_K(false, true);
      else
        XKV_ATTEND_K(false, false);
    }
#undef XKV_ATTEND_K
#undef XKV_ATTEND
  } else {
    hipError_t e;
    if (ev_start && (e = hipEventRecord(ev_start, st)) != hipSuccess) return e;
    if (bf16)
      hipLaunchKernelGGL(sr_attend_generic_kernel<uint16_t>, grid, dim3(256), 0, st, P);
    else
      hipLaunchKernelGGL(sr_attend_generic_kernel<float>, grid, dim3(256), 0, st, P);
    if (ev_stop && (e = hipEventRecord(ev_stop, st)) != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_sr_merge(const SrParams& P, hipStream_t st) {
  if (P.mfma && !P.exact_v)
    hipLaunchKernelGGL(sr_merge_rank_kernel, dim3(P.Hkv, P.grp * MQ, P.batch), dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL(sr_merge_kernel, dim3(P.Hq, P.batch), dim3(256), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int rows, int n_cand, long ld, int k, int* sel, hipStream_t st) {
  if (n_cand <= TKT * 2)
    hipLaunchKernelGGL(topk_rows_kernel<2>, dim3(rows), dim3(TKT), 0, st, scores, n_cand, ld, k, sel);
  else if (n_cand <= TKT * 8)
    hipLaunchKernelGGL(topk_rows_kernel<8>, dim3(rows), dim3(TKT), 0, st, scores, n_cand, ld, k, sel);
  else
    hipLaunchKernelGGL(topk_rows_kernel<32>, dim3(rows), dim3(TKT), 0, st, scores, n_cand, ld, k, sel);
  return hipGetLastError();
}

// The decode scratch of xkv_sr_decode_layers_noalloc: one array per GPU, in the
// library's code object.  Host code never uses the array's name as an address (on
// the host it only stands for the symbol); the address on each device comes from
// hipGetSymbolAddress, looked up once per device with that device current.
namespace {
__device__ __align__(256) unsigned char scratch[kSrScratchBytes];
std::mutex scratch_mu;
void* scratch_dev[kSrScratchDevices] = {};
}  // namespace

hipError_t sr_scratch_setup(int device) {
  if (device < 0 || device >= kSrScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[device]) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  scratch_dev[device] = p;
  return hipSuccess;
}

void* sr_scratch_ptr(int device) {
  if (device < 0 || device >= kSrScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  return scratch_dev[device];
}

}  // namespace xkv
