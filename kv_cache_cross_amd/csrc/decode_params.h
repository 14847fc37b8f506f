// Kernel-argument block of the Selective Reconstruction decode kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace xkv {

constexpr int MAX_RANK_MFMA = 4096;

struct SrParams {
  int batch, Hq, Hkv, d, T, n_gen, chunk, top_k, n_sink, n_local, r_k, r_v;
  int n_cand;        // candidate chunks (not wholly inside the local window)
  int n_chunks;      // T / chunk (landmark rows per head)
  int k_eff;         // min(top_k, n_cand)
  int n_splits;      // 64-row splits of the selected rows
  int n_exact;       // 16-row tiles of the exact tail (sink + local + generated), at least 1
  int grp;           // query heads per KV head
  int mfma;          // matrix-core attend path (bf16, head_dim 128, r_k % 128 == 0,
                     // r_k <= MAX_RANK_MFMA, r_v == r_k or r_v == 0)
  int exact_v;       // on that path with r_v == 0: partials hold sum_t p_t v_t (value space);
                     // otherwise they hold sum_t p_t A_v[t] (rank space) and the merge
                     // applies B_v once
  int vdim;          // width of a split partial's weighted sum: r_v in rank space, else d
  int cps;           // chunks per split
  long q_pos;        // query position p
  int score_blocks;  // select-kernel blocks per KV head
  int ld_sc;         // row stride of `scores`: n_cand rounded up to a multiple of 4
  int fuse_topk;     // every attend block selects the head's top-k chunks itself (no separate
                     // top-k launch): the combined entry points on the matrix-core path with
                     // n_cand <= 16384 and an attend grid within the device's compute units
  float scale;
  double theta;
  double turns[64];  // theta^(-2i/d) / (2 pi) for i < d/2, formed on the host in float64
  const void* q;
  const void* A_k; long ld_A_k, bs_A_k;
  const void* Bt_k; long ld_Bt_k, bs_Bt_k;
  const void* A_v; long ld_A_v, bs_A_v;
  const void* Bt_v; long ld_Bt_v, bs_Bt_v;
  const void* V_full; long ld_V, bs_V;
  const void* lm; long bs_lm;
  void* k_tail; void* v_tail; long ld_tail, bs_tail;
  const void* k_new; const void* v_new; long bs_new;
  float* out;
  int* sel;          // batch x Hkv x top_k
  float* scores;     // batch x Hkv rows of ld_sc (n_cand used)
  float* part;       // batch x Hkv x n_splits x grp x (2 + vdim): max, sum, weighted sum
  float* part_ex;    // batch x Hkv x n_exact x grp x (2 + d)
};

// Stream-ordered stages of one decode step: exact rows + scores (+ append), top-k
// (unless the attend kernel selects), rebuild + attend of the selected rows, merge.
hipError_t launch_sr_score(const SrParams& P, int bf16, hipStream_t st);
hipError_t launch_sr_topk(const SrParams& P, int bf16, hipStream_t st);
// ev_start / ev_stop (optional, both or neither): timing events stamped at the attend
// kernel's start and end.
hipError_t launch_sr_attend(const SrParams& P, int bf16, hipStream_t st, hipEvent_t ev_start = nullptr,
                            hipEvent_t ev_stop = nullptr);
hipError_t launch_sr_merge(const SrParams& P, hipStream_t st);

}  // namespace xkv
