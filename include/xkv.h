/*
 * xkv.h -- C ABI of libxkv: cross-layer low-rank KV-cache compression (xKV)
 * and Selective Reconstruction (SR) decode attention on AMD Instinct MI355X
 * (gfx950).
 *
 * What the library computes (sources are the published pages, by title):
 *
 *  - Compression of one group side ("xKV: Cross-Layer KV-Cache Compression via
 *    Aligned Singular Vector Extraction", abstract; the xKV blog explainer,
 *    section on what xKV does).  The keys (or values) of G adjacent layers are
 *    concatenated horizontally into X (T x n, n = G*d_kv) and factored once:
 *    V_r = top-r right singular vectors of X, taken as the top-r eigenvectors
 *    of the uncentred Gram C = X^T X (KV-CoRE, section 2.A).  The shared token
 *    basis is A = X V_r (T x r); layer l is rebuilt as A B_l with B = V_r^T
 *    and B_l its l-th column slice of width d_kv.  Keys are compressed before
 *    RoPE and rotated after reconstruction (KQ-SVD, section 2, the ShadowKV
 *    precedent).
 *  - Selective Reconstruction decode (xKV blog, section on Selective
 *    Reconstruction): a landmark-guided top-k chunk selector picks chunks per
 *    KV head, only their rows are rebuilt, and attention runs over those rows
 *    plus exact sink / local-window / generated rows
 *    (h = softmax(q K^T / sqrt(d)) V, KQ-SVD section 3.2).
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked (host).  Matrices are
 *    row-major with the stated leading dimension (in elements).
 *  - The caller owns all memory, including the workspace.  The library never
 *    allocates or frees device memory and keeps no pointer after a call
 *    returns; its only device memory is the fixed decode scratch of
 *    xkv_sr_decode_layers_noalloc, part of its code object.  A context owns
 *    host-side resources only (pinned staging for
 *    the Rayleigh-Ritz round trip, host solver threads, and the solvers'
 *    working memory, ~27 MB per side at r = 512, G d_kv = 4096, kept until
 *    xkv_ctx_destroy so that later compressions reuse it).
 *  - Work is enqueued on the caller's HIP stream (passed as void*; NULL is
 *    the default stream).  Arguments are validated before anything is
 *    enqueued; a failed validation enqueues nothing.
 *  - Return codes are XKV_OK or a negative XKV_E* code; xkv_last_error()
 *    returns a message for the last failure on the calling thread.  No C++
 *    exception crosses this interface.
 *  - A context is used by one host thread at a time.
 *  - dtype XKV_BF16: every KV input and every compressed output is bfloat16;
 *    XKV_F32: float32.  Queries share the dtype; decode outputs are float32.
 *  - RoPE is the rotate-half form on pairs (i, i + d/2) with frequency
 *    theta^(-2i/d); angles are formed in float64.
 */
#ifndef XKV_H
#define XKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  XKV_OK = 0,
  XKV_EINVAL = -1,        /* bad argument (null, size, stride, alignment)           */
  XKV_EUNSUPPORTED = -2,  /* shape or device outside what the kernels implement     */
  XKV_EWORKSPACE = -3,    /* ws_bytes smaller than the matching *_ws_size query      */
  XKV_EHIP = -4,          /* a HIP runtime call failed (message has the HIP string) */
  XKV_ENUMERIC = -5,      /* Cholesky breakdown or non-finite value in the iteration */
  XKV_ENOTCONV = -6       /* subspace error estimate above tol after max_rounds; outputs written */
};

enum xkv_dtype { XKV_F32 = 0, XKV_BF16 = 1 };

typedef struct xkv_ctx_s* xkv_ctx;

/* Library version (major*10000 + minor*100 + patch). */
int xkv_version(void);

/* Create a context bound to HIP device `device`; `host_threads` bounds the
 * threads used for the host Rayleigh-Ritz eigenvalue solves (<= 0: 16).  On success *out receives the context. */
int xkv_ctx_create(int device, int host_threads, xkv_ctx* out);
void xkv_ctx_destroy(xkv_ctx ctx);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* xkv_last_error(void);

/* ------------------------------------------------------------------------ */
/* Compression of group sides                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
  int T;              /* tokens in the prefix; > 0                                    */
  int G;              /* layers per group; 1..16                                      */
  int d_kv;           /* columns per layer (n_kv_heads * head_dim); multiple of 8     */
  int r;              /* rank; 1 <= r <= G*d_kv                                       */
  int dtype;          /* enum xkv_dtype of the layers and of A, Bt, landmarks        */
  int n_kv_heads;     /* landmark layout; d_kv == n_kv_heads * head_dim              */
  int head_dim;       /* even                                                         */
  int chunk;          /* tokens per chunk; T % chunk == 0 when landmarks are asked   */
  double rope_theta;  /* RoPE base for the landmarks (10000 in every workload)       */
  int oversample;     /* p: iteration block k_b = r + p (capped at G*d_kv); < 0 -> r/2 */
  int fp32_iters;     /* subspace iterations on a float32 copy of C (>= 0)           */
  int fp64_iters;     /* trailing float64 iterations (>= 1)                          */
  uint64_t seed;      /* seed of the Gaussian start block                            */
  double tol;         /* target for the estimated ||P - P_exact||_F of V_r (0 -> 1e-4); see below */
  int max_rounds;     /* Rayleigh-Ritz rounds before XKV_ENOTCONV (0 -> 8)           */
} xkv_compress_desc;

typedef struct {
  const void* const* layers; /* (host) G device pointers; layer l is T x d_kv, row stride ld_layer */
  long ld_layer;             /* >= d_kv; for bf16 a multiple of 8                                  */
  void* A;                   /* T x r, row stride r: A = X V_r                                     */
  void* Bt;                  /* n x r, row stride r: Bt = V_r = B^T; B_l^T = rows [l*d_kv, (l+1)*d_kv) */
  void* landmarks;           /* G x n_kv_heads x (T/chunk) x head_dim means of post-RoPE keys,   */
                             /* or NULL (no landmarks: the value side)                           */
  double* eigvals;           /* (host) r leading Ritz values of C, descending; nullable          */
  double* Vr64;              /* nullable: n x r float64 copy of V_r before rounding to dtype     */
  double* stats;             /* (host) nullable, 5 entries: estimated ||P - P_exact||_F, relative */
                             /* Ritz gap (theta_r - theta_r+1)/theta_r, sweeps, rounds, and the   */
                             /* total energy trace(C) = ||X||_F^2 (the sum of all eigenvalues)    */
} xkv_side;

/* Workspace bytes needed by xkv_compress_sides for `n_sides` sides. */
int xkv_compress_ws_size(const xkv_compress_desc* desc, int n_sides, size_t* bytes);

/* Factor `n_sides` independent group sides of identical shape.
 * Steps (sides batched): Gram C = X^T X (bf16 MFMA, float64 totals) ->
 * block subspace iteration Y = C Q with CholeskyQR orthonormalisation ->
 * Rayleigh-Ritz H = Q^T C Q (float64) -> eigenvalues of H on the host (plain
 * C: Householder reduction, shared by two threads per side when k_b >= 256 and
 * host threads allow, then implicit QR whose plane rotations are logged) ->
 * the wanted eigenvectors Z_r on the GPU (the logged rotations applied to unit
 * vectors, for k_b >= 256 in 2 or 4 pieces side by side that float64 products
 * then multiply together, then the reflectors as compact-WY products) -> V_r = Q Z_r ->
 * A = X V_r and the landmarks.  With 4 or more sides the sides go in two
 * halves (the larger first), so that the GPU steps of the second half run while
 * the host solves the first half's eigenvalues.  A side's results do not depend
 * on how many sides share the call.  Allocates the rotation logs' pinned staging
 * and device copy in the context (kept and grown between calls).
 * Convergence: after each Rayleigh-Ritz round the Ritz residuals
 * r_i = C v_i - theta_i v_i give the estimate
 * sqrt(2 sum_i ||r_i||^2 / (theta_i - theta_{r+1})^2) of ||P - P_exact||_F
 * (P = V_r V_r^T; a per-pair sin-theta bound); rounds with more float64
 * sweeps run until it is <= tol or max_rounds is reached (XKV_ENOTCONV, with
 * every output written).  A block that spans all n columns is exact.
 * Blocks the calling thread once per round, for the Rayleigh-Ritz round trip;
 * the projection is enqueued on `stream` when the call returns.
 * XKV_ENUMERIC if a Cholesky pivot falls below 1e-14 of its column's squared
 * norm (e.g. X has rank < k_b). */
int xkv_compress_sides(xkv_ctx ctx, const xkv_compress_desc* desc, int n_sides,
                       const xkv_side* sides, void* ws, size_t ws_bytes, void* stream);

/* One group side: xkv_compress_sides with n_sides = 1. */
int xkv_compress_group(xkv_ctx ctx, const xkv_compress_desc* desc, const xkv_side* side,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Tokens appended after a compressed prefix (multi-turn growth)             */
/* ------------------------------------------------------------------------ */

/* The rows of m tokens generated after a compressed prefix are projected onto
 * the group's stored basis, a_new = [x_l1 | ... | x_lG] V_r with V_r = Bt as
 * stored, so that A_new B_l rebuilds them like the prefix rows ([xKV blog]
 * "xKV 到底做了什么？": the shared token basis A = X V_r; the pages leave the
 * compression of generated tokens open, this is the projection onto the
 * existing basis), and for a key side the landmarks of the new chunks are
 * formed at positions pos0 + t.  Writing A_new at A + pos0 * r (an A allocated
 * with room for growth) extends the prefix to T' = pos0 + m; the landmarks of
 * the new chunks follow the prefix's along each head's chunk axis. */
typedef struct {
  int m;                     /* appended tokens, > 0                                           */
  long pos0;                 /* position of the first appended token (the prefix length)      */
  int G, d_kv, r;            /* as in xkv_compress_desc (n = G * d_kv, r <= n)                */
  int dtype;                 /* enum xkv_dtype of the rows, Bt, A_new and landmarks_new        */
  int n_kv_heads, head_dim;  /* landmark layout; d_kv == n_kv_heads * head_dim                */
  int chunk;                 /* with landmarks: m % chunk == 0 and pos0 % chunk == 0          */
  double rope_theta;
  const void* const* layers; /* (host) G device pointers; layer l: m x d_kv rows, stride ld_layer */
  long ld_layer;             /* >= d_kv; for bf16 a multiple of 8 (rows 16-byte aligned)       */
  const void* Bt;            /* n x r stored basis (Bt = V_r), row stride r                    */
  void* A_new;               /* m x r output rows, row stride r                                */
  void* landmarks_new;       /* nullable: G x n_kv_heads x (m/chunk) x head_dim                 */
} xkv_append_args;

/* Workspace bytes for xkv_compress_append (the transposed basis, r x n). */
int xkv_append_ws_size(const xkv_append_args* args, size_t* bytes);

/* Enqueue the projection (bf16 matrix cores, float32 sums) and the landmarks on
 * `stream`.  Errors: XKV_EINVAL (sizes, NULL pointers, alignment). */
int xkv_compress_append(xkv_ctx ctx, const xkv_append_args* args, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Selective Reconstruction decode (one layer, one step, `batch` sequences)  */
/* ------------------------------------------------------------------------ */

typedef struct {
  int batch;            /* sequences                                                      */
  int n_q_heads;        /* multiple of n_kv_heads (query head j uses KV head j / (H_q/H_kv)) */
  int n_kv_heads;
  int head_dim;         /* 64 or 128                                                      */
  int T;                /* compressed prefix length; T % chunk == 0                       */
  int n_gen;            /* generated tokens in the tail, including the current one;     */
                        /* query position p = T + n_gen - 1 (p = T when n_gen == 0)       */
  int chunk;            /* 8..64, power of two                                            */
  int top_k;            /* chunks kept per KV head (all candidates if larger)            */
  int n_sink;           /* exact rows [0, n_sink)                                          */
  int n_local;          /* exact rows [T - n_local, T); candidates are chunks c with       */
                        /* c*chunk < T - n_local                                          */
  int r_k, r_v;         /* ranks of the key / value bases; r_v == 0: values are exact     */
  int dtype;            /* enum xkv_dtype of q, A, Bt, landmarks, tails, V_full            */
  float scale;          /* softmax scale, usually 1/sqrt(head_dim)                        */
  double rope_theta;

  const void* q;        /* batch x n_q_heads x head_dim, pre-RoPE, at position p          */
  const void* A_k;      /* per sequence T x r_k, row stride ld_A_k                         */
  long ld_A_k, bstride_A_k;
  const void* Bt_k;     /* per sequence: this layer's d_kv x r_k rows of Bt, row stride ld_Bt_k */
  long ld_Bt_k, bstride_Bt_k;
  const void* A_v;      /* as A_k for values (r_v > 0)                                     */
  long ld_A_v, bstride_A_v;
  const void* Bt_v;
  long ld_Bt_v, bstride_Bt_v;
  const void* V_full;   /* r_v == 0: per sequence T x d_kv exact values, row stride ld_V  */
  long ld_V, bstride_V;
  const void* landmarks;/* per sequence n_kv_heads x (T/chunk) x head_dim                 */
  long bstride_lm;
  void* k_tail;         /* per sequence (n_sink + n_local + max_gen) x d_kv pre-RoPE rows: */
  void* v_tail;         /* sink positions, then positions T-n_local..T-1, then T, T+1, ...  */
  long ld_tail, bstride_tail;
  const void* k_new;    /* nullable: per sequence d_kv row written to tail row           */
  const void* v_new;    /* n_sink + n_local + n_gen - 1 before attention (the new token)  */
  long bstride_new;
  float* out;           /* batch x n_q_heads x head_dim                                   */
  int* sel;             /* batch x n_kv_heads x top_k selected chunk ids, ascending; unused */
                        /* slots (fewer candidates than top_k) are -1                      */
} xkv_sr_args;

/* Workspace bytes for xkv_sr_decode / xkv_sr_select / xkv_sr_attend. */
int xkv_sr_ws_size(const xkv_sr_args* args, size_t* bytes);

/* Append the new token (if given), score every candidate chunk against the
 * landmarks, and write the top-k chunk ids of each KV head to args->sel. */
int xkv_sr_select(xkv_ctx ctx, const xkv_sr_args* args, void* ws, size_t ws_bytes, void* stream);

/* Rebuild the selected rows (A rows x B_l, then RoPE for keys), attend over
 * them and the exact rows with split-K online softmax, merge, write args->out.
 * Reads args->sel as written by xkv_sr_select.  Compressed values are applied
 * in rank space, (sum_t p_t A_v[t]) B_v,l, which equals sum_t p_t (A_v[t] B_v,l)
 * up to rounding. */
int xkv_sr_attend(xkv_ctx ctx, const xkv_sr_args* args, void* ws, size_t ws_bytes, void* stream);

/* xkv_sr_select followed by xkv_sr_attend.  On the matrix-core path (below), with at most
 * 16384 candidates and an attend grid (KV heads x 64-row splits x batch) no larger than the
 * device's compute units, the attend kernel selects the top-k itself (one launch fewer): the
 * same selection, written to args->sel by the attend blocks.
 * Limits (XKV_EUNSUPPORTED beyond them): at most 32768 candidate chunks per KV
 * head; the selected rows (64 per attend block) plus the exact rows (16 per
 * tile) at most 1088 blocks per head on the matrix-core path with compressed
 * values (bf16, head_dim 128, r_k == r_v a multiple of 128 up to 4096; enough
 * for every chunk of a 64k prefix, i.e. full reconstruction) and 257 otherwise.
 * With r_v == 0 (xK-SR: keys compressed, values exact in V_full) the keys take
 * the same matrix-core path when r_k is a multiple of 128 (V_full 16-byte
 * aligned, strides multiples of 8 elements; XKV_EINVAL otherwise) and the exact
 * value rows are summed in value space. */
int xkv_sr_decode(xkv_ctx ctx, const xkv_sr_args* args, void* ws, size_t ws_bytes, void* stream);

/* One decode step through `n_layers` layers in order (args[l] describes layer l;
 * all share `ws`, which must satisfy xkv_sr_ws_size for every layer): the
 * select and attend kernels of each layer are enqueued back to back on
 * `stream`, with no host synchronisation (the top-k inside the attend kernel
 * under the conditions of xkv_sr_decode).  attend_events (nullable): host array
 * of 2*n_layers hipEvent_t (timing enabled); events 2l and 2l+1 mark the start
 * and the end of layer l's attend kernel (stamped by its dispatch on the
 * matrix-core path, recorded on `stream` around the launch otherwise). */
int xkv_sr_decode_layers(xkv_ctx ctx, int n_layers, const xkv_sr_args* args, void* ws, size_t ws_bytes,
                         void* stream, void* const* attend_events);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same decode
 * step as xkv_sr_decode_layers, with the same kernels and results, but its
 * scratch (chunk scores, split partials) lives in a device array owned by the
 * library, XKV_SR_SCRATCH_BYTES per GPU, held from the first xkv_ctx_create on
 * that GPU until the process ends.  The caller still passes every input and
 * output (args as for xkv_sr_decode_layers).  Nothing is allocated or freed.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe.  Errors: XKV_EWORKSPACE when a
 * layer's xkv_sr_ws_size exceeds XKV_SR_SCRATCH_BYTES (e.g. full reconstruction
 * of a long prefix), plus those of xkv_sr_decode_layers. */
#define XKV_SR_SCRATCH_BYTES (64u << 20)
int xkv_sr_decode_layers_noalloc(xkv_ctx ctx, int n_layers, const xkv_sr_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Dense decode baseline (full attention over the whole cache)               */
/* ------------------------------------------------------------------------ */

/* Decode attention of one query position over every cached position: the
 * full-attention reference that Selective Reconstruction is measured against
 * ([xKV blog] "图 5、图 6、图 7 分别说明了什么？": attention latency of SR
 * against full attention; decode attention as in [KQ-SVD] section 3.2).
 * bf16 only, head_dim 128, query heads j of KV head j / (H_q / H_kv).  The
 * cache holds keys AFTER RoPE (row t rotated at position t, as a standard KV
 * cache stores them; see xkv_rope_rows); the query is rotated here at q_pos.
 * out[b][j] = softmax_t(RoPE(q_j, q_pos) . K[t] * scale) V[t] over t < n_ctx.
 * Splits of 128..2048 rows (chosen from the grid size) merged by log-sum-exp;
 * n_ctx <= 512 * 2048.  The scores use the bf16 matrix cores with the rotated,
 * scaled query split into two bf16 parts (about 16 significant bits); weights
 * and sums stay float32.
 * Errors: XKV_EINVAL (sizes, NULL pointers, misaligned rows: q, K, V 16-byte
 * aligned with ld_kv and bstride_kv multiples of 8), XKV_EUNSUPPORTED. */
typedef struct {
  int batch;
  int n_q_heads;        /* multiple of n_kv_heads, at most 8 per KV head */
  int n_kv_heads;
  int head_dim;         /* 128 */
  long n_ctx;           /* cached positions 0 .. n_ctx - 1 */
  long q_pos;           /* the query's position */
  int dtype;            /* XKV_BF16 */
  float scale;          /* usually 1/sqrt(head_dim) */
  double rope_theta;
  const void* q;        /* batch x n_q_heads x head_dim, pre-RoPE */
  const void* K;        /* per sequence n_ctx x (n_kv_heads*head_dim) post-RoPE keys */
  const void* V;        /* per sequence n_ctx x (n_kv_heads*head_dim) values */
  long ld_kv, bstride_kv;
  float* out;           /* batch x n_q_heads x head_dim */
} xkv_dense_args;

/* Workspace bytes for xkv_dense_decode (the split partials). */
int xkv_dense_ws_size(const xkv_dense_args* args, size_t* bytes);
int xkv_dense_decode(xkv_ctx ctx, const xkv_dense_args* args, void* ws, size_t ws_bytes, void* stream);

/* y[row] = RoPE(x[row], pos0 + row) for `rows` rows of n_heads x head_dim
 * (rotate-half pairs (i, i + head_dim/2), angle (pos0 + row) * theta^(-2i/d)
 * reduced in float64): builds the post-RoPE key cache the dense baseline reads.
 * x and y may be the same rows (in place).  dtype XKV_F32 or XKV_BF16. */
int xkv_rope_rows(const void* x, long ld_x, void* y, long ld_y, int rows, long pos0, int n_heads, int head_dim,
                  double rope_theta, int dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Rank diagnostics                                                          */
/* ------------------------------------------------------------------------ */

/* Diagnostics of a spectrum: `eigvals` (host, n_vals values, any order) are
 * eigenvalues of a side's Gram C = X^T X, i.e. squared singular values of X,
 * e.g. the Ritz values xkv_compress_sides returns (negative values count as 0).
 *   energy_rank: the smallest k whose k largest eigenvalues reach frac * total
 *     ([xKV blog] "xKV 到底做了什么？" figure 2(c): the rank that keeps 95 % of the
 *     cumulative eigenvalues); total = the trace of C (stats[4] of
 *     xkv_compress_sides), or <= 0 to use the sum of the given values; -1 when the
 *     given values do not reach the target;
 *   covered: their sum / total;
 *   for a complete spectrum (complete != 0; e.g. a compression at r = n, whose
 *   Ritz values are exact) numerical_rank r = #{sigma_i > n_vals * eps * sigma_1},
 *   erank = exp(-sum p_i ln p_i) with p_i = sigma_i / sum_{j<r} sigma_j, and
 *   ner = erank / r ([KV-CoRE] section 2.B); otherwise -1, NaN, NaN.
 * Host only; no device work.  Errors: XKV_EINVAL (NULL pointers, n_vals < 0,
 * frac outside (0, 1]). */
typedef struct {
  int energy_rank;
  double covered;
  int numerical_rank;
  double erank;
  double ner;
} xkv_rank_info;

int xkv_rank_stats(const double* eigvals, int n_vals, double total, double frac, int complete, xkv_rank_info* out);

/* Adaptive rank at a fixed total budget ([KV-CoRE] implications: compressibility
 * differs across layers and should guide a layer-aware compression strategy;
 * [xKV blog] figure 5: the rank that pays off differs by task).  Side s keeps r_s
 * of its leading eigenvalues, r_s a multiple of `granule` in [r_min, r_max], with
 * sum_s r_s <= budget, chosen to keep the most energy
 * sum_s sum_{i < r_s} lambda_i^(s), i.e. (Eckart-Young) the least total squared
 * reconstruction error of the rank-r_s truncations.  A side compressed at rank
 * r_max and truncated to its first r_s columns of A and rows of B is exactly its
 * rank-r_s factorisation (the columns of V_r come in eigenvalue order), so the
 * caller compresses once at r_max and decodes each side with r_k / r_v = r_s and
 * the r_max leading dimensions (a granule of 128 keeps the decode on the matrix
 * cores).
 * eigvals (host): n_sides rows, row stride ld >= r_max, each the side's leading
 * eigenvalues in descending order (the eigvals of xkv_compress_sides at r_max).
 * ranks (host, out): n_sides ints; kept (host, out, nullable): the energy kept.
 * Host only.  Errors: XKV_EINVAL (NULL pointers, ranks not multiples of the
 * granule, r_min > r_max, ld < r_max, budget < n_sides * r_min). */
int xkv_rank_allocate(const double* eigvals, int n_sides, int ld, int r_max, long budget, int granule, int r_min,
                      int* ranks, double* kept);

/* ------------------------------------------------------------------------ */
/* Component entry points used by the parity tests                           */
/* ------------------------------------------------------------------------ */

/* Gram of the concatenated layers of `n_sides` sides, one launch (the kernel
 * and batching of xkv_compress_sides): layers (host) holds n_sides*G device
 * pointers (side-major); C receives n_sides matrices n x n float64 (row stride
 * n, side stride n*n), C_s = X_s^T X_s.  For bf16 the layer pointers must be
 * 16-byte aligned and ld_layer a multiple of 8.  n_sides*G <= 256. */
int xkv_gram(const void* const* layers, int n_sides, long ld_layer, int T, int G, int d_kv, int dtype,
             double* C, void* stream);

/* Top-k of each of `rows` score rows (float32, row stride ld) over the first
 * n_cand entries: ascending ids of the k largest, ties to the lower id, -1
 * padding; the same kernel as xkv_sr_select.  n_cand <= 32768. */
int xkv_topk(const float* scores, int rows, int n_cand, long ld, int k, int* sel, void* stream);

/* Host symmetric eigensolver used for the Rayleigh-Ritz step (plain C,
 * Householder tridiagonalisation + implicit QR with Wilkinson shifts).
 * H (host, n x n, row stride n, symmetric) is not modified.  Writes the nvec
 * largest eigenvalues to w (host, descending) and their eigenvectors as the
 * columns of Z (host, n x nvec, row stride nvec).  Runs without a GPU, in the
 * calling thread and one more (the reduction's row passes shared by the two, as
 * compressions run it for k_b >= 256 when host threads allow). */
int xkv_host_eigh(int n, const double* H, int nvec, double* w, double* Z);

#ifdef __cplusplus
}
#endif
#endif /* XKV_H */
