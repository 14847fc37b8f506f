// C ABI of libxkv: argument validation, workspace layout and the order of
// kernel launches.  Every numeric step runs in the HIP kernels of this
// directory or, for the Rayleigh-Ritz eigensolve only, in host_eigh.c.
#include "xkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "decode_params.h"
#include "dense_params.h"
#include "xkv_kernels.h"

#include "host_eigh.h"
extern "C" int xkv_rank_allocate_impl(const double* eig, int n_sides, int ld, int r_max, long budget, int granule,
                                      int r_min, int* ranks, double* kept);
extern "C" int xkv_rank_stats_impl(const double* vals, int n, double total, double frac, int complete,
                                   int* energy_rank, double* covered, int* num_rank, double* erank, double* ner);

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define XKV_HIP(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(XKV_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Sequential carving of a workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align256(count * sizeof(T));
    return p;
  }
};

// A compression's sides go in up to this many parts, so that the GPU work of a later part runs
// while the host solves an earlier part's Rayleigh-Ritz problems.
constexpr int kMaxParts = 2;

}  // namespace

struct xkv_ctx_s {
  int device = 0;
  int n_cu = 0;                 // compute units of the device
  int host_threads = 16;
  double* pin = nullptr;        // pinned staging for H, residuals (down) and reflectors (up)
  size_t pin_doubles = 0;
  // Per part of a compression's sides (up to kMaxParts): the rotation logs of the Rayleigh-Ritz
  // eigensolves (pinned staging and the device copy the vector kernel reads), grown as needed.
  void* lpin[kMaxParts] = {};
  size_t lpin_bytes[kMaxParts] = {};
  void* ldev[kMaxParts] = {};
  size_t ldev_bytes[kMaxParts] = {};
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  // Host memory of the Rayleigh-Ritz eigensolves, two per side (value state + first half of
  // the vectors, second half of the vectors), kept between calls so that repeated
  // compressions neither map nor fault pages.
  std::vector<xkv_eigh_scratch> eig_side;
  // Marks the Rayleigh-Ritz matrices of each part of the sides as copied to the host.
  hipEvent_t half_done[kMaxParts] = {};
};

extern "C" {

int xkv_version(void) { return 100; }

const char* xkv_last_error(void) { return g_err.c_str(); }

int xkv_ctx_create(int device, int host_threads, xkv_ctx* out) {
  if (!out) return fail(XKV_EINVAL, "xkv_ctx_create: out is NULL");
  int n = 0;
  XKV_HIP(hipGetDeviceCount(&n));
  if (device < 0 || device >= n) return fail(XKV_EINVAL, "xkv_ctx_create: device %d of %d", device, n);
  hipDeviceProp_t prop;
  XKV_HIP(hipGetDeviceProperties(&prop, device));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(XKV_EUNSUPPORTED, "xkv_ctx_create: device %d is %s; only gfx950 is supported", device,
                prop.gcnArchName);
  xkv_ctx c = new xkv_ctx_s();
  c->device = device;
  c->n_cu = prop.multiProcessorCount;
  c->host_threads = host_threads > 0 ? host_threads : 16;
  XKV_HIP(hipSetDevice(device));
  {
    // The decode scratch of xkv_sr_decode_layers_noalloc: its address on this device.
    const hipError_t e = xkv::sr_scratch_setup(device);
    if (e != hipSuccess) {
      delete c;
      return fail(XKV_EHIP, "xkv_ctx_create: address of the decode scratch on device %d: %s", device,
                  hipGetErrorString(e));
    }
  }
  XKV_HIP(hipEventCreateWithFlags(&c->upload_done, hipEventDisableTiming));
  for (hipEvent_t& e : c->half_done) XKV_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  *out = c;
  return XKV_OK;
}

void xkv_ctx_destroy(xkv_ctx ctx) {
  if (!ctx) return;
  if (ctx->upload_done) {
    (void)hipEventSynchronize(ctx->upload_done);
    (void)hipEventDestroy(ctx->upload_done);
  }
  for (hipEvent_t e : ctx->half_done)
    if (e) (void)hipEventDestroy(e);
  if (ctx->pin) (void)hipHostFree(ctx->pin);
  for (int h = 0; h < kMaxParts; ++h) {
    if (ctx->lpin[h]) (void)hipHostFree(ctx->lpin[h]);
    if (ctx->ldev[h]) (void)hipFree(ctx->ldev[h]);
  }
  for (auto& sc : ctx->eig_side) xkv_eigh_scratch_release(&sc);
  delete ctx;
}

int xkv_rank_stats(const double* eigvals, int n_vals, double total, double frac, int complete, xkv_rank_info* out) {
  if (!out || n_vals < 0 || (n_vals > 0 && !eigvals) || !(frac > 0.0 && frac <= 1.0))
    return fail(XKV_EINVAL, "xkv_rank_stats: bad arguments (n_vals=%d, frac=%g)", n_vals, frac);
  if (xkv_rank_stats_impl(eigvals, n_vals, total, frac, complete, &out->energy_rank, &out->covered,
                          &out->numerical_rank, &out->erank, &out->ner))
    return fail(XKV_EINVAL, "xkv_rank_stats: out of host memory");
  return XKV_OK;
}

int xkv_rank_allocate(const double* eigvals, int n_sides, int ld, int r_max, long budget, int granule, int r_min,
                      int* ranks, double* kept) {
  const int rc = xkv_rank_allocate_impl(eigvals, n_sides, ld, r_max, budget, granule, r_min, ranks, kept);
  if (rc == -2) return fail(XKV_EINVAL, "xkv_rank_allocate: out of host memory");
  if (rc)
    return fail(XKV_EINVAL, "xkv_rank_allocate: bad arguments (n_sides=%d, ld=%d, r_max=%d, budget=%ld, "
                "granule=%d, r_min=%d; ranks are multiples of the granule, r_min <= r_max <= ld, "
                "budget >= n_sides * r_min)", n_sides, ld, r_max, budget, granule, r_min);
  return XKV_OK;
}

int xkv_host_eigh(int n, const double* H, int nvec, double* w, double* Z) {
  if (n <= 0 || !H || !w || !Z || nvec <= 0 || nvec > n)
    return fail(XKV_EINVAL, "xkv_host_eigh: bad arguments (n=%d, nvec=%d)", n, nvec);
  std::vector<double> all(n);
  // The two phases as compressions run them: the value phase shared by two threads, the
  // vector phase in two column ranges, the second with working memory of its own (the way a
  // helper thread takes half of a side).
  xkv_eigh_scratch sc{}, helper{};
  xkv_eigh_pair pr{};
  int wrc = 0;
  std::thread worker([&]() { wrc = xkv_eigh_values_pair(n, H, nvec, nullptr, &sc, &helper, &pr, 1, nullptr); });
  int rc = xkv_eigh_values_pair(n, H, nvec, all.data(), &sc, &helper, &pr, 0, nullptr);
  worker.join();
  if (rc == 0 && wrc != 0) rc = wrc;
  if (rc == 0) rc = xkv_eigh_vectors(&sc, 0, nvec / 2, Z, &sc);
  if (rc == 0) rc = xkv_eigh_vectors(&sc, nvec / 2, nvec, Z, &helper);
  xkv_eigh_scratch_release(&sc);
  xkv_eigh_scratch_release(&helper);
  if (rc == 0) std::memcpy(w, all.data(), nvec * sizeof(double));
  if (rc == -1) return fail(XKV_EINVAL, "xkv_host_eigh: out of host memory");
  if (rc == -4) return fail(XKV_ENUMERIC, "xkv_host_eigh: H has an entry that is not finite");
  if (rc != 0) return fail(XKV_ENUMERIC, "xkv_host_eigh: QR iteration did not converge");
  return XKV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Compression
// ---------------------------------------------------------------------------
namespace {

struct CompressPlan {
  int T, G, d_kv, n, r, kb, bf16, fp32_iters, fp64_iters, nblk;
};

int plan_compress(const xkv_compress_desc* d, int n_sides, CompressPlan* p) {
  if (!d) return fail(XKV_EINVAL, "compress: desc is NULL");
  if (n_sides <= 0) return fail(XKV_EINVAL, "compress: n_sides must be positive");
  if (d->T <= 0 || d->G <= 0 || d->G > 16 || d->d_kv <= 0 || d->d_kv % 8)
    return fail(XKV_EINVAL, "compress: need T > 0, 1 <= G <= 16, d_kv a positive multiple of 8");
  if (d->dtype != XKV_F32 && d->dtype != XKV_BF16) return fail(XKV_EINVAL, "compress: unknown dtype");
  const int n = d->G * d->d_kv;
  if (d->r <= 0 || d->r > n) return fail(XKV_EINVAL, "compress: rank %d outside [1, %d]", d->r, n);
  if (d->fp32_iters < 0 || d->fp64_iters < 1) return fail(XKV_EINVAL, "compress: need fp32_iters >= 0, fp64_iters >= 1");
  if (d->n_kv_heads <= 0 || d->head_dim <= 0 || d->head_dim % 2 || d->n_kv_heads * d->head_dim != d->d_kv)
    return fail(XKV_EINVAL, "compress: d_kv must equal n_kv_heads * head_dim (even head_dim)");
  if (d->head_dim > 512 || 256 % (d->head_dim / 2) != 0)
    return fail(XKV_EUNSUPPORTED, "compress: head_dim must be 2..512 with head_dim/2 dividing 256");
  if (d->chunk <= 0) return fail(XKV_EINVAL, "compress: chunk must be positive");
  if (!(d->tol >= 0.0) || d->max_rounds < 0) return fail(XKV_EINVAL, "compress: tol and max_rounds must be >= 0");
  const int p_over = d->oversample < 0 ? d->r / 2 : d->oversample;
  p->T = d->T;
  p->G = d->G;
  p->d_kv = d->d_kv;
  p->n = n;
  p->r = d->r;
  p->kb = std::min(n, d->r + p_over);
  p->bf16 = d->dtype == XKV_BF16;
  p->fp32_iters = d->fp32_iters;
  p->fp64_iters = d->fp64_iters;
  p->nblk = (p->kb + 63) / 64;
  return XKV_OK;
}

constexpr int kWSplit = 3;   // K ranges of W = Y^T Y at most (workspace for their partial products)

struct CompressWs {
  double* C64; float* C32;
  float* Q32; float* Y32;
  double* Q64; double* Y64;
  double* W; double* L; double* Dinv;
  double* H; double* Z; double* Vr;
  double* Rf; int* pos; double* Wb;   // packed reflector blocks, wanted positions, block products
  double* Zs;                         // working memory of the rotation kernel
  double* Zseg; double* Zsegs;        // with the log in pieces: each piece's product and working memory
  double* Wpart;                      // partial products of W = Y^T Y (kWSplit per side)
  double* wdiag;
  double* YZ; double* theta; double* res2;
  void* VrT;
  double* trace;
  int* info;
  size_t bytes;
};

CompressWs carve_compress(void* ws, const CompressPlan& p, int S) {
  Carver c(ws);
  CompressWs w;
  const size_t nn = (size_t)p.n * p.n, nk = (size_t)p.n * p.kb, kk = (size_t)p.kb * p.kb;
  w.C64 = c.take<double>(S * nn);
  w.C32 = p.fp32_iters > 0 ? c.take<float>(S * nn) : nullptr;
  w.Q32 = c.take<float>(S * nk);
  w.Y32 = p.fp32_iters > 0 ? c.take<float>(S * nk) : nullptr;
  w.Q64 = c.take<double>(S * nk);
  w.Y64 = c.take<double>(S * nk);
  w.W = c.take<double>(S * kk);
  w.L = c.take<double>(S * kk);
  w.Dinv = c.take<double>((size_t)S * p.nblk * 64 * 64);
  w.H = c.take<double>(S * kk);
  w.Z = c.take<double>((size_t)S * p.kb * p.r);
  w.Rf = c.take<double>((size_t)S * xkv_eigh_refl_doubles(p.kb));
  w.pos = c.take<int>((size_t)S * p.r);
  w.Wb = c.take<double>((size_t)S * 2 * XKV_EIGH_NBG * p.r);
  w.Zs = c.take<double>((size_t)S * xkv::ritz_scratch_doubles(p.kb, p.r));
  const int parts = xkv::ritz_parts(p.kb);
  w.Zseg = parts > 1 ? c.take<double>((size_t)S * parts * kk) : nullptr;
  w.Zsegs = parts > 1 ? c.take<double>((size_t)S * parts * xkv::ritz_scratch_doubles(p.kb, p.kb)) : nullptr;
  w.Wpart = c.take<double>((size_t)S * kWSplit * kk);
  w.Vr = c.take<double>((size_t)S * p.n * p.r);
  w.wdiag = c.take<double>((size_t)S * p.kb);
  w.YZ = c.take<double>((size_t)S * p.n * p.r);
  w.theta = c.take<double>((size_t)S * p.r);
  w.res2 = c.take<double>((size_t)S * p.r);
  w.VrT = c.take<float>((size_t)S * p.n * p.r);
  w.trace = c.take<double>(S);
  w.info = c.take<int>(S);
  w.bytes = c.off;
  return w;
}

// The workspace arrays from side s0 on (every array holds its sides back to back).
CompressWs shift_compress_ws(const CompressWs& w, const CompressPlan& p, int s0) {
  const size_t nn = (size_t)p.n * p.n, nk = (size_t)p.n * p.kb, kk = (size_t)p.kb * p.kb;
  const size_t nr = (size_t)p.n * p.r, es = p.bf16 ? 2 : 4;
  CompressWs v = w;
  v.C64 += s0 * nn;
  if (v.C32) v.C32 += s0 * nn;
  v.Q32 += s0 * nk;
  if (v.Y32) v.Y32 += s0 * nk;
  v.Q64 += s0 * nk;
  v.Y64 += s0 * nk;
  v.W += s0 * kk;
  v.L += s0 * kk;
  v.Dinv += (size_t)s0 * p.nblk * 64 * 64;
  v.H += s0 * kk;
  v.Z += (size_t)s0 * p.kb * p.r;
  v.Rf += (size_t)s0 * xkv_eigh_refl_doubles(p.kb);
  v.pos += (size_t)s0 * p.r;
  v.Wb += (size_t)s0 * 2 * XKV_EIGH_NBG * p.r;
  v.Zs += (size_t)s0 * xkv::ritz_scratch_doubles(p.kb, p.r);
  const int parts = xkv::ritz_parts(p.kb);
  if (v.Zseg) v.Zseg += (size_t)s0 * parts * kk;
  if (v.Zsegs) v.Zsegs += (size_t)s0 * parts * xkv::ritz_scratch_doubles(p.kb, p.kb);
  v.Wpart += (size_t)s0 * kWSplit * kk;
  v.Vr += s0 * nr;
  v.wdiag += (size_t)s0 * p.kb;
  v.YZ += s0 * nr;
  v.theta += (size_t)s0 * p.r;
  v.res2 += (size_t)s0 * p.r;
  v.VrT = (char*)v.VrT + s0 * nr * es;
  v.trace += s0;
  v.info += s0;
  return v;
}

xkv::GemmDesc gdesc(int M, int N, int K, int ta, int tb, int tA, int tB, int tC, const void* A, long lda, long sA,
                    const void* B, long ldb, long sB, void* C, long ldc, long sC, double alpha, double beta,
                    int batch) {
  xkv::GemmDesc g;
  g.M = M; g.N = N; g.K = K; g.ta = ta; g.tb = tb;
  g.typeA = tA; g.typeB = tB; g.typeC = tC; g.acc = xkv::GF64;
  g.A = A; g.lda = lda; g.sA = sA;
  g.B = B; g.ldb = ldb; g.sB = sB;
  g.C = C; g.ldc = ldc; g.sC = sC;
  g.alpha = alpha; g.beta = beta; g.batch = batch;
  g.sym = 0;
  g.ksplit = 1;
  g.part = nullptr;
  return g;
}

#define XKV_K(call)                                                                        \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return fail(XKV_EHIP, "kernel launch %s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// CholeskyQR pass: Q = Y R^-1 with Y^T Y = R^T R (R = L^T).  Y is overwritten.
// A symmetric k_b x k_b product over K = n: only the tiles on or above the diagonal, mirrored.
// Those tiles alone leave the device's workgroup slots (4 per compute unit) short of two rounds
// at the 64k sizes, each tile a long run over K, so K is split into ranges of at least 512 (up to
// kWSplit) whose partial products (in `part`) are summed in a fixed order.  The split depends on
// n only, so that a side's result does not depend on how many sides share the call.
void sym_split(xkv::GemmDesc& g, int n, double* part) {
  g.sym = 1;
  const int ks = std::max(1, std::min(kWSplit, n / 512));
  if (ks > 1) {
    g.ksplit = ks;
    g.part = part;
  }
}

int cholqr(const CompressPlan& p, const CompressWs& w, int S, void* Y, int tY, void* Q, int tQ, hipStream_t st) {
  using namespace xkv;
  const int n = p.n, kb = p.kb;
  const long nk = (long)n * kb, kk = (long)kb * kb, dstride = (long)p.nblk * 4096;
  GemmDesc wd = gdesc(kb, kb, n, 1, 0, tY, tY, GF64, Y, kb, nk, Y, kb, nk, w.W, kb, kk, 1.0, 0.0, S);
  sym_split(wd, n, w.Wpart);   // W = Y^T Y
  XKV_K(gemm(wd, st));
  XKV_K(launch_copy_diag(w.W, kb, kk, w.wdiag, kb, kb, S, st));
  for (int jb = 0; jb < p.nblk; ++jb) {
    const int j0 = jb * 64, nbj = std::min(64, kb - j0), rem = kb - j0 - nbj;
    double* Dj = w.Dinv + (long)jb * 4096;
    // float32 sweeps clamp tiny pivots; float64 sweeps report them as a breakdown
    XKV_K(launch_potrf_diag(w.W, kb, kk, w.L, kb, kk, Dj, dstride, j0, nbj, w.wdiag, kb, tY == GF32, S, w.info,
                            st));
    if (rem > 0) {
      const long off = (long)(j0 + nbj) * kb + j0;
      XKV_K(gemm(gdesc(rem, nbj, nbj, 0, 1, GF64, GF64, GF64, w.W + off, kb, kk, Dj, 64, dstride, w.L + off, kb, kk,
                       1.0, 0.0, S), st));
      const long toff = (long)(j0 + nbj) * kb + (j0 + nbj);
      XKV_K(gemm(gdesc(rem, rem, nbj, 0, 1, GF64, GF64, GF64, w.L + off, kb, kk, w.L + off, kb, kk, w.W + toff, kb,
                       kk, -1.0, 1.0, S), st));
    }
  }
  const size_t esY = tY == GF64 ? 8 : 4, esQ = tQ == GF64 ? 8 : 4;
  for (int jb = 0; jb < p.nblk; ++jb) {
    const int j0 = jb * 64, nbj = std::min(64, kb - j0);
    void* Yj = (char*)Y + j0 * esY;
    void* Qj = (char*)Q + j0 * esQ;
    if (j0 > 0)
      XKV_K(gemm(gdesc(n, nbj, j0, 0, 1, tQ, GF64, tY, Q, kb, nk, w.L + (long)j0 * kb, kb, kk, Yj, kb, nk, -1.0, 1.0,
                       S), st));
    XKV_K(gemm(gdesc(n, nbj, nbj, 0, 1, tY, GF64, tQ, Yj, kb, nk, w.Dinv + (long)jb * 4096, 64, dstride, Qj, kb, nk,
                     1.0, 0.0, S), st));
  }
  return XKV_OK;
}

}  // namespace

extern "C" int xkv_compress_ws_size(const xkv_compress_desc* desc, int n_sides, size_t* bytes) {
  if (!bytes) return fail(XKV_EINVAL, "xkv_compress_ws_size: bytes is NULL");
  CompressPlan p;
  int rc = plan_compress(desc, n_sides, &p);
  if (rc) return rc;
  *bytes = carve_compress(nullptr, p, n_sides).bytes;
  return XKV_OK;
}

extern "C" int xkv_compress_sides(xkv_ctx ctx, const xkv_compress_desc* desc, int n_sides, const xkv_side* sides,
                                  void* ws, size_t ws_bytes, void* stream) {
  using namespace xkv;
  if (!ctx) return fail(XKV_EINVAL, "compress: ctx is NULL");
  CompressPlan p;
  int rc = plan_compress(desc, n_sides, &p);
  if (rc) return rc;
  if (!sides) return fail(XKV_EINVAL, "compress: sides is NULL");
  const int S = n_sides;
  const size_t need = carve_compress(nullptr, p, S).bytes;
  if (!ws || ws_bytes < need) return fail(XKV_EWORKSPACE, "compress: workspace %zu bytes < %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(XKV_EINVAL, "compress: workspace must be 16-byte aligned");
  bool any_lm = false;
  for (int s = 0; s < S; ++s) {
    const xkv_side& sd = sides[s];
    if (!sd.layers || !sd.A || !sd.Bt) return fail(XKV_EINVAL, "compress: side %d has a NULL pointer", s);
    if (sd.ld_layer < p.d_kv) return fail(XKV_EINVAL, "compress: side %d ld_layer %ld < d_kv", s, sd.ld_layer);
    if (sd.ld_layer != sides[0].ld_layer) return fail(XKV_EINVAL, "compress: every side must share ld_layer");
    if (p.bf16 && sd.ld_layer % 8) return fail(XKV_EINVAL, "compress: bf16 ld_layer must be a multiple of 8");
    for (int l = 0; l < p.G; ++l) {
      if (!sd.layers[l]) return fail(XKV_EINVAL, "compress: side %d layer %d is NULL", s, l);
      if (!aligned16(sd.layers[l])) return fail(XKV_EINVAL, "compress: layer pointers must be 16-byte aligned");
    }
    if (sd.landmarks) {
      any_lm = true;
      if (p.T % desc->chunk) return fail(XKV_EINVAL, "compress: landmarks need T %% chunk == 0");
    }
  }
  hipStream_t st = (hipStream_t)stream;
  XKV_HIP(hipSetDevice(ctx->device));
  CompressWs w = carve_compress(ws, p, S);
  const int n = p.n, kb = p.kb, r = p.r;
  const long nn = (long)n * n, nk = (long)n * kb, kk = (long)kb * kb;

  XKV_K(launch_zero_i32(w.info, S, st));
  // The sides go in two parts (halves) when there are at least 4, the larger first: the GPU work
  // of the second half runs while the host solves the first half's Rayleigh-Ritz problems
  // (stream order; the host waits on per-half events, not on the stream).  Three parts of the
  // 64k workload's 16 sides (6 + 5 + 5) measured slower, 0.130 s against 0.123 s: the host
  // solves the parts one after another, and the smaller batches leave the GPU's small kernels
  // less to do per launch.
  struct Half {
    CompressWs w;   // the workspace arrays from this half's first side on
    int s0, cnt;
    void* Qcur;
    int tQ;
    double* Qa;
    double* Ya;
  };
  const int nh = S >= 4 ? 2 : 1;
  Half hv[kMaxParts];
  for (int h = 0, s0 = 0; h < nh; ++h) {
    Half& hf = hv[h];
    hf.s0 = s0;
    hf.cnt = S / nh + (h < S % nh ? 1 : 0);
    s0 += hf.cnt;
    hf.w = shift_compress_ws(w, p, hf.s0);
    hf.Qcur = hf.w.Q32;
    hf.tQ = GF32;
    hf.Qa = hf.w.Q64;
    hf.Ya = hf.w.Y64;
  }
  const int per = std::max(1, kMaxPtrs / p.G);
  // C is exactly symmetric (both Gram kernels give C[i][j] and C[j][i] the same value), so the
  // products C Q read it as C^T: the GEMM then stages it into LDS along its contiguous rows.
  auto fp64_sweeps = [&](Half& hf, int count) -> int {
    for (int it = 0; it < count; ++it) {
      if (hf.tQ == GF32) {
        // the float32 sweeps' basis, widened (the float64 product then runs on one type)
        XKV_K(launch_widen((const float*)hf.Qcur, hf.Qa, (long)hf.cnt * nk, st));
        hf.Qcur = hf.Qa;
        hf.tQ = GF64;
      }
      XKV_K(gemm(gdesc(n, kb, n, 1, 0, GF64, hf.tQ, GF64, hf.w.C64, n, nn, hf.Qcur, kb, nk, hf.Ya, kb, nk, 1.0, 0.0,
                       hf.cnt), st));
      int e = cholqr(p, hf.w, hf.cnt, hf.Ya, GF64, hf.Qa, GF64, st);       // Qa = orth(Ya)
      if (e) return e;
      if (it + 1 == count) {
        e = cholqr(p, hf.w, hf.cnt, hf.Qa, GF64, hf.Ya, GF64, st);         // second pass: Ya = orth(Qa)
        if (e) return e;
        std::swap(hf.Qa, hf.Ya);                                           // Qa holds the basis
      }
      hf.Qcur = hf.Qa;
      hf.tQ = GF64;
    }
    return XKV_OK;
  };
  // 1.-2. Per half: Gram of every side (batched, at most kMaxPtrs layer pointers per launch),
  // its trace (total energy), then the block subspace iteration: float32 sweeps on a float32
  // copy of C, then float64 sweeps (CholeskyQR, CholeskyQR2 on the last sweep of a round).
  auto pre_work = [&](Half& hf) -> int {
    for (int s0 = hf.s0; s0 < hf.s0 + hf.cnt; s0 += per) {
      const int cnt = std::min(per, hf.s0 + hf.cnt - s0);
      PtrTable tab{};
      for (int s = 0; s < cnt; ++s)
        for (int l = 0; l < p.G; ++l) tab.p[s * p.G + l] = sides[s0 + s].layers[l];
      double* C = w.C64 + s0 * nn;
      float* C32 = w.C32 ? w.C32 + s0 * nn : nullptr;
      if (p.bf16) XKV_K(launch_gram_bf16(tab, cnt, p.G, sides[s0].ld_layer, p.T, p.d_kv, C, C32, st));
      else XKV_K(launch_gram_f32(tab, cnt, p.G, sides[s0].ld_layer, p.T, p.d_kv, C, C32, st));
    }
    XKV_K(launch_trace(hf.w.C64, nn, n, hf.cnt, hf.w.trace, st));
    XKV_K(launch_init_q(hf.w.Q32, n, kb, nk, hf.cnt, desc->seed, st));
    for (int it = 0; it < p.fp32_iters; ++it) {
      GemmDesc cq = gdesc(n, kb, n, 1, 0, GF32, GF32, GF32, hf.w.C32, n, nn, hf.w.Q32, kb, nk, hf.w.Y32, kb, nk, 1.0,
                          0.0, hf.cnt);
      cq.acc = GF32;   // float32 matrix cores for the float32 iterations
      XKV_K(gemm(cq, st));
      int e = cholqr(p, hf.w, hf.cnt, hf.w.Y32, GF32, hf.w.Q32, GF32, st);
      if (e) return e;
    }
    return fp64_sweeps(hf, p.fp64_iters);
  };
  int total_iters = p.fp32_iters + p.fp64_iters;

  // Pinned staging: H (down), packed reflectors and Ritz values (up), residual norms, traces
  // and info (down), wanted positions (up).
  const size_t refl = xkv_eigh_refl_doubles(kb);
  const size_t need_pin = (size_t)S * kk + (size_t)S * refl + (size_t)S * r + (size_t)S * r + (size_t)S + (size_t)S +
                          ((size_t)S * r + 1) / 2;
  if (ctx->upload_pending) {
    XKV_HIP(hipEventSynchronize(ctx->upload_done));
    ctx->upload_pending = false;
  }
  if (ctx->pin_doubles < need_pin) {
    if (ctx->pin) XKV_HIP(hipHostFree(ctx->pin));
    ctx->pin = nullptr;
    ctx->pin_doubles = 0;
    XKV_HIP(hipHostMalloc((void**)&ctx->pin, need_pin * sizeof(double), hipHostMallocDefault));
    ctx->pin_doubles = need_pin;
  }
  // From the first copy to or from the pinned staging on, an early error return (a
  // Cholesky breakdown, a failed host solve, a launch error) can leave such copies in
  // flight on `st`; the guard then marks them with upload_done, so that the next call on
  // this context waits for them before its host writes to the staging.
  struct PinGuard {
    xkv_ctx c;
    hipStream_t s;
    bool armed;
    ~PinGuard() {
      if (!armed) return;
      if (hipEventRecord(c->upload_done, s) == hipSuccess) c->upload_pending = true;
      else (void)hipStreamSynchronize(s);
    }
  } pin_guard{ctx, st, true};
  double* hH = ctx->pin;
  double* hRefl = hH + (size_t)S * kk;
  double* hTheta = hRefl + (size_t)S * refl;
  double* hRes = hTheta + (size_t)S * r;
  double* hTrace = hRes + (size_t)S * r;
  int* hinfo = (int*)(hTrace + S);
  int* hPos = (int*)(hTrace + 2 * S);

  // 3. Rayleigh-Ritz rounds.  After each, the Ritz residuals R = (C Q) Z - V_r diag(theta)
  //    bound the subspace error (per-pair sin-theta bounds, below).  Unconverged rounds add
  //    float64 sweeps.
  const double tol = desc->tol > 0 ? desc->tol : 1e-4;
  const int max_rounds = desc->max_rounds > 0 ? desc->max_rounds : 8;
  std::vector<std::vector<double>> evals(S, std::vector<double>(kb));
  std::vector<double> est(S, 0.0), relgap(S, 0.0);
  int rounds = 0;
  bool converged = false;
  // Host memory of the eigensolves, kept in the context: per side the value phase's state
  // (also the working memory of the first half of the vectors) and the working memory of the
  // second half of the vectors.
  if ((int)ctx->eig_side.size() < 2 * S) ctx->eig_side.resize(2 * S, xkv_eigh_scratch{});
  // The Rayleigh-Ritz matrix H = Q^T C Q of a half (and its info), copied down, then an event.
  auto rr_matrix = [&](Half& hf, int h, bool first) -> int {
    XKV_K(gemm(gdesc(n, kb, n, 1, 0, GF64, GF64, GF64, hf.w.C64, n, nn, hf.Qa, kb, nk, hf.Ya, kb, nk, 1.0, 0.0,
                     hf.cnt), st));
    // H = Q^T (C Q) is symmetric up to rounding (the host takes the mean of its triangles): the
    // upper tiles, mirrored, with K split as for W
    GemmDesc hd = gdesc(kb, kb, n, 1, 0, GF64, GF64, GF64, hf.Qa, kb, nk, hf.Ya, kb, nk, hf.w.H, kb, kk, 1.0, 0.0,
                        hf.cnt);
    sym_split(hd, n, hf.w.Wpart);
    XKV_K(gemm(hd, st));
    XKV_HIP(hipMemcpyAsync(hH + (size_t)hf.s0 * kk, hf.w.H, (size_t)hf.cnt * kk * sizeof(double),
                           hipMemcpyDeviceToHost, st));
    XKV_HIP(hipMemcpyAsync(hinfo + hf.s0, hf.w.info, hf.cnt * sizeof(int), hipMemcpyDeviceToHost, st));
    if (first)
      XKV_HIP(hipMemcpyAsync(hTrace + hf.s0, hf.w.trace, hf.cnt * sizeof(double), hipMemcpyDeviceToHost, st));
    XKV_HIP(hipEventRecord(ctx->half_done[h], st));
    return XKV_OK;
  };
  // The host eigensolves of a half: the value phase one thread per side, or two (a leader and a
  // worker sharing the reduction's row passes; the worker then packs the reflectors while the
  // leader runs the QR iteration) where every pair gets threads of its own and the side is
  // large enough to pay for a barrier per pass; all on at most ctx->host_threads threads.
  // The vector phase runs on the device (post_work): each side's rotation log is packed here
  // into the half's pinned staging, its reflector blocks and wanted positions into ctx->pin.
  const RitzGrouping rg = ritz_grouping();
  const int run_cap = rg.run_cap;
  // With the log in P > 1 pieces, side i of a half is P virtual sides i P + q of the rotation
  // kernel: piece 0 applied to the wanted unit vectors (padded to k_b columns), piece q > 0 to
  // the identity, each with meta of its own and k_b positions in the staging.
  const int P = ritz_parts(kb);
  std::vector<long long> meta(4 * (size_t)S, 0);
  size_t log_bytes[kMaxParts] = {}, pos_off[kMaxParts] = {};
  long long runs_total[kMaxParts] = {};
  auto run_threads = [&](int nthr, int ntask, auto&& task) {
    if (nthr <= 1) {
      for (int t = 0; t < ntask; ++t) task(t);
      return;
    }
    std::vector<std::thread> pool;
    for (int t0 = 0; t0 < nthr; ++t0)
      pool.emplace_back([&, t0]() {
        for (int t = t0; t < ntask; t += nthr) task(t);
      });
    for (auto& th : pool) th.join();
  };
  auto solve_half = [&](const Half& hf, int h) -> int {
    std::vector<int> erc(hf.cnt, 0), nruns(hf.cnt, 0);
    const bool paired = kb >= 256 && 2 * hf.cnt <= ctx->host_threads;
    auto finish = [&](int i) {   // after a side's values: its positions and run count
      const int s = hf.s0 + i;
      xkv_eigh_positions(&ctx->eig_side[2 * s], hPos + (size_t)s * r);
      nruns[i] = xkv_eigh_runs(&ctx->eig_side[2 * s], run_cap);
    };
    if (paired) {
      // 2 cnt tasks on 2 cnt threads, so both members of a pair run at once
      std::vector<xkv_eigh_pair> prs(hf.cnt, xkv_eigh_pair{});
      std::vector<int> wrc(hf.cnt, 0);
      run_threads(2 * hf.cnt, 2 * hf.cnt, [&](int t) {
        const int i = t / 2, tid = t % 2, s = hf.s0 + i;
        const int rc = xkv_eigh_values_pair(kb, hH + (size_t)s * kk, r, evals[s].data(), &ctx->eig_side[2 * s],
                                            &ctx->eig_side[2 * s + 1], &prs[i], tid, hRefl + (size_t)s * refl);
        (tid ? wrc[i] : erc[i]) = rc;
        if (tid == 0 && rc == 0) finish(i);
      });
      for (int i = 0; i < hf.cnt; ++i)
        if (erc[i] == 0 && wrc[i] != 0) erc[i] = wrc[i];
    } else {
      run_threads(std::min(hf.cnt, ctx->host_threads), hf.cnt, [&](int i) {
        const int s = hf.s0 + i;
        erc[i] = xkv_eigh_values(kb, hH + (size_t)s * kk, r, evals[s].data(), &ctx->eig_side[2 * s]);
        if (erc[i] == 0) {
          xkv_eigh_pack_reflectors(&ctx->eig_side[2 * s], hRefl + (size_t)s * refl);
          finish(i);
        }
      });
    }
    for (int i = 0; i < hf.cnt; ++i) {
      if (erc[i] == -4) return fail(XKV_ENUMERIC, "compress: non-finite Rayleigh-Ritz matrix on side %d", hf.s0 + i);
      if (erc[i]) return fail(XKV_ENUMERIC, "compress: host eigensolve failed on side %d (code %d)", hf.s0 + i, erc[i]);
    }
    // The half's log staging: meta (4 per side or virtual side: first run, first pair, first
    // group, groups) | runs (4 ints each) | groups (2 ints each, room for one per run) | (c, s)
    // pairs | with P > 1, the virtual sides' positions (k_b each).
    long long runs_tot = 0, rot_tot = 0;
    for (int i = 0; i < hf.cnt; ++i) {
      const int s = hf.s0 + i;
      meta[4 * s] = runs_tot;
      meta[4 * s + 1] = rot_tot;
      meta[4 * s + 2] = runs_tot;
      runs_tot += nruns[i];
      rot_tot += ctx->eig_side[2 * s].log.n;
    }
    const size_t meta_b = 32 * (size_t)P * hf.cnt, runs_b = 16 * (size_t)runs_tot, grp_b = 8 * (size_t)runs_tot;
    const size_t pos_b = P > 1 ? 4 * (size_t)P * hf.cnt * kb : 0;
    const size_t need = meta_b + runs_b + grp_b + 16 * (size_t)rot_tot + pos_b;
    pos_off[h] = meta_b + runs_b + grp_b + 16 * (size_t)rot_tot;
    if (ctx->lpin_bytes[h] < need) {
      // no copy reads this half's staging now: each compression round ends with a stream
      // synchronisation, and an earlier call's copies are waited for on entry
      if (ctx->lpin[h]) XKV_HIP(hipHostFree(ctx->lpin[h]));
      ctx->lpin[h] = nullptr;
      ctx->lpin_bytes[h] = 0;
      const size_t want = need + need / 4;
      XKV_HIP(hipHostMalloc(&ctx->lpin[h], want, hipHostMallocDefault));
      ctx->lpin_bytes[h] = want;
    }
    char* lp = (char*)ctx->lpin[h];
    run_threads(std::min(hf.cnt, ctx->host_threads), hf.cnt, [&](int i) {
      const int s = hf.s0 + i;
      int* rs = (int*)(lp + meta_b) + 4 * meta[4 * s];
      xkv_eigh_pack_log(&ctx->eig_side[2 * s], run_cap, rs, (double*)(lp + meta_b + runs_b + grp_b) + 2 * meta[4 * s + 1]);
      const int* gs = (int*)(lp + meta_b + runs_b) + 2 * meta[4 * s + 2];
      meta[4 * s + 3] = xkv_eigh_group_runs(rs, nruns[i], rg.per_group, rg.spread, rg.max_steps, (int*)gs);
      if (P > 1) {
        int bnd[5];
        xkv_eigh_split_groups(rs, gs, (int)meta[4 * s + 3], rg.overhead, P, bnd);
        long long* vm = (long long*)lp + 4 * (size_t)i * P;
        int* vp = (int*)(lp + pos_off[h]) + (size_t)i * P * kb;
        for (int q = 0; q < P; ++q) {
          vm[4 * q] = meta[4 * s];
          vm[4 * q + 1] = meta[4 * s + 1];
          vm[4 * q + 2] = meta[4 * s + 2] + bnd[q];
          vm[4 * q + 3] = bnd[q + 1] - bnd[q];
          for (int j = 0; j < kb; ++j) vp[(size_t)q * kb + j] = (q == 0 && j < r) ? hPos[(size_t)s * r + j] : j;
        }
      }
    });
    if (P == 1) std::memcpy(lp, meta.data() + 4 * (size_t)hf.s0, meta_b);
    log_bytes[h] = need;
    runs_total[h] = runs_tot;
    for (int i = 0; i < hf.cnt; ++i)
      std::memcpy(hTheta + (size_t)(hf.s0 + i) * r, evals[hf.s0 + i].data(), r * sizeof(double));
    return XKV_OK;
  };
  // The Ritz vectors Z of a half on the device (the rotations of each side's QR iteration applied
  // to its wanted unit vectors, then its reflectors, last block first, as S2 -= Y (T (Y^T S2))),
  // then V_r = Q Z and the residual of every Ritz pair.  With the log in P pieces, piece q's
  // product S_q comes out of the rotation kernel as a k_b x k_b matrix (piece 0 applied to the
  // wanted unit vectors, its first r columns used) and Z = S_{P-1} ... S_1 S_0 E by P - 1 float64
  // products, the last of them written to Z.
  auto post_work = [&](Half& hf, int h) -> int {
    const int NBG = XKV_EIGH_NBG;
    XKV_HIP(hipMemcpyAsync(hf.w.Rf, hRefl + (size_t)hf.s0 * refl, (size_t)hf.cnt * refl * sizeof(double),
                           hipMemcpyHostToDevice, st));
    if (P == 1)
      XKV_HIP(hipMemcpyAsync(hf.w.pos, hPos + (size_t)hf.s0 * r, (size_t)hf.cnt * r * sizeof(int),
                             hipMemcpyHostToDevice, st));
    if (ctx->ldev_bytes[h] < log_bytes[h]) {
      // the previous reader of this half's device log finished before its round's synchronisation
      if (ctx->ldev[h]) XKV_HIP(hipFree(ctx->ldev[h]));
      ctx->ldev[h] = nullptr;
      ctx->ldev_bytes[h] = 0;
      const size_t want = log_bytes[h] + log_bytes[h] / 4;
      XKV_HIP(hipMalloc(&ctx->ldev[h], want));
      ctx->ldev_bytes[h] = want;
    }
    XKV_HIP(hipMemcpyAsync(ctx->ldev[h], ctx->lpin[h], log_bytes[h], hipMemcpyHostToDevice, st));
    const char* ld = (const char*)ctx->ldev[h];
    const size_t meta_b = 32 * (size_t)P * hf.cnt;
    const size_t runs_tot = (size_t)runs_total[h];
    const int4* d_runs = (const int4*)(ld + meta_b);
    const int2* d_groups = (const int2*)(ld + meta_b + 16 * runs_tot);
    const double2* d_cs = (const double2*)(ld + meta_b + 24 * runs_tot);
    if (P == 1) {
      XKV_K(launch_ritz_rotate(d_runs, d_cs, d_groups, (const long long*)ld, hf.w.pos, kb, r, hf.w.Z, (long)kb * r,
                               hf.w.Zs, ritz_scratch_doubles(kb, r), hf.cnt, st));
    } else {
      XKV_K(launch_ritz_rotate(d_runs, d_cs, d_groups, (const long long*)ld, (const int*)(ld + pos_off[h]), kb, kb,
                               hf.w.Zseg, kk, hf.w.Zsegs, ritz_scratch_doubles(kb, kb), P * hf.cnt, st));
      // side i's piece q at Zseg + (i P + q) k_b^2; the products alternate between Z (ld r) and
      // piece 0's memory (ld r once piece 0 has been read), ending in Z.  P is 2 or 4, so the
      // first product, which reads piece 0, writes Z.
      const long sP = (long)P * kk;
      const double* in = hf.w.Zseg;
      long ld_in = kb, s_in = sP;
      for (int q = 1; q < P; ++q) {
        const bool into_z = (P - 1 - q) % 2 == 0;
        double* out = into_z ? hf.w.Z : hf.w.Zseg;
        const long s_out = into_z ? (long)kb * r : sP;
        XKV_K(gemm(gdesc(kb, r, kb, 0, 0, GF64, GF64, GF64, hf.w.Zseg + (size_t)q * kk, kb, sP, in, ld_in, s_in, out, r,
                         s_out, 1.0, 0.0, hf.cnt), st));
        in = out;
        ld_in = r;
        s_in = s_out;
      }
    }
    const int nref = kb - 2;
    const int nblk = nref > 0 ? (nref + NBG - 1) / NBG : 0;
    const size_t ytot = refl - (size_t)nblk * NBG * NBG;
    double* W1 = hf.w.Wb;
    double* W2 = hf.w.Wb + (size_t)NBG * r;
    const long sWb = 2L * NBG * r;
    for (int b = nblk - 1; b >= 0; --b) {
      const int r0 = NBG * b + 1, M = kb - r0;
      const size_t yoff = (size_t)NBG * ((size_t)b * (kb - 1) - (size_t)NBG * b * (b - 1) / 2);
      const double* Y = hf.w.Rf + yoff;
      const double* T = hf.w.Rf + ytot + (size_t)b * NBG * NBG;
      double* S2 = hf.w.Z + (size_t)r0 * r;
      XKV_K(gemm(gdesc(NBG, r, M, 1, 0, GF64, GF64, GF64, Y, NBG, (long)refl, S2, r, (long)kb * r, W1, r, sWb, 1.0,
                       0.0, hf.cnt), st));
      XKV_K(gemm(gdesc(NBG, r, NBG, 0, 0, GF64, GF64, GF64, T, NBG, (long)refl, W1, r, sWb, W2, r, sWb, 1.0, 0.0,
                       hf.cnt), st));
      XKV_K(gemm(gdesc(M, r, NBG, 0, 0, GF64, GF64, GF64, Y, NBG, (long)refl, W2, r, sWb, S2, r, (long)kb * r, -1.0,
                       1.0, hf.cnt), st));
    }
    XKV_HIP(hipMemcpyAsync(hf.w.theta, hTheta + (size_t)hf.s0 * r, (size_t)hf.cnt * r * sizeof(double),
                           hipMemcpyHostToDevice, st));
    XKV_K(gemm(gdesc(n, r, kb, 0, 0, GF64, GF64, GF64, hf.Qa, kb, nk, hf.w.Z, r, (long)kb * r, hf.w.Vr, r,
                     (long)n * r, 1.0, 0.0, hf.cnt), st));
    XKV_K(gemm(gdesc(n, r, kb, 0, 0, GF64, GF64, GF64, hf.Ya, kb, nk, hf.w.Z, r, (long)kb * r, hf.w.YZ, r,
                     (long)n * r, 1.0, 0.0, hf.cnt), st));
    XKV_K(launch_ritz_residual(hf.w.YZ, hf.w.Vr, hf.w.theta, n, r, hf.w.res2, hf.cnt, st));
    XKV_HIP(hipMemcpyAsync(hRes + (size_t)hf.s0 * r, hf.w.res2, (size_t)hf.cnt * r * sizeof(double),
                           hipMemcpyDeviceToHost, st));
    return XKV_OK;
  };
  // Bt = V_r and the projection A = X V_r of sides [s_begin, s_end).  Every part but the last
  // is projected as soon as its first round's V_r is on the device, in the GPU's wait for the
  // later parts' eigenvalues; a later round projects every side again.
  const long nr = (long)n * r;
  auto project = [&](int s_begin, int s_end) -> int {
    for (int s0 = s_begin; s0 < s_end; s0 += per) {
      const int cnt = std::min(per, s_end - s0);
      PtrTable bt{}, aout{}, lay{};
      for (int s = 0; s < cnt; ++s) {
        bt.p[s] = sides[s0 + s].Bt;
        aout.p[s] = sides[s0 + s].A;
        for (int l = 0; l < p.G; ++l) lay.p[s * p.G + l] = sides[s0 + s].layers[l];
      }
      const size_t es = p.bf16 ? 2 : 4;
      void* VrT = (char*)w.VrT + (size_t)s0 * nr * es;
      XKV_K(launch_vr_outputs(w.Vr + s0 * nr, nr, n, r, bt, p.bf16, VrT, nr, cnt, st));
      if (p.bf16)
        XKV_K(launch_project_bf16(lay, cnt, p.G, sides[s0].ld_layer, p.T, p.d_kv, (const uint16_t*)VrT, nr, r, aout,
                                  st));
      else
        XKV_K(launch_project_f32(lay, cnt, p.G, sides[s0].ld_layer, p.T, p.d_kv, (const float*)VrT, nr, r, aout, st));
    }
    return XKV_OK;
  };
  for (int h = 0; h < nh; ++h) {
    rc = pre_work(hv[h]);
    if (rc) return rc;
    rc = rr_matrix(hv[h], h, true);
    if (rc) return rc;
  }
  // Landmarks of the sides that ask for them: they depend on the keys alone, so they go
  // behind the Rayleigh-Ritz products and run while the host solves.
  if (any_lm) {
    PtrTable lay{}, lmo{};
    int cnt = 0;
    auto flush = [&]() -> int {
      if (cnt == 0) return XKV_OK;
      XKV_K(launch_landmarks(lay, cnt, p.G, sides[0].ld_layer, p.T, desc->n_kv_heads, desc->head_dim, desc->chunk,
                             desc->rope_theta, lmo, p.bf16, st));
      cnt = 0;
      return XKV_OK;
    };
    const long per_layer = (long)desc->n_kv_heads * (p.T / desc->chunk) * desc->head_dim * (p.bf16 ? 2 : 4);
    for (int s = 0; s < S; ++s) {
      if (!sides[s].landmarks) continue;
      if ((cnt + 1) * p.G > kMaxPtrs) {
        rc = flush();
        if (rc) return rc;
      }
      for (int l = 0; l < p.G; ++l) {
        lay.p[cnt * p.G + l] = sides[s].layers[l];
        lmo.p[cnt * p.G + l] = (char*)sides[s].landmarks + l * per_layer;
      }
      ++cnt;
    }
    rc = flush();
    if (rc) return rc;
  }
  for (;;) {
    ++rounds;
    for (int h = 0; h < nh; ++h) {
      Half& hf = hv[h];
      XKV_HIP(hipEventSynchronize(ctx->half_done[h]));   // H of this half is on the host
      for (int i = 0; i < hf.cnt; ++i)
        if (hinfo[hf.s0 + i])
          return fail(XKV_ENUMERIC, "compress: Cholesky breakdown on side %d (rank of X below %d?)", hf.s0 + i, kb);
      rc = solve_half(hf, h);
      if (rc) return rc;
      rc = post_work(hf, h);
      if (rc) return rc;
      if (h + 1 < nh && rounds == 1) {
        rc = project(hf.s0, hf.s0 + hf.cnt);
        if (rc) return rc;
      }
    }
    XKV_HIP(hipEventRecord(ctx->upload_done, st));
    ctx->upload_pending = true;
    XKV_HIP(hipStreamSynchronize(st));
    ctx->upload_pending = false;
    converged = true;
    for (int s = 0; s < S; ++s) {
      // Each Ritz pair (theta_i, v_i) with residual r_i = C v_i - theta_i v_i has
      // ||(I - P_exact) v_i|| <= ||r_i|| / (theta_i - lambda_r+1) (P_exact the spectral
      // projector of the r largest eigenvalues; lambda_r+1 estimated by the Ritz value
      // theta_r+1), so ||P - P_exact||_F = sqrt(2) ||(I - P_exact) V_r||_F is bounded by
      // sqrt(2 sum_i ||r_i||^2 / (theta_i - theta_r+1)^2).
      const double th_r = evals[s][r - 1];
      const double th_next = r < kb ? evals[s][r] : 0.0;
      const double gap = th_r - th_next;
      relgap[s] = th_r > 0 ? gap / th_r : 0.0;
      double w2 = 0.0;
      bool gap_ok = gap > 0;
      for (int i = 0; i < r && gap_ok; ++i) {
        const double gi = evals[s][i] - th_next;
        w2 += hRes[(size_t)s * r + i] / (gi * gi);
      }
      // A block that spans the whole space gives the exact eigenvectors.
      est[s] = (kb == n) ? 0.0 : (gap_ok ? std::sqrt(2.0 * w2) : INFINITY);
      if (!(est[s] <= tol)) converged = false;
    }
    if (converged || rounds >= max_rounds) break;
    // Sweeps of the next round: an unconverged side's error shrinks by about
    // rho = lambda_kb+1 / lambda_r per sweep, estimated by theta_kb / theta_r (the block's
    // smallest Ritz value over the r-th; a Ritz value lies below its eigenvalue, so the
    // estimate can be optimistic), so est rho^m <= tol / 2 takes m = log(tol / (2 est)) /
    // log(rho) sweeps, taken with a margin of 1.5 m + 2.  At least the default count; the
    // default where rho is not below 1, the estimate is not finite (no gap at r) or the
    // prediction exceeds 32 sweeps (a side that one round cannot bring to tol, such as one
    // whose r-th eigenvalue lies in a flat noise bulk, gains nothing from more).
    int next = p.fp32_iters + p.fp64_iters;
    for (int s = 0; s < S; ++s) {
      if (est[s] <= tol || !std::isfinite(est[s]) || !(evals[s][r - 1] > 0.0)) continue;
      const double rho = evals[s][kb - 1] / evals[s][r - 1];
      if (!(rho > 0.0 && rho < 0.999)) continue;
      const double m = std::ceil(1.5 * std::log(tol / (2.0 * est[s])) / std::log(rho)) + 2.0;
      if (m > next && m <= 32.0) next = (int)m;
    }
    for (int h = 0; h < nh; ++h) {
      rc = fp64_sweeps(hv[h], next);
      if (rc) return rc;
      rc = rr_matrix(hv[h], h, false);
      if (rc) return rc;
    }
    total_iters += next;
  }
  pin_guard.armed = false;   // the last round ended with a stream synchronisation
  for (int s = 0; s < S; ++s) {
    if (sides[s].eigvals) std::memcpy(sides[s].eigvals, evals[s].data(), r * sizeof(double));
    if (sides[s].stats) {
      sides[s].stats[0] = est[s];
      sides[s].stats[1] = relgap[s];
      sides[s].stats[2] = total_iters;
      sides[s].stats[3] = rounds;
      sides[s].stats[4] = hTrace[s];
    }
  }

  // 4. The stored Bt = V_r and the projection A = X V_r.
  for (int s = 0; s < S; ++s)
    if (sides[s].Vr64)
      XKV_HIP(hipMemcpyAsync(sides[s].Vr64, w.Vr + (long)s * n * r, (size_t)n * r * sizeof(double),
                             hipMemcpyDeviceToDevice, st));
  rc = project(nh > 1 && rounds == 1 ? hv[nh - 1].s0 : 0, S);
  if (rc) return rc;
  if (!converged)
    return fail(XKV_ENOTCONV, "compress: subspace error estimate above %.1e after %d rounds (%d sweeps); "
                "outputs are written", tol, rounds, total_iters);
  return XKV_OK;
}

extern "C" int xkv_compress_group(xkv_ctx ctx, const xkv_compress_desc* desc, const xkv_side* side, void* ws,
                                  size_t ws_bytes, void* stream) {
  return xkv_compress_sides(ctx, desc, 1, side, ws, ws_bytes, stream);
}

extern "C" int xkv_gram(const void* const* layers, int n_sides, long ld_layer, int T, int G, int d_kv, int dtype,
                        double* C, void* stream) {
  if (!layers || !C || n_sides <= 0 || T <= 0 || G <= 0 || G > 16 || d_kv <= 0 || d_kv % 8 || ld_layer < d_kv ||
      n_sides * G > xkv::kMaxPtrs)
    return fail(XKV_EINVAL, "xkv_gram: bad arguments");
  if (dtype != XKV_F32 && dtype != XKV_BF16) return fail(XKV_EINVAL, "xkv_gram: unknown dtype");
  xkv::PtrTable tab{};
  for (int l = 0; l < n_sides * G; ++l) {
    if (!layers[l]) return fail(XKV_EINVAL, "xkv_gram: layer pointer %d is NULL", l);
    if (dtype == XKV_BF16 && (!aligned16(layers[l]) || ld_layer % 8))
      return fail(XKV_EINVAL, "xkv_gram: bf16 layers need 16-byte alignment and ld %% 8 == 0");
    tab.p[l] = layers[l];
  }
  hipStream_t st = (hipStream_t)stream;
  if (dtype == XKV_BF16) XKV_K(xkv::launch_gram_bf16(tab, n_sides, G, ld_layer, T, d_kv, C, nullptr, st));
  else XKV_K(xkv::launch_gram_f32(tab, n_sides, G, ld_layer, T, d_kv, C, nullptr, st));
  return XKV_OK;
}

extern "C" int xkv_topk(const float* scores, int rows, int n_cand, long ld, int k, int* sel, void* stream) {
  if (!scores || !sel || rows <= 0 || n_cand <= 0 || ld < n_cand || k <= 0 || n_cand > 32768)
    return fail(XKV_EINVAL, "xkv_topk: bad arguments");
  XKV_K(xkv::launch_topk(scores, rows, n_cand, ld, k, sel, (hipStream_t)stream));
  return XKV_OK;
}

// ---------------------------------------------------------------------------
// Selective Reconstruction decode
// ---------------------------------------------------------------------------
namespace {

int plan_sr(const xkv_sr_args* a, xkv::SrParams* P, size_t* ws_need) {
  if (!a) return fail(XKV_EINVAL, "sr: args is NULL");
  if (a->batch <= 0 || a->n_kv_heads <= 0 || a->n_q_heads <= 0 || a->n_q_heads % a->n_kv_heads)
    return fail(XKV_EINVAL, "sr: batch/heads invalid (n_q_heads must be a multiple of n_kv_heads)");
  const int grp = a->n_q_heads / a->n_kv_heads;
  if (grp > 8) return fail(XKV_EUNSUPPORTED, "sr: at most 8 query heads per KV head");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(XKV_EUNSUPPORTED, "sr: head_dim must be 64 or 128");
  if (a->chunk < 8 || a->chunk > 64 || (a->chunk & (a->chunk - 1)))
    return fail(XKV_EUNSUPPORTED, "sr: chunk must be a power of two in [8, 64]");
  if (a->T <= 0 || a->T % a->chunk) return fail(XKV_EINVAL, "sr: T must be a positive multiple of chunk");
  if (a->n_sink < 0 || a->n_local < 0 || a->n_gen < 0 || a->top_k < 0)
    return fail(XKV_EINVAL, "sr: negative sizes");
  if (a->n_sink + a->n_local > a->T) return fail(XKV_EINVAL, "sr: n_sink + n_local must not exceed T");
  if (a->dtype != XKV_F32 && a->dtype != XKV_BF16) return fail(XKV_EINVAL, "sr: unknown dtype");
  if (a->r_k <= 0 || a->r_v < 0) return fail(XKV_EINVAL, "sr: r_k must be positive and r_v >= 0");
  if (a->r_v % 2) return fail(XKV_EUNSUPPORTED, "sr: r_v must be even");
  const int d_kv = a->n_kv_heads * a->head_dim;
  const int n_cand = std::max(0, (a->T - a->n_local + a->chunk - 1) / a->chunk);
  const int k_eff = std::min(a->top_k, n_cand);
  if (a->n_sink + a->n_local + a->n_gen == 0 && k_eff == 0) return fail(XKV_EINVAL, "sr: nothing to attend");
  const int mfma = a->dtype == XKV_BF16 && a->head_dim == 128 && a->r_k % 128 == 0 &&
                   (a->r_v == a->r_k || a->r_v == 0) && a->r_k <= xkv::MAX_RANK_MFMA;
  const int exact_v = mfma && a->r_v == 0;   // xK-SR on the matrix-core key path
  const int cps = 64 / a->chunk;   // chunks per attend block of 64 rows
  const int n_splits = (k_eff + cps - 1) / cps;
  if (n_cand > 32768) return fail(XKV_EUNSUPPORTED, "sr: at most 32768 candidate chunks per head");
  const int n_exact = std::max(1, (a->n_sink + a->n_local + a->n_gen + 15) / 16);   // 16-row tiles
  const int max_blocks = (mfma && !exact_v) ? 1088 : 257;   // rank-space / value-space merge
  if (n_splits + n_exact > max_blocks)
    return fail(XKV_EUNSUPPORTED, "sr: selected chunks plus exact-row tiles exceed %d attend blocks per head",
                max_blocks);
  {
    // Exact tails and new tokens are read 8 elements at a time.
    const long q = a->dtype == XKV_BF16 ? 8 : 4;
    if (!aligned16(a->k_tail) || !aligned16(a->v_tail) || a->ld_tail % q || a->bstride_tail % q ||
        (a->k_new && (!aligned16(a->k_new) || !aligned16(a->v_new) || a->bstride_new % q)))
      return fail(XKV_EINVAL, "sr: tails and new tokens need 16-byte alignment and strides of 16 bytes");
  }
  if (!a->q || !a->A_k || !a->Bt_k || !a->landmarks || !a->k_tail || !a->v_tail || !a->out || !a->sel)
    return fail(XKV_EINVAL, "sr: a required pointer is NULL");
  if (a->r_v > 0 ? (!a->A_v || !a->Bt_v) : !a->V_full) return fail(XKV_EINVAL, "sr: value pointers missing");
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) return fail(XKV_EINVAL, "sr: give both k_new and v_new or neither");
  if (a->ld_A_k < a->r_k || a->ld_Bt_k < a->r_k || a->ld_tail < d_kv) return fail(XKV_EINVAL, "sr: leading dimension too small");
  if (a->r_v > 0 && (a->ld_A_v < a->r_v || a->ld_Bt_v < a->r_v)) return fail(XKV_EINVAL, "sr: value leading dimension too small");
  if (a->r_v == 0 && a->ld_V < d_kv) return fail(XKV_EINVAL, "sr: ld_V too small");
  const int vdim = (mfma && !exact_v) ? a->r_v : a->head_dim;
  if (mfma) {
    // matrix-core path: 16-byte loads of A and Bt rows
    if (!aligned16(a->A_k) || !aligned16(a->Bt_k) || a->ld_A_k % 8 || a->ld_Bt_k % 8 || a->bstride_A_k % 8 ||
        a->bstride_Bt_k % 8 ||
        (!exact_v && (!aligned16(a->A_v) || !aligned16(a->Bt_v) || a->ld_A_v % 8 || a->ld_Bt_v % 8 ||
                      a->bstride_A_v % 8 || a->bstride_Bt_v % 8)))
      return fail(XKV_EINVAL, "sr: bf16 A/Bt need 16-byte alignment and strides that are multiples of 8");
    // exact values: rows gathered 16 bytes at a time
    if (exact_v && (!aligned16(a->V_full) || a->ld_V % 8 || a->bstride_V % 8))
      return fail(XKV_EINVAL, "sr: bf16 V_full needs 16-byte alignment and strides that are multiples of 8");
  }
  if (!aligned16(a->landmarks) || a->bstride_lm % (a->dtype == XKV_BF16 ? 8 : 4))
    return fail(XKV_EINVAL, "sr: landmarks need 16-byte alignment");

  xkv::SrParams& p = *P;
  std::memset(&p, 0, sizeof(p));
  p.batch = a->batch; p.Hq = a->n_q_heads; p.Hkv = a->n_kv_heads; p.d = a->head_dim; p.T = a->T;
  p.n_gen = a->n_gen; p.chunk = a->chunk; p.top_k = a->top_k; p.n_sink = a->n_sink; p.n_local = a->n_local;
  p.r_k = a->r_k; p.r_v = a->r_v; p.n_cand = n_cand; p.n_chunks = a->T / a->chunk; p.k_eff = k_eff;
  p.n_splits = n_splits; p.n_exact = n_exact; p.grp = grp; p.cps = cps; p.mfma = mfma; p.exact_v = exact_v; p.vdim = vdim;
  p.q_pos = a->n_gen > 0 ? (long)a->T + a->n_gen - 1 : a->T;
  // Scoring blocks per head: about 128 candidates each, at most 64.
  p.score_blocks = std::max(1, std::min(64, (n_cand + 127) / 128));
  p.ld_sc = (n_cand + 3) & ~3;
  p.fuse_topk = 0;   // set by the combined entry points (fuse_selection)
  p.scale = a->scale; p.theta = a->rope_theta;
  for (int i = 0; i < a->head_dim / 2; ++i)
    p.turns[i] = std::pow(a->rope_theta, -2.0 * i / a->head_dim) / (2.0 * M_PI);
  p.q = a->q;
  p.A_k = a->A_k; p.ld_A_k = a->ld_A_k; p.bs_A_k = a->bstride_A_k;
  p.Bt_k = a->Bt_k; p.ld_Bt_k = a->ld_Bt_k; p.bs_Bt_k = a->bstride_Bt_k;
  p.A_v = a->A_v; p.ld_A_v = a->ld_A_v; p.bs_A_v = a->bstride_A_v;
  p.Bt_v = a->Bt_v; p.ld_Bt_v = a->ld_Bt_v; p.bs_Bt_v = a->bstride_Bt_v;
  p.V_full = a->V_full; p.ld_V = a->ld_V; p.bs_V = a->bstride_V;
  p.lm = a->landmarks; p.bs_lm = a->bstride_lm;
  p.k_tail = a->k_tail; p.v_tail = a->v_tail; p.ld_tail = a->ld_tail; p.bs_tail = a->bstride_tail;
  p.k_new = a->k_new; p.v_new = a->v_new; p.bs_new = a->bstride_new;
  p.out = a->out;
  p.sel = a->sel;

  Carver c(nullptr);
  const size_t bh = (size_t)a->batch * a->n_kv_heads;
  c.take<float>(bh * std::max((n_cand + 3) & ~3, 4));
  c.take<float>(bh * std::max(n_splits, 1) * grp * (2 + vdim));
  c.take<float>(bh * n_exact * grp * (2 + a->head_dim));
  *ws_need = c.off;
  return XKV_OK;
}

void bind_sr_ws(xkv::SrParams* p, void* ws) {
  Carver c(ws);
  const size_t bh = (size_t)p->batch * p->Hkv;
  p->scores = c.take<float>(bh * std::max(p->ld_sc, 4));
  p->part = c.take<float>(bh * std::max(p->n_splits, 1) * p->grp * (2 + p->vdim));
  p->part_ex = c.take<float>(bh * p->n_exact * p->grp * (2 + p->d));
}

// The combined decode entry points let the matrix-core attend kernel select the top-k
// itself (one launch fewer) when its grid fits the device's compute units in one round:
// each attend block then repeats the selection, which a second round of blocks would pay
// again.  The separate xkv_sr_select / xkv_sr_attend calls keep `sel` as their hand-off.
void fuse_selection(xkv_ctx ctx, xkv::SrParams* P) {
  P->fuse_topk = P->mfma && P->k_eff > 0 && P->n_cand <= 16384 &&
                 (long)P->Hkv * P->n_splits * P->batch <= (long)ctx->n_cu;
}

int sr_prepare(xkv_ctx ctx, const xkv_sr_args* a, void* ws, size_t ws_bytes, xkv::SrParams* P) {
  if (!ctx) return fail(XKV_EINVAL, "sr: ctx is NULL");
  size_t need = 0;
  int rc = plan_sr(a, P, &need);
  if (rc) return rc;
  if (!ws || ws_bytes < need) return fail(XKV_EWORKSPACE, "sr: workspace %zu bytes < %zu", ws_bytes, need);
  bind_sr_ws(P, ws);
  return XKV_OK;
}

}  // namespace

extern "C" int xkv_sr_ws_size(const xkv_sr_args* args, size_t* bytes) {
  if (!bytes) return fail(XKV_EINVAL, "xkv_sr_ws_size: bytes is NULL");
  xkv::SrParams P;
  return plan_sr(args, &P, bytes);
}

extern "C" int xkv_sr_select(xkv_ctx ctx, const xkv_sr_args* args, void* ws, size_t ws_bytes, void* stream) {
  xkv::SrParams P;
  int rc = sr_prepare(ctx, args, ws, ws_bytes, &P);
  if (rc) return rc;
  // The score kernel always runs: it also appends the new token and attends the exact rows.
  XKV_K(xkv::launch_sr_score(P, args->dtype == XKV_BF16, (hipStream_t)stream));
  XKV_K(xkv::launch_sr_topk(P, args->dtype == XKV_BF16, (hipStream_t)stream));
  return XKV_OK;
}

extern "C" int xkv_sr_attend(xkv_ctx ctx, const xkv_sr_args* args, void* ws, size_t ws_bytes, void* stream) {
  xkv::SrParams P;
  int rc = sr_prepare(ctx, args, ws, ws_bytes, &P);
  if (rc) return rc;
  XKV_K(xkv::launch_sr_attend(P, args->dtype == XKV_BF16, (hipStream_t)stream));
  XKV_K(xkv::launch_sr_merge(P, (hipStream_t)stream));
  return XKV_OK;
}

extern "C" int xkv_sr_decode(xkv_ctx ctx, const xkv_sr_args* args, void* ws, size_t ws_bytes, void* stream) {
  xkv::SrParams P;
  int rc = sr_prepare(ctx, args, ws, ws_bytes, &P);
  if (rc) return rc;
  fuse_selection(ctx, &P);
  const int bf16 = args->dtype == XKV_BF16;
  hipStream_t st = (hipStream_t)stream;
  XKV_K(xkv::launch_sr_score(P, bf16, st));
  XKV_K(xkv::launch_sr_topk(P, bf16, st));
  XKV_K(xkv::launch_sr_attend(P, bf16, st));
  XKV_K(xkv::launch_sr_merge(P, st));
  return XKV_OK;
}

extern "C" int xkv_sr_decode_layers(xkv_ctx ctx, int n_layers, const xkv_sr_args* args, void* ws, size_t ws_bytes,
                                    void* stream, void* const* attend_events) {
  if (n_layers <= 0 || !args) return fail(XKV_EINVAL, "xkv_sr_decode_layers: need n_layers > 0 and args");
  std::vector<xkv::SrParams> P(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    int rc = sr_prepare(ctx, &args[l], ws, ws_bytes, &P[l]);
    if (rc) return rc;
    fuse_selection(ctx, &P[l]);
  }
  hipStream_t st = (hipStream_t)stream;
  for (int l = 0; l < n_layers; ++l) {
    const int bf16 = args[l].dtype == XKV_BF16;
    xkv::SrParams& p = P[l];
    XKV_K(xkv::launch_sr_score(p, bf16, st));
    XKV_K(xkv::launch_sr_topk(p, bf16, st));
    XKV_K(xkv::launch_sr_attend(p, bf16, st, attend_events ? (hipEvent_t)attend_events[2 * l] : nullptr,
                                attend_events ? (hipEvent_t)attend_events[2 * l + 1] : nullptr));
    XKV_K(xkv::launch_sr_merge(p, st));
  }
  return XKV_OK;
}

extern "C" int xkv_sr_decode_layers_noalloc(xkv_ctx ctx, int n_layers, const xkv_sr_args* args, void* stream) {
  if (!ctx) return fail(XKV_EINVAL, "xkv_sr_decode_layers_noalloc: ctx is NULL");
  if (n_layers <= 0 || !args) return fail(XKV_EINVAL, "xkv_sr_decode_layers_noalloc: need n_layers > 0 and args");
  void* ws = xkv::sr_scratch_ptr(ctx->device);
  if (!ws) return fail(XKV_EHIP, "xkv_sr_decode_layers_noalloc: no decode scratch on device %d", ctx->device);
  std::vector<xkv::SrParams> P(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    size_t need = 0;
    int rc = plan_sr(&args[l], &P[l], &need);
    if (rc) return rc;
    if (need > xkv::kSrScratchBytes)
      return fail(XKV_EWORKSPACE, "xkv_sr_decode_layers_noalloc: layer %d needs %zu bytes of scratch, above the "
                  "library's %zu (use xkv_sr_decode_layers with a workspace)", l, need, xkv::kSrScratchBytes);
    bind_sr_ws(&P[l], ws);
    fuse_selection(ctx, &P[l]);
  }
  hipStream_t st = (hipStream_t)stream;
  for (int l = 0; l < n_layers; ++l) {
    const int bf16 = args[l].dtype == XKV_BF16;
    XKV_K(xkv::launch_sr_score(P[l], bf16, st));
    XKV_K(xkv::launch_sr_topk(P[l], bf16, st));
    XKV_K(xkv::launch_sr_attend(P[l], bf16, st, nullptr, nullptr));
    XKV_K(xkv::launch_sr_merge(P[l], st));
  }
  return XKV_OK;
}

// ---------------------------------------------------------------------------
// Tokens appended after a compressed prefix
// ---------------------------------------------------------------------------
namespace {

int check_append(const xkv_append_args* a, size_t* ws_need) {
  if (!a) return fail(XKV_EINVAL, "append: args is NULL");
  if (a->m <= 0 || a->pos0 < 0 || a->G <= 0 || a->G > 16 || a->d_kv <= 0 || a->d_kv % 8 || a->r <= 0 ||
      a->r > a->G * a->d_kv)
    return fail(XKV_EINVAL, "append: bad sizes (m=%d, G=%d, d_kv=%d, r=%d)", a->m, a->G, a->d_kv, a->r);
  if (a->dtype != XKV_F32 && a->dtype != XKV_BF16) return fail(XKV_EINVAL, "append: unknown dtype");
  if (!a->layers || !a->Bt || !a->A_new) return fail(XKV_EINVAL, "append: a required pointer is NULL");
  if (a->ld_layer < a->d_kv) return fail(XKV_EINVAL, "append: ld_layer too small");
  for (int l = 0; l < a->G; ++l) {
    if (!a->layers[l]) return fail(XKV_EINVAL, "append: layer pointer %d is NULL", l);
    if (a->dtype == XKV_BF16 && (!aligned16(a->layers[l]) || a->ld_layer % 8))
      return fail(XKV_EINVAL, "append: bf16 rows need 16-byte alignment and ld_layer %% 8 == 0");
  }
  if ((long)a->m * a->ld_layer >= (1L << 31)) return fail(XKV_EINVAL, "append: m * ld_layer too large");
  if (a->landmarks_new) {
    if (a->n_kv_heads <= 0 || a->head_dim <= 0 || a->head_dim % 2 || a->n_kv_heads * a->head_dim != a->d_kv)
      return fail(XKV_EINVAL, "append: landmark layout does not match d_kv");
    if (a->chunk <= 0 || a->m % a->chunk || a->pos0 % a->chunk)
      return fail(XKV_EINVAL, "append: m and pos0 must be multiples of chunk for landmarks");
  }
  const size_t es = a->dtype == XKV_BF16 ? 2 : 4;
  *ws_need = align256((size_t)a->r * a->G * a->d_kv * es);
  return XKV_OK;
}

}  // namespace

extern "C" int xkv_append_ws_size(const xkv_append_args* args, size_t* bytes) {
  if (!bytes) return fail(XKV_EINVAL, "xkv_append_ws_size: bytes is NULL");
  return check_append(args, bytes);
}

extern "C" int xkv_compress_append(xkv_ctx ctx, const xkv_append_args* a, void* ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(XKV_EINVAL, "append: ctx is NULL");
  size_t need = 0;
  int rc = check_append(a, &need);
  if (rc) return rc;
  if (!ws || ws_bytes < need) return fail(XKV_EWORKSPACE, "append: workspace %zu bytes < %zu", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  XKV_HIP(hipSetDevice(ctx->device));
  const int n = a->G * a->d_kv, bf16 = a->dtype == XKV_BF16;
  xkv::PtrTable lay{}, aout{};
  for (int l = 0; l < a->G; ++l) lay.p[l] = a->layers[l];
  aout.p[0] = a->A_new;
  XKV_K(xkv::launch_transpose_basis(a->Bt, a->r, n, a->r, ws, bf16, st));
  if (bf16)
    XKV_K(xkv::launch_project_bf16(lay, 1, a->G, a->ld_layer, a->m, a->d_kv, (const uint16_t*)ws, 0, a->r, aout, st));
  else
    XKV_K(xkv::launch_project_f32(lay, 1, a->G, a->ld_layer, a->m, a->d_kv, (const float*)ws, 0, a->r, aout, st));
  if (a->landmarks_new) {
    xkv::PtrTable lmo{};
    const long per_layer = (long)a->n_kv_heads * (a->m / a->chunk) * a->head_dim * (bf16 ? 2 : 4);
    for (int l = 0; l < a->G; ++l) lmo.p[l] = (char*)a->landmarks_new + l * per_layer;
    XKV_K(xkv::launch_landmarks(lay, 1, a->G, a->ld_layer, a->m, a->n_kv_heads, a->head_dim, a->chunk, a->rope_theta,
                                lmo, bf16, st, a->pos0));
  }
  return XKV_OK;
}

// ---------------------------------------------------------------------------
// Dense decode baseline
// ---------------------------------------------------------------------------
namespace {

int plan_dense(const xkv_dense_args* a, xkv::DenseParams* P, size_t* ws_need) {
  if (!a) return fail(XKV_EINVAL, "dense: args is NULL");
  if (a->batch <= 0 || a->n_kv_heads <= 0 || a->n_q_heads <= 0 || a->n_q_heads % a->n_kv_heads)
    return fail(XKV_EINVAL, "dense: batch/heads invalid (n_q_heads must be a multiple of n_kv_heads)");
  const int grp = a->n_q_heads / a->n_kv_heads;
  if (grp > 8) return fail(XKV_EUNSUPPORTED, "dense: at most 8 query heads per KV head");
  if (a->head_dim != 128) return fail(XKV_EUNSUPPORTED, "dense: head_dim must be 128");
  if (a->dtype != XKV_BF16) return fail(XKV_EUNSUPPORTED, "dense: bf16 only");
  if (a->n_ctx <= 0) return fail(XKV_EINVAL, "dense: n_ctx must be positive");
  // Rows per block: a multiple of 128, the smallest that keeps the grid within about two
  // resident blocks per compute unit (512), at most 16 tiles of 32 rows per wave.
  const long units = (long)a->batch * a->n_kv_heads;
  long rpb = 128;
  while (rpb < 2048 && units * ((a->n_ctx + rpb - 1) / rpb) > 512) rpb += 128;
  const long n_splits = (a->n_ctx + rpb - 1) / rpb;
  if (n_splits > xkv::DMAXP) return fail(XKV_EUNSUPPORTED, "dense: n_ctx above %d", xkv::DMAXP * 2048);
  if (!a->q || !a->K || !a->V || !a->out) return fail(XKV_EINVAL, "dense: a required pointer is NULL");
  const long d_kv = (long)a->n_kv_heads * a->head_dim;
  if (a->ld_kv < d_kv) return fail(XKV_EINVAL, "dense: ld_kv too small");
  if (a->n_ctx * a->ld_kv >= (1L << 31)) return fail(XKV_EUNSUPPORTED, "dense: n_ctx * ld_kv must stay below 2^31");
  if (!aligned16(a->q) || !aligned16(a->K) || !aligned16(a->V) || a->ld_kv % 8 || a->bstride_kv % 8)
    return fail(XKV_EINVAL, "dense: q, K and V need 16-byte alignment and strides that are multiples of 8");
  xkv::DenseParams& p = *P;
  std::memset(&p, 0, sizeof(p));
  p.batch = a->batch; p.Hq = a->n_q_heads; p.Hkv = a->n_kv_heads; p.grp = grp;
  p.n_ctx = a->n_ctx; p.q_pos = a->q_pos; p.n_splits = (int)n_splits; p.rows_per_block = (int)rpb;
  p.scale = a->scale;
  for (int i = 0; i < a->head_dim / 2; ++i)
    p.turns[i] = std::pow(a->rope_theta, -2.0 * i / a->head_dim) / (2.0 * M_PI);
  p.q = a->q; p.K = a->K; p.V = a->V; p.ld_kv = a->ld_kv; p.bs_kv = a->bstride_kv; p.out = a->out;
  *ws_need = align256((size_t)a->batch * a->n_kv_heads * n_splits * grp * (2 + a->head_dim) * sizeof(float));
  return XKV_OK;
}

}  // namespace

extern "C" int xkv_dense_ws_size(const xkv_dense_args* args, size_t* bytes) {
  if (!bytes) return fail(XKV_EINVAL, "xkv_dense_ws_size: bytes is NULL");
  xkv::DenseParams P;
  return plan_dense(args, &P, bytes);
}

extern "C" int xkv_dense_decode(xkv_ctx ctx, const xkv_dense_args* args, void* ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(XKV_EINVAL, "dense: ctx is NULL");
  xkv::DenseParams P;
  size_t need = 0;
  int rc = plan_dense(args, &P, &need);
  if (rc) return rc;
  if (!ws || ws_bytes < need) return fail(XKV_EWORKSPACE, "dense: workspace %zu bytes < %zu", ws_bytes, need);
  P.part = (float*)ws;
  XKV_K(xkv::launch_dense_decode(P, (hipStream_t)stream));
  return XKV_OK;
}

extern "C" int xkv_rope_rows(const void* x, long ld_x, void* y, long ld_y, int rows, long pos0, int n_heads,
                             int head_dim, double rope_theta, int dtype, void* stream) {
  if (!x || !y || rows < 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 2 || pos0 < 0)
    return fail(XKV_EINVAL, "xkv_rope_rows: bad arguments");
  if (dtype != XKV_F32 && dtype != XKV_BF16) return fail(XKV_EINVAL, "xkv_rope_rows: unknown dtype");
  if (ld_x < (long)n_heads * head_dim || ld_y < (long)n_heads * head_dim)
    return fail(XKV_EINVAL, "xkv_rope_rows: leading dimension too small");
  XKV_K(xkv::launch_rope_rows(x, ld_x, y, ld_y, rows, pos0, n_heads, head_dim, rope_theta, dtype == XKV_BF16,
                              (hipStream_t)stream));
  return XKV_OK;
}
