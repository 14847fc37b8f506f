// Kernel-argument block of the dense decode baseline.
#pragma once
#include <hip/hip_runtime.h>

namespace xkv {

constexpr int DMAXP = 512;    // splits that the dense merge supports

struct DenseParams {
  int batch, Hq, Hkv, grp;
  long n_ctx;         // cached positions 0 .. n_ctx - 1
  long q_pos;         // the query's position
  int n_splits;       // ceil(n_ctx / rows_per_block)
  int rows_per_block; // a multiple of 128 (four waves of 32-row tiles)
  float scale;
  double turns[64];   // theta^(-2i/d) / (2 pi) for i < d/2, formed on the host in float64
  const void* q;      // batch x Hq x 128 pre-RoPE
  const void* K;      // per sequence n_ctx x d_kv post-RoPE keys (row stride ld_kv)
  const void* V;
  long ld_kv, bs_kv;
  float* out;         // batch x Hq x 128
  float* part;        // batch x Hkv x n_splits x grp x (2 + 128)
};

hipError_t launch_dense_decode(const DenseParams& P, hipStream_t st);
hipError_t launch_rope_rows(const void* x, long ldx, void* y, long ldy, int rows, long pos0, int n_heads, int d,
                            double theta, int bf16, hipStream_t st);

}  // namespace xkv
