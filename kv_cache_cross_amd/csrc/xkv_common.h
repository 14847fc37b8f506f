// Device-side helpers shared by the libxkv HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));

#define XKV_DEV __device__ __forceinline__

XKV_DEV float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
XKV_DEV uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Scalar load / store of the storage types used at the ABI (float or bf16 bits).
XKV_DEV float ld_elem(const float* p) { return *p; }
XKV_DEV float ld_elem(const uint16_t* p) { return bf16_bits_to_f32(*p); }
XKV_DEV void st_elem(float* p, float v) { *p = v; }
XKV_DEV void st_elem(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }

XKV_DEV bf16x8_t as_bf16x8(uint4 v) {
  union { uint4 u; bf16x8_t b; } c;
  c.u = v;
  return c.b;
}

// RoPE angle of position t for pair index i: t * theta^(-2i/d), formed in
// float64 and reduced to [-pi, pi] before the float32 sine/cosine.
XKV_DEV double rope_freq(double theta, int i, int d) { return pow(theta, -2.0 * (double)i / (double)d); }
XKV_DEV void rope_cs(long t, double freq, float* c, float* s) {
  const double a = (double)t * freq;
  const double k = rint(a * 0.15915494309189535);          // 1 / (2 pi)
  const float ar = (float)fma(-k, 6.283185307179586, a);   // 2 pi
  sincosf(ar, s, c);
}

// Decode-path variant: `turns` = theta^(-2i/d) / (2 pi) comes from a host table; the
// angle t * turns is reduced to [-1/2, 1/2] turn in float64 and fed to the hardware
// sine/cosine, which take their argument in turns (absolute error ~1e-6).
XKV_DEV void rope_cs_turns(long t, double turns, float* c, float* s) {
  const double a = (double)t * turns;
  const float x = (float)(a - rint(a));
  *s = __builtin_amdgcn_sinf(x);
  *c = __builtin_amdgcn_cosf(x);
}
