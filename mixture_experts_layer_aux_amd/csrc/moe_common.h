// Shared device/host helpers of libmoe (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bfloat16
// Storage is raw uint16 bit patterns; arithmetic is fp32.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even, in one v_cvt_pk_bf16_f32 per pair of values.
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f));
}

// Element access for the two activation storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ------------------------------------------------------------------ streaming stores
// Non-temporal global stores for the GEMM outputs (each written once, and far larger than
// the L2s, so no later tile of the same kernel reads them back): they do not displace the
// operand lines that other tiles of the kernel still reuse.
typedef unsigned int nt_u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int nt_u32x4_t __attribute__((ext_vector_type(4)));
typedef float nt_f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(uint2* p, uint2 v) {
  __builtin_nontemporal_store(nt_u32x2_t{v.x, v.y}, reinterpret_cast<nt_u32x2_t*>(p));
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
  __builtin_nontemporal_store(nt_u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4_t*>(p));
}
__device__ __forceinline__ void store_nt(float4* p, float4 v) {
  __builtin_nontemporal_store(nt_f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f32x4_t*>(p));
}

// ------------------------------------------------------------------ wave reductions
// Fixed butterfly order: deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float sigmoid_f(float g) { return 1.0f / (1.0f + __expf(-g)); }

// The experts' gated activation (The Ultimate MoE Training Handbook, §3.4 Activation):
// kind 0 SwiGLU, silu(g) u; kind 1 the hard clamp, g clamped from above at c and u to
// [-c, c] before SwiGLU; kind 2 SiTU-GLU, c tanh(g/c) sigma(g) times u, or times
// cl tanh(u/cl) when cl > 0.
struct Glu {
  int kind;
  float c, cl;
};
__device__ __forceinline__ float glu_f(const Glu& p, float g, float u) {
  if (p.kind == 1) return silu_f(fminf(g, p.c)) * fminf(fmaxf(u, -p.c), p.c);
  if (p.kind == 2) {
    const float ul = p.cl > 0.0f ? p.cl * tanhf(u / p.cl) : u;
    return p.c * tanhf(g / p.c) * sigmoid_f(g) * ul;
  }
  return silu_f(g) * u;
}
// dgate, dup from dAct (chain rule; a clamp passes the gradient inside its closed interval).
__device__ __forceinline__ void glu_grad_f(const Glu& p, float g, float u, float da, float& dg, float& du) {
  if (p.kind == 2) {
    const float th = tanhf(g / p.c), s = sigmoid_f(g);
    const float a = p.c * th * s;
    const float dadg = (1.0f - th * th) * s + p.c * th * s * (1.0f - s);
    float ul = u, dul = 1.0f;
    if (p.cl > 0.0f) {
      const float tl = tanhf(u / p.cl);
      ul = p.cl * tl;
      dul = 1.0f - tl * tl;
    }
    dg = da * ul * dadg;
    du = da * a * dul;
    return;
  }
  float gc = g, uc = u;
  if (p.kind == 1) {
    gc = fminf(g, p.c);
    uc = fminf(fmaxf(u, -p.c), p.c);
  }
  const float sg = sigmoid_f(gc);
  dg = da * uc * sg * (1.0f + gc * (1.0f - sg));
  du = da * gc * sg;
  if (p.kind == 1) {
    if (!(g <= p.c)) dg = 0.0f;
    if (!(fabsf(u) <= p.c)) du = 0.0f;
  }
}
inline Glu glu_of(const moe_config_t& c) { return Glu{c.glu_kind, c.glu_c, c.glu_c_linear}; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ host status
void set_error(const char* fmt, ...);
moe_status_t fail(moe_status_t s, const char* fmt, ...);
moe_status_t check_launch(const char* what);

}  // namespace moe
