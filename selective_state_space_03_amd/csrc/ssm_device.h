// Device helpers shared by the gfx950 kernels: element loads/stores for the
// two storage types and the fp32 pointwise functions of the layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct bf16s {  // bf16 storage (bit pattern); arithmetic happens in fp32
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16s v) { return __uint_as_float(static_cast<uint32_t>(v.bits) << 16); }

template <typename T>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  return to_f32(static_cast<const T*>(p)[i]);
}

template <typename T>
__device__ __forceinline__ void st(void* p, size_t i, float v);

template <>
__device__ __forceinline__ void st<float>(void* p, size_t i, float v) {
  static_cast<float*>(p)[i] = v;
}

template <>
__device__ __forceinline__ void st<bf16s>(void* p, size_t i, float v) {
  // v_cvt_pk_bf16_f32: round to nearest even
  __bf16 b = static_cast<__bf16>(v);
  static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, b);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// SiLU(x) = x / (1 + e^-x).  For very negative x the exponential overflows to
// +inf and the reciprocal to 0, giving -0; for large x it tends to x.
__device__ __forceinline__ float silu(float x) {
  return x * rcp_fast(1.0f + exp2_fast(-x * kLog2e));
}

// softplus(x) = max(x, 0) + log1p(e^-|x|).  log1p(w) is evaluated as
// log(u) * w / (u - 1) with u = 1 + w, which keeps full relative accuracy for
// small w (the rounding of u cancels between numerator and denominator).
__device__ __forceinline__ float softplus(float x) {
  const float w = exp2_fast(-fabsf(x) * kLog2e);
  const float u = 1.0f + w;
  const float l1p = (u == 1.0f) ? w : log2_fast(u) * kLn2 * (w * rcp_fast(u - 1.0f));
  return fmaxf(x, 0.0f) + l1p;
}

// dt = clip(softplus(pre), lo, hi) with exact shortcuts: pre >= sp_hi implies
// softplus(pre) >= hi and pre <= sp_lo implies softplus(pre) <= lo (softplus is
// increasing; the host rounds the thresholds outward), so the transcendental
// work only runs for lanes inside the unsaturated band.
__device__ __forceinline__ float dt_softplus_clip(float pre, float lo, float hi, float sp_lo, float sp_hi) {
  float r;
  if (pre >= sp_hi) {
    r = hi;
  } else if (pre <= sp_lo) {
    r = lo;
  } else {
    r = fminf(fmaxf(softplus(pre), lo), hi);
  }
  return r;
}

__device__ __forceinline__ float dt_clip(float pre, float lo, float hi) { return fminf(fmaxf(pre, lo), hi); }

// phi(z) = (e^z - 1) / z, given e^z (ez), for the zero-order-hold input
// coefficient (e^{dt A} - 1) / A = dt phi(dt A).  For |z| <= 1/2 the quotient
// would lose digits to cancellation, so there phi is its Taylor series
// 1 + z/2 + z^2/6 + ... through z^7/8! (truncation below 2e-7 relative); beyond
// it the quotient itself is accurate to a few ulp.
__device__ __forceinline__ float zoh_phi(float z, float ez) {
  float p = 1.0f / 40320.0f;
  p = fmaf(p, z, 1.0f / 5040.0f);
  p = fmaf(p, z, 1.0f / 720.0f);
  p = fmaf(p, z, 1.0f / 120.0f);
  p = fmaf(p, z, 1.0f / 24.0f);
  p = fmaf(p, z, 1.0f / 6.0f);
  p = fmaf(p, z, 0.5f);
  p = fmaf(p, z, 1.0f);
  return fabsf(z) <= 0.5f ? p : (ez - 1.0f) * rcp_fast(z);
}

// Non-temporal 16-byte load and store, for data touched once per launch (a
// recurrent state streamed through a decode step).
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float4* p) {
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(float4* p, float4 v) {
  const v4f w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<v4f*>(p));
}

// 16 bytes from p where ok holds, zeros elsewhere (lanes without ok issue no
// load).  Returning by value keeps the zero out of memory: a conditional
// between a global location and a local zero would make the compiler take the
// local's address and load through a generic pointer.
__device__ __forceinline__ uint4 load16_if(const void* p, bool ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) v = *static_cast<const uint4*>(p);
  return v;
}

// Make a wave-uniform value provably uniform to the compiler (SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace ssm
