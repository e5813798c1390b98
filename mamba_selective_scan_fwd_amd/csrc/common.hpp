// common.hpp -- element types and f32 math shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mamba {

// I/O element types. bf16 is the compiler's native __bf16: loads widen with a shift,
// stores go through gfx950's v_cvt_pk_bf16_f32 (round to nearest even).
using bf16 = __bf16;

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// exp(x) as 2^(x*log2 e) on the hardware exp2 (v_exp_f32).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// silu(z) = z * sigmoid(z) = z / (1 + exp(-z)). For z << 0, exp(-z) overflows to +inf and
// the reciprocal gives 0, so silu -> -0 as it should.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + fast_exp(-z));
}

// log1p(e) for e in [0, 1], accurate to a few ulp: w = 1 + e is rounded, and its rounding
// error c = (w - 1) - e is exact (w - 1 is exact, and it is within a factor of two of e, or
// zero). log(1 + e) = log(w - c) = log(w) - c / w + O(c^2), and since |c| <= 2^-24 the
// first-order term -c stands for -c / w to well under an ulp of the result. For e below
// 2^-25, w = 1 and the result is exactly e.
__device__ __forceinline__ float log1p_small(float e) {
  const float w = 1.0f + e;
  const float c = (w - 1.0f) - e;
  return __builtin_amdgcn_logf(w) * kLn2 - c;
}

// softplus(v) = log(1 + exp(v)) = max(v, 0) + log1p(exp(-|v|)), with no overflow.
// At the dt-bias values of Mamba layers (v around -7..-2) a plain log(1 + exp(v)) in f32
// loses most of its digits; the compensated log1p keeps the relative error near 1e-7. (The
// log1p is written out here so that max(v, 0) - c and the log share one fma.)
__device__ __forceinline__ float softplus(float v) {
  const float e = fast_exp(-fabsf(v));
  const float w = 1.0f + e;
  const float c = (w - 1.0f) - e;  // the rounding error of w, exactly
  return fmaf(__builtin_amdgcn_logf(w), kLn2, (v > 0.0f ? v : 0.0f) - c);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 16-byte load and store of data streamed through once (a state read and rewritten by one
// step): marked non-temporal, so they do not push reused data (weights, shared rows) out of
// the caches. p must be 16-byte aligned.
__device__ __forceinline__ float4 load_stream4(const float* p) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_stream4(float* p, float4 v) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(f4{v.x, v.y, v.z, v.w}, reinterpret_cast<f4*>(p));
}

}  // namespace mamba
