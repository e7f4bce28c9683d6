// Device helpers shared by the kernel files: element conversion and the gate
// nonlinearities.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace gdr {

typedef __bf16 bf16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }  // RNE

// softplus(x) = max(x, 0) + log(1 + exp(-|x|)): no overflow for any x.
__device__ __forceinline__ float softplus_f32(float x) {
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

// Log decay g = -exp(A_log) * softplus(a + dt_bias) (GatedDeltaRule.ixx File
// Reference, "Detailed Description"); neg_exp_A_log = -exp(A_log) is hoisted.
__device__ __forceinline__ float log_decay(float neg_exp_A_log, float a, float dt_bias) {
  return neg_exp_A_log * softplus_f32(a + dt_bias);
}

// Load 4 consecutive elements as floats (16-byte aligned for fp32, 8 for bf16).
__device__ __forceinline__ float4 load4(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
__device__ __forceinline__ float4 load4(const bf16 *p) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
  return make_float4(static_cast<float>(v[0]), static_cast<float>(v[1]),
                     static_cast<float>(v[2]), static_cast<float>(v[3]));
}
__device__ __forceinline__ void store4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
__device__ __forceinline__ void store4(bf16 *p, float4 v) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 w;
  w[0] = static_cast<bf16>(v.x);
  w[1] = static_cast<bf16>(v.y);
  w[2] = static_cast<bf16>(v.z);
  w[3] = static_cast<bf16>(v.w);
  *reinterpret_cast<bf16x4 *>(p) = w;
}

// Sequence bounds [t0, t1) of sequence n: from cu_seqlens, or dense.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int seq_len, int n, int64_t &t0,
                                           int64_t &t1) {
  if (cu) {
    t0 = cu[n];
    t1 = cu[n + 1];
  } else {
    t0 = (int64_t)n * seq_len;
    t1 = t0 + seq_len;
  }
}

}  // namespace gdr
