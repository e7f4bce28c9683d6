// Gates and q/k normalisation as a standalone kernel (the gdr_gates entry point).
//
// GatedDeltaRule.ixx File Reference, "Detailed Description": beta = sigmoid(b),
// g = -exp(A_log) * softplus(a + dt_bias), derived inside the component from
// the raw projections; q and k are L2-normalised and q is scaled by
// 1/sqrt(d_k).  The forward kernels derive the same quantities in their own
// prologues; this kernel exists for callers that want them materialised.
//
// Launch: one 256-thread block per token (grid-stride for very long batches).
// Each wave normalises whole rows of q or k (one row of d_k <= 128 elements per
// wave iteration, a wave-wide sum of squares); the threads then derive the
// H_v gates of the token.  Bandwidth-bound elementwise work.
#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kGatesThreads = 256;

template <typename T>
struct GatesParams {
  const T *q, *k, *a, *b;
  const float *A_log, *dt_bias;
  T *q_hat, *k_hat;
  float *g, *beta;
  int64_t total;
  int H_k, H_v;
  float scale, eps;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int DK, typename T>
__global__ __launch_bounds__(kGatesThreads) void gates_kernel(GatesParams<T> p) {
  constexpr int E = (DK + 63) / 64;  // elements per lane
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const bool want_rows = p.q_hat != nullptr || p.k_hat != nullptr;
  const bool want_gates = p.g != nullptr || p.beta != nullptr;
  for (int64_t t = blockIdx.x; t < p.total; t += gridDim.x) {
    if (want_rows) {
      for (int r = wave; r < 2 * p.H_k; r += kGatesThreads / 64) {
        const bool is_q = r < p.H_k;
        const int hk = is_q ? r : r - p.H_k;
        T *dst = is_q ? p.q_hat : p.k_hat;
        if (dst == nullptr) continue;  // uniform per wave
        const T *src = (is_q ? p.q : p.k) + (t * p.H_k + hk) * DK;
        float x[E];
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = lane + 64 * e;
          x[e] = (i < DK) ? to_f32(src[i]) : 0.0f;
          ss += x[e] * x[e];
        }
        ss = wave_sum(ss);
        const float inv = rsqrtf(ss + p.eps) * (is_q ? p.scale : 1.0f);
        T *out = dst + (t * p.H_k + hk) * DK;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = lane + 64 * e;
          if (i < DK) out[i] = from_f32<T>(x[e] * inv);
        }
      }
    }
    if (want_gates) {
      for (int h = threadIdx.x; h < p.H_v; h += kGatesThreads) {
        const float a = to_f32(p.a[t * p.H_v + h]);
        const float b = to_f32(p.b[t * p.H_v + h]);
        if (p.g) p.g[t * p.H_v + h] = log_decay(-expf(p.A_log[h]), a, p.dt_bias[h]);
        if (p.beta) p.beta[t * p.H_v + h] = sigmoid_f32(b);
      }
    }
  }
}

template <int DK, typename T>
hipError_t launch_typed(const Problem &pr, const GatesArgs &x, hipStream_t s) {
  GatesParams<T> p;
  p.q = static_cast<const T *>(x.q);
  p.k = static_cast<const T *>(x.k);
  p.a = static_cast<const T *>(x.a);
  p.b = static_cast<const T *>(x.b);
  p.A_log = x.A_log;
  p.dt_bias = x.dt_bias;
  p.q_hat = static_cast<T *>(x.q_hat);
  p.k_hat = static_cast<T *>(x.k_hat);
  p.g = x.g;
  p.beta = x.beta;
  p.total = pr.total;
  p.H_k = pr.H_k;
  p.H_v = pr.H_v;
  p.scale = pr.scale;
  p.eps = pr.eps;
  if (pr.total == 0) return hipSuccess;
  const int64_t grid = pr.total < (1 << 20) ? pr.total : (1 << 20);
  hipLaunchKernelGGL((gates_kernel<DK, T>), dim3((unsigned)grid), dim3(kGatesThreads), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dk(const Problem &pr, const GatesArgs &x, hipStream_t s) {
  switch (pr.d_k) {
    case 16: return launch_typed<16, T>(pr, x, s);
    case 32: return launch_typed<32, T>(pr, x, s);
    case 64: return launch_typed<64, T>(pr, x, s);
    case 128: return launch_typed<128, T>(pr, x, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gates(const Problem &pr, const GatesArgs &x, hipStream_t s) {
  return pr.dtype == GDR_F32 ? launch_dk<float>(pr, x, s) : launch_dk<bf16>(pr, x, s);
}

}  // namespace gdr
