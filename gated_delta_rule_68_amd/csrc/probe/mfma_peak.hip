// Achievable dense bf16 matrix-core rate on this GPU, for the roofline's
// denominator beside the published peak: every wave issues a long run of
// independent v_mfma_f32_16x16x32_bf16 (eight accumulators, so that no
// product waits on the one before), with no memory traffic inside the loop.
// Built into its own library (libgdr_probe.so); not part of the C ABI of
// include/gdr.h.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int ACC = 8;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_peak_kernel(float *out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  f32x4 acc[ACC];
  for (int j = 0; j < ACC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < ACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < ACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 1234.5f) out[blockIdx.x] = s;  // keeps the products live; never true for these inputs
}

}  // namespace

// Launch `blocks` workgroups of four waves, each wave running iters x 8
// matrix products of 16 x 16 x 32 (16384 flop each), on `stream`.  Returns a
// hipError_t value.
extern "C" __attribute__((visibility("default"))) int gdr_probe_mfma_bf16(int blocks, int iters,
                                                                          float *out,
                                                                          hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}

// flop of one launch with these arguments.
extern "C" __attribute__((visibility("default"))) double gdr_probe_mfma_bf16_flop(int blocks,
                                                                                  int iters) {
  return (double)blocks * 4.0 * (double)iters * ACC * 16384.0;
}
