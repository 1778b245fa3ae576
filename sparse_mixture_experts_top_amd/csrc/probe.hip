// Diagnostic kernel: the matrix cores' reachable bf16 rate on this device.
// Every wave keeps 16 independent 32x32 accumulators in registers and issues
// `iters` rounds of 16 v_mfma_f32_32x32x16_bf16 on constant operands: no
// memory traffic inside the loop, so the rate it reaches (and the clock the
// chip holds while it runs) bounds what any kernel here can sustain.
#include "common.h"
#include "kernels.h"

namespace smoe {

typedef __bf16 bf16x8p_t __attribute__((ext_vector_type(8)));
typedef float f32x16p_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters) {
  f32x16p_t acc[16];
  for (int i = 0; i < 16; ++i)
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  bf16x8p_t a, b;
  for (int v = 0; v < 8; ++v) {
    a[v] = static_cast<__bf16>(float(threadIdx.x) * 1e-3f);
    b[v] = static_cast<__bf16>(float(v) * 1e-3f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i)
    for (int v = 0; v < 16; ++v) s += acc[i][v];
  out[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_mfma_loop(float* out, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

}  // namespace smoe
