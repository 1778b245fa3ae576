// HBM-bound kernels around the grouped products: the top-k gate-weighted
// combine (SMoE output = gate-weighted sum of the chosen experts' outputs:
// article "This Machine Learning Research Presents ScatterMoE", body,
// para. 1), the k-sum of dX contributions, and the deterministic reductions
// of the gate-gradient and split weight-gradient partials.
#include "common.h"
#include "kernels.h"

namespace smoe {

constexpr int kEwThreads = 256;

static unsigned grid_for(int64_t n, int per_block) {
  int64_t g = (n + per_block - 1) / per_block;
  return unsigned(std::min<int64_t>(std::max<int64_t>(g, 1), 1 << 20));
}

// out[t][c] = sum_j w(t,j) * pairs[t*k+j][c], 4 columns per thread, fp32 sum
// in ascending j.
template <class OutT>
__global__ __launch_bounds__(kEwThreads) void combine_kernel(const float* __restrict__ pairs,
                                                             const float* __restrict__ gates, int64_t T, int k,
                                                             int64_t d4, OutT* __restrict__ out) {
  const int64_t n = T * d4;
  for (int64_t i = blockIdx.x * int64_t(kEwThreads) + threadIdx.x; i < n; i += int64_t(gridDim.x) * kEwThreads) {
    const int64_t t = i / d4, c = (i - t * d4) * 4;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int64_t p = t * k + j;
      const float w = gates ? gates[p] : 1.f;
      const float4 v = *reinterpret_cast<const float4*>(pairs + p * (d4 * 4) + c);
      s[0] += w * v.x; s[1] += w * v.y; s[2] += w * v.z; s[3] += w * v.w;
    }
    st4<OutT>(out + t * (d4 * 4) + c, s);
  }
}

hipError_t launch_combine(const float* pairs, const float* gates, int64_t T, int k, int64_t d, void* out,
                          int out_bf16, hipStream_t st) {
  const int64_t d4 = d / 4;
  const int64_t n = T * d4;
  if (n == 0) return hipSuccess;
  const unsigned g = grid_for(n, kEwThreads);
  if (out_bf16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(g), dim3(kEwThreads), 0, st, pairs, gates, T, k, d4,
                       static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(g), dim3(kEwThreads), 0, st, pairs, gates, T, k, d4,
                       static_cast<float*>(out));
  return hipGetLastError();
}

__global__ __launch_bounds__(kEwThreads) void reduce_dg_kernel(const float* __restrict__ part, int slots, int M,
                                                               const int* __restrict__ offsets, int E,
                                                               const int* __restrict__ sidx, float* __restrict__ dg) {
  const int rows = offsets[E];
  for (int r = blockIdx.x * kEwThreads + threadIdx.x; r < rows; r += gridDim.x * kEwThreads) {
    float s = 0.f;
    for (int q = 0; q < slots; ++q) s += part[int64_t(q) * M + r];
    dg[sidx[r]] = s;
  }
}

hipError_t launch_reduce_dg(const float* part, int slots, int M, const int* offsets, int E, const int* sidx,
                            float* dg, hipStream_t st) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_dg_kernel, dim3(grid_for(M, kEwThreads)), dim3(kEwThreads), 0, st, part, slots, M,
                     offsets, E, sidx, dg);
  return hipGetLastError();
}

// grid: (element blocks, E).  Experts whose rows formed one chunk were
// written in place by the GEMM and are skipped.
__global__ __launch_bounds__(kEwThreads) void reduce_dw_kernel(const float* __restrict__ partial,
                                                               const int* __restrict__ offsets, int KS,
                                                               int64_t elems4, float* __restrict__ dw) {
  __shared__ int first_s, n_s;
  const int e = blockIdx.y;
  if (threadIdx.x == 0) {
    int first, n;
    expert_items(offsets, e, KS, first, n);
    first_s = first;
    n_s = n;
  }
  __syncthreads();
  const int first = first_s, n = n_s;
  if (n == 1) return;
  float4* out = reinterpret_cast<float4*>(dw) + int64_t(e) * elems4;
  for (int64_t i = blockIdx.x * int64_t(kEwThreads) + threadIdx.x; i < elems4; i += int64_t(gridDim.x) * kEwThreads) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < n; ++c) {
      const float4 v = reinterpret_cast<const float4*>(partial)[int64_t(first + c) * elems4 + i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    out[i] = s;
  }
}

hipError_t launch_reduce_dw(const float* partial, const int* offsets, int E, int KS, int64_t elems, float* dw,
                            hipStream_t st) {
  const int64_t e4 = elems / 4;
  if (e4 == 0 || E == 0) return hipSuccess;
  const unsigned gx = std::min<unsigned>(grid_for(e4, kEwThreads), 4096u);
  hipLaunchKernelGGL(reduce_dw_kernel, dim3(gx, E), dim3(kEwThreads), 0, st, partial, offsets, KS, e4, dw);
  return hipGetLastError();
}

// one grouped row per block-iteration, 4 columns per thread
template <class T>
__global__ __launch_bounds__(kEwThreads) void scale_rows_kernel(const T* __restrict__ x, int x_grouped, int fan,
                                                                const float* __restrict__ gates,
                                                                const int* __restrict__ sidx,
                                                                const int* __restrict__ offsets, int E, int64_t d,
                                                                T* __restrict__ out) {
  const int rows = offsets[E];
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const int s = sidx[r];
    const int64_t xr = x_grouped ? r : s / fan;
    const float g = gates[s];
    for (int64_t c = int64_t(threadIdx.x) * 4; c < d; c += int64_t(kEwThreads) * 4) {
      float v[4];
      ld4<T>(x + xr * d + c, v);
      for (int i = 0; i < 4; ++i) v[i] *= g;
      st4<T>(out + int64_t(r) * d + c, v);
    }
  }
}

hipError_t launch_scale_rows(const void* x, int x_grouped, int fan, const float* gates, const int* sidx,
                             const int* offsets, int E, int M, int64_t d, void* out, int bf16, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const unsigned g = unsigned(std::min(M, 1 << 16));
  if (bf16)
    hipLaunchKernelGGL(scale_rows_kernel<uint16_t>, dim3(g), dim3(kEwThreads), 0, st,
                       static_cast<const uint16_t*>(x), x_grouped, fan, gates, sidx, offsets, E, d,
                       static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(scale_rows_kernel<float>, dim3(g), dim3(kEwThreads), 0, st, static_cast<const float*>(x),
                       x_grouped, fan, gates, sidx, offsets, E, d, static_cast<float*>(out));
  return hipGetLastError();
}

__global__ __launch_bounds__(kEwThreads) void zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(kEwThreads) + threadIdx.x; i < n; i += int64_t(gridDim.x) * kEwThreads)
    p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t n = int64_t(bytes / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n, kEwThreads)), dim3(kEwThreads), 0, st,
                     static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace smoe
