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
// in ascending j.  Grid: x over 4-column groups, y over tokens.  The k rows
// of a token are loaded before any is summed (KK = k known at compile time,
// or groups of four), so each thread keeps several loads in flight: with one
// load per trip a thread waits a full memory latency per row.
template <class OutT, int KK>
__global__ __launch_bounds__(kEwThreads) void combine_kernel(const float* __restrict__ pairs,
                                                             const float* __restrict__ gates, int64_t T, int k,
                                                             int64_t d4, OutT* __restrict__ out) {
  const int64_t c4 = int64_t(blockIdx.x) * kEwThreads + threadIdx.x;
  if (c4 >= d4) return;
  const float4* pv = reinterpret_cast<const float4*>(pairs);
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](float w, const float4& v) SMOE_INL {
      s[0] += w * v.x; s[1] += w * v.y; s[2] += w * v.z; s[3] += w * v.w;
    };
    if constexpr (KK > 0) {
      float4 v[KK];
      float w[KK];
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        v[j] = pv[(t * KK + j) * d4 + c4];
        w[j] = gates ? gates[t * KK + j] : 1.f;
      }
#pragma unroll
      for (int j = 0; j < KK; ++j) add(w[j], v[j]);
    } else {
      int j = 0;
      for (; j + 4 <= k; j += 4) {
        float4 v[4];
        float w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = pv[(t * k + j + q) * d4 + c4];
          w[q] = gates ? gates[t * k + j + q] : 1.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) add(w[q], v[q]);
      }
      for (; j < k; ++j) add(gates ? gates[t * k + j] : 1.f, pv[(t * k + j) * d4 + c4]);
    }
    st4<OutT>(out + t * (d4 * 4) + c4 * 4, s);
  }
}

template <class OutT>
static void go_combine(const float* pairs, const float* gates, int64_t T, int k, int64_t d4, OutT* out,
                       hipStream_t st) {
  const dim3 grid(unsigned((d4 + kEwThreads - 1) / kEwThreads), unsigned(std::min<int64_t>(T, 65535)));
  switch (k) {
    case 1: hipLaunchKernelGGL((combine_kernel<OutT, 1>), grid, dim3(kEwThreads), 0, st, pairs, gates, T, k, d4, out); break;
    case 2: hipLaunchKernelGGL((combine_kernel<OutT, 2>), grid, dim3(kEwThreads), 0, st, pairs, gates, T, k, d4, out); break;
    case 4: hipLaunchKernelGGL((combine_kernel<OutT, 4>), grid, dim3(kEwThreads), 0, st, pairs, gates, T, k, d4, out); break;
    case 8: hipLaunchKernelGGL((combine_kernel<OutT, 8>), grid, dim3(kEwThreads), 0, st, pairs, gates, T, k, d4, out); break;
    default: hipLaunchKernelGGL((combine_kernel<OutT, 0>), grid, dim3(kEwThreads), 0, st, pairs, gates, T, k, d4, out);
  }
}

hipError_t launch_combine(const float* pairs, const float* gates, int64_t T, int k, int64_t d, void* out,
                          int out_bf16, hipStream_t st) {
  const int64_t d4 = d / 4;
  if (T == 0 || d4 == 0) return hipSuccess;
  if (out_bf16) go_combine(pairs, gates, T, k, d4, static_cast<uint16_t*>(out), st);
  else go_combine(pairs, gates, T, k, d4, static_cast<float*>(out), st);
  return hipGetLastError();
}

// dg[sidx[r]] = sum over slots of part[slot][r].  A block takes 64 grouped
// rows; its four waves sum disjoint quarters of the slots (one row per lane,
// four loads in flight), and the quarter sums are added in wave order, so
// the result does not depend on timing.
__global__ __launch_bounds__(kEwThreads) void reduce_dg_kernel(const float* __restrict__ part, int slots, int M,
                                                               const int* __restrict__ offsets, int E,
                                                               const int* __restrict__ sidx, float* __restrict__ dg) {
  __shared__ float qs[kEwThreads / kWave][kWave];
  const int rows = offsets[E];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  constexpr int NW = kEwThreads / kWave;
  const int q0 = w * slots / NW, q1 = (w + 1) * slots / NW;
  for (int base = blockIdx.x * kWave; base < rows; base += gridDim.x * kWave) {
    const int r = base + lane;
    float s = 0.f;
    if (r < rows) {
      int q = q0;
      for (; q + 4 <= q1; q += 4) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = part[int64_t(q + u) * M + r];
#pragma unroll
        for (int u = 0; u < 4; ++u) s += v[u];
      }
      for (; q < q1; ++q) s += part[int64_t(q) * M + r];
    }
    qs[w][lane] = s;
    __syncthreads();
    if (w == 0 && r < rows) {
      float t = qs[0][lane];
#pragma unroll
      for (int u = 1; u < NW; ++u) t += qs[u][lane];
      dg[sidx[r]] = t;
    }
    __syncthreads();
  }
}

hipError_t launch_reduce_dg(const float* part, int slots, int M, const int* offsets, int E, const int* sidx,
                            float* dg, hipStream_t st) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_dg_kernel, dim3(grid_for(M, kWave)), dim3(kEwThreads), 0, st, part, slots, M, offsets,
                     E, sidx, dg);
  return hipGetLastError();
}

// grid: (element blocks, E).  Experts whose rows formed one chunk were
// written in place by the GEMM and are skipped, unless every chunk wrote a
// partial (all_partial: a bf16 or accumulated result).
template <class OutT>
__global__ __launch_bounds__(kEwThreads) void reduce_dw_kernel(const float* __restrict__ partial,
                                                               const int* __restrict__ offsets, int KS,
                                                               int64_t elems4, OutT* __restrict__ dw,
                                                               int all_partial, int accumulate) {
  __shared__ int first_s, n_s;
  const int e = blockIdx.y;
  if (threadIdx.x < kWave) {
    // chunks of the experts before e: one wave sums them 64 experts at a
    // time (a serial walk by one thread made every block wait E loads)
    const int lane = threadIdx.x;
    int before = 0;
    for (int i0 = 0; i0 < e; i0 += kWave) {
      const int i = i0 + lane;
      int items = 0;
      if (i < e) items = (offsets[i + 1] - offsets[i] + KS - 1) / KS;
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) items += __shfl_xor(items, o, kWave);
      before += items;
    }
    if (lane == 0) {
      first_s = before;
      n_s = (offsets[e + 1] - offsets[e] + KS - 1) / KS;
    }
  }
  __syncthreads();
  const int first = first_s, n = n_s;
  if (n == 1 && !all_partial) return;
  OutT* out = dw + int64_t(e) * elems4 * 4;
  const float4* pv = reinterpret_cast<const float4*>(partial) + int64_t(first) * elems4;
  for (int64_t i = blockIdx.x * int64_t(kEwThreads) + threadIdx.x; i < elems4; i += int64_t(gridDim.x) * kEwThreads) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    // chunks in ascending order; four loads in flight before they are summed
    int c = 0;
    for (; c + 4 <= n; c += 4) {
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = pv[int64_t(c + q) * elems4 + i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s[0] += v[q].x; s[1] += v[q].y; s[2] += v[q].z; s[3] += v[q].w;
      }
    }
    for (; c < n; ++c) {
      const float4 v = pv[int64_t(c) * elems4 + i];
      s[0] += v.x; s[1] += v.y; s[2] += v.z; s[3] += v.w;
    }
    if (accumulate) {
      float o[4];
      ld4<OutT>(out + i * 4, o);
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] += o[q];
    }
    st4<OutT>(out + i * 4, s);
  }
}

hipError_t launch_reduce_dw(const float* partial, const int* offsets, int E, int KS, int64_t elems, void* dw,
                            int all_partial, int accumulate, int out_bf16, hipStream_t st) {
  const int64_t e4 = elems / 4;
  if (e4 == 0 || E == 0) return hipSuccess;
  const unsigned gx = std::min<unsigned>(grid_for(e4, kEwThreads), 4096u);
  if (out_bf16)
    hipLaunchKernelGGL(reduce_dw_kernel<uint16_t>, dim3(gx, E), dim3(kEwThreads), 0, st, partial, offsets, KS, e4,
                       static_cast<uint16_t*>(dw), all_partial, accumulate);
  else
    hipLaunchKernelGGL(reduce_dw_kernel<float>, dim3(gx, E), dim3(kEwThreads), 0, st, partial, offsets, KS, e4,
                       static_cast<float*>(dw), all_partial, accumulate);
  return hipGetLastError();
}

__global__ __launch_bounds__(kEwThreads) void grouped_gates_kernel(const float* __restrict__ gates,
                                                                   const int* __restrict__ sidx,
                                                                   const int* __restrict__ offsets, int E, int M,
                                                                   float* __restrict__ gg) {
  const int rows = offsets[E];
  for (int r = blockIdx.x * kEwThreads + threadIdx.x; r < M; r += gridDim.x * kEwThreads)
    gg[r] = r < rows ? gates[sidx[r]] : 0.f;
}

hipError_t launch_grouped_gates(const float* gates, const int* sidx, const int* offsets, int E, int M, float* gg,
                                hipStream_t st) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gates_kernel, dim3(grid_for(M, kEwThreads)), dim3(kEwThreads), 0, st, gates, sidx,
                     offsets, E, M, gg);
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
