// The SMoE router on the GPU: the gate product logits = x G, each token's k
// largest logits (descending, ties to the lower expert id) and the softmax
// over them (article "This Machine Learning Research Presents ScatterMoE",
// body, para. 1: a token goes to k of E experts and its output is their
// gate-weighted sum), and the backward of that softmax: dG = x^T dlogits and
// the router's part of dx = dlogits G^T.  E <= 64 and k <= 8; d is a
// multiple of 8.  Every pass streams x (or dx) once from HBM; G is small and
// stays in cache.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace smoe {

constexpr int kGateThreads = 256;   // 4 waves
constexpr int kGateWaves = kGateThreads / kWave;
constexpr int kGateMaxK = 8;

// ---- forward -------------------------------------------------------------
// A wave takes TT = 64 / EMAX tokens at once, so every lane holds 64 partial
// sums (TT tokens x EMAX experts) and each G value it loads serves TT
// tokens.  Lane l sums the products of columns 4l..4l+3, 4l+256, ... in
// column order.

// G row c into gv (zeros past E); four values per load when E % 4 == 0
// (rows then start on 16-byte boundaries for fp32, 8-byte for bf16)
template <class InT, int EMAX>
SMOE_DEV void load_grow(const InT* __restrict__ gr, int E, bool g4, float (&gv)[EMAX]) {
  if (g4) {
    static_for<EMAX / 4>([&](auto q) {
      constexpr int e0 = decltype(q)::value * 4;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (e0 < E) ld4<InT>(gr + e0, v);
      gv[e0] = v[0];
      gv[e0 + 1] = v[1];
      gv[e0 + 2] = v[2];
      gv[e0 + 3] = v[3];
    });
  } else {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) gv[e] = e < E ? ld<InT>(gr + e) : 0.f;
  }
}

// Wave-wide sum of 64 per-lane values that leaves lane l with the sum of
// element l: six exchange rounds, each halving what a lane carries (lanes
// l and l^h split the current array; the lane whose bit h is set keeps the
// upper half).  63 shuffles in all, against 6 per value for a butterfly.
SMOE_DEV float wave_transpose_sum(float (&v)[64]) {
  const int l = lane_id();
  static_for<6>([&](auto s) {
    constexpr int h = 32 >> decltype(s)::value;
    const bool up = (l & h) != 0;
#pragma unroll
    for (int j = 0; j < h; ++j) {
      const float send = up ? v[j] : v[j + h];
      const float keep = up ? v[j + h] : v[j];
      v[j] = keep + __shfl_xor(send, h, kWave);
    }
  });
  return v[0];
}

template <class InT, int EMAX>
__global__ __launch_bounds__(kGateThreads) void gate_fwd_kernel(const InT* __restrict__ x, const InT* __restrict__ g,
                                                                int64_t T, int d, int E, int k, int g4,
                                                                int* __restrict__ idx_out,
                                                                float* __restrict__ gates_out,
                                                                float* __restrict__ logits_out) {
  constexpr int TT = kWave / EMAX;
  const int lane = lane_id();
  const int64_t wave0 = int64_t(blockIdx.x) * kGateWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t nwaves = int64_t(gridDim.x) * kGateWaves;
  for (int64_t t0 = wave0 * TT; t0 < T; t0 += nwaves * TT) {
    const int nt = int(T - t0 < TT ? T - t0 : TT);
    float acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = 0.f;
    for (int c0 = 4 * lane; c0 < d; c0 += 4 * kWave) {
      float xv[TT][4];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt < nt) {
          ld4<InT>(x + (t0 + tt) * int64_t(d) + c0, xv[tt]);
        } else {
          xv[tt][0] = xv[tt][1] = xv[tt][2] = xv[tt][3] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float gv[EMAX];
        load_grow<InT, EMAX>(g + int64_t(c0 + i) * E, E, g4 != 0, gv);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int e = 0; e < EMAX; ++e) acc[tt * EMAX + e] += xv[tt][i] * gv[e];
      }
    }
    // lane l: token t0 + l / EMAX, expert l % EMAX
    const float z = wave_transpose_sum(acc);
    const int tt = lane / EMAX, e = lane % EMAX;
    const int64_t t = t0 + tt;
    const bool real = tt < nt;
    if (logits_out && real && e < E) logits_out[t * E + e] = z;
    // k rounds of an argmax within each group of EMAX lanes: larger value
    // first, equal values to the lower expert id; the winner leaves the race
    float live = e < E ? z : -INFINITY;
    float zsel = 0.f, zmax = 0.f;
    int esel = 0;
    for (int j = 0; j < k; ++j) {
      float bv = live;
      int bi = e < E ? e : kWave;
#pragma unroll
      for (int o = EMAX / 2; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (j == 0) zmax = bv;
      if (e == j) {
        zsel = bv;
        esel = bi;
      }
      if (e == bi) live = -INFINITY;
    }
    // softmax over the chosen logits (group lanes 0..k-1), max subtracted
    const float w = e < k ? __expf(zsel - zmax) : 0.f;
    float s = w;
#pragma unroll
    for (int o = EMAX / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
    if (real && e < k) {
      idx_out[t * k + e] = esel;
      gates_out[t * k + e] = w / s;
    }
  }
}

// ---- backward ------------------------------------------------------------
// dlog[t][j] = g_j (dg_j - sum_i g_i dg_i) for choice j of token t (the sum
// over all k choices), 0 where the expert id is outside [0, E); one thread
// per token.
__global__ __launch_bounds__(kGateThreads) void gate_dlogit_kernel(int64_t T, int E, int k,
                                                                   const int* __restrict__ idx,
                                                                   const float* __restrict__ gates,
                                                                   const float* __restrict__ dgates,
                                                                   float* __restrict__ dlog) {
  for (int64_t t = int64_t(blockIdx.x) * kGateThreads + threadIdx.x; t < T; t += int64_t(gridDim.x) * kGateThreads) {
    float gv[kGateMaxK], dv[kGateMaxK];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kGateMaxK; ++j) {
      gv[j] = j < k ? gates[t * k + j] : 0.f;
      dv[j] = j < k ? dgates[t * k + j] : 0.f;
      s += gv[j] * dv[j];
    }
#pragma unroll
    for (int j = 0; j < kGateMaxK; ++j) {
      if (j < k) {
        const int e = idx[t * k + j];
        dlog[t * k + j] = (e >= 0 && e < E) ? gv[j] * (dv[j] - s) : 0.f;
      }
    }
  }
}

// Router dx: dx[t][c] (+)= sum_j dlog[t][j] G[c][e_j].  Block (column tile
// of 256, token chunk): the tile's G rows sit transposed in LDS,
// Gt[e][c - c0], so a token's k reads are whole LDS rows; lane l of each
// wave owns columns c0+4l..c0+4l+3, the four waves split the tokens.
constexpr int kDxCols = 4 * kWave;
constexpr int kDxTokChunk = 128;
template <class InT>
__global__ __launch_bounds__(kGateThreads) void gate_dx_kernel(const InT* __restrict__ g, int64_t T, int d, int E,
                                                               int k, const int* __restrict__ idx,
                                                               const float* __restrict__ dlog, InT* __restrict__ dx,
                                                               int accumulate) {
  extern __shared__ float gt[];   // [E][kDxCols]
  const int c0 = blockIdx.x * kDxCols;
  const int ncol = min(kDxCols, d - c0);   // a multiple of 8
  for (int i = threadIdx.x; i < ncol * E; i += kGateThreads) {
    const int c = i / E, e = i - c * E;
    gt[e * kDxCols + c] = ld<InT>(g + int64_t(c0) * E + i);
  }
  __syncthreads();
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t t0 = int64_t(blockIdx.y) * kDxTokChunk;
  const int64_t t1 = t0 + kDxTokChunk < T ? t0 + kDxTokChunk : T;
  const int cl = 4 * lane;
  const bool mine = cl < ncol;
  for (int64_t t = t0 + w; t < t1; t += kGateWaves) {
    float r[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      const float dl = dlog[t * k + j];
      if (e >= 0 && e < E) {
        const float4 gv = *reinterpret_cast<const float4*>(gt + e * kDxCols + cl);
        r[0] += dl * gv.x;
        r[1] += dl * gv.y;
        r[2] += dl * gv.z;
        r[3] += dl * gv.w;
      }
    }
    if (mine) {
      InT* p = dx + t * int64_t(d) + c0 + cl;
      if (accumulate) {
        float v[4];
        ld4<InT>(p, v);
        r[0] = v[0] + r[0];
        r[1] = v[1] + r[1];
        r[2] = v[2] + r[2];
        r[3] = v[3] + r[3];
      }
      st4<InT>(p, r);
    }
  }
}

// dG partials: block (column tile of 256, token chunk q) sums x[t][c] dlog
// into LDS acc[e][c - c0] (a thread per column; each address has one owner,
// so the adds land in token order), then writes its contiguous slice
// part[q][c0 .. c0+255][0 .. E).
constexpr int kDgCols = kGateThreads;
constexpr int kDgPitch = kDgCols + 1;
template <class InT>
__global__ __launch_bounds__(kGateThreads) void gate_dg_partial_kernel(const InT* __restrict__ x, int64_t T, int d,
                                                                       int E, int k, const int* __restrict__ idx,
                                                                       const float* __restrict__ dlog, int64_t chunk,
                                                                       float* __restrict__ part) {
  extern __shared__ float acc[];   // [E][kDgPitch]
  const int c0 = blockIdx.x * kDgCols;
  const int ncol = min(kDgCols, d - c0);
  const int tid = threadIdx.x;
  for (int i = tid; i < E * kDgPitch; i += kGateThreads) acc[i] = 0.f;
  __syncthreads();
  const int64_t t0 = int64_t(blockIdx.y) * chunk;
  const int64_t t1 = t0 + chunk < T ? t0 + chunk : T;
  const bool mine = tid < ncol;
  const InT* xc = x + c0 + (mine ? tid : 0);
  float* my = acc + tid;
  constexpr int U = 8;   // tokens whose x loads are in flight together
  int64_t t = t0;
  for (; t + U <= t1; t += U) {
    float xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) xv[u] = ld<InT>(xc + (t + u) * int64_t(d));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[(t + u) * k + j];
        if (e >= 0 && e < E) my[e * kDgPitch] += xv[u] * dlog[(t + u) * k + j];
      }
    }
  }
  for (; t < t1; ++t) {
    const float xv = ld<InT>(xc + t * int64_t(d));
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) my[e * kDgPitch] += xv * dlog[t * k + j];
    }
  }
  __syncthreads();
  float* out = part + (int64_t(blockIdx.y) * d + c0) * E;
  for (int i = tid; i < ncol * E; i += kGateThreads) {
    const int c = i / E, e = i - c * E;
    out[i] = acc[e * kDgPitch + c];
  }
}

// dG[i] = sum over chunks q of part[q][i], in chunk order
__global__ __launch_bounds__(kGateThreads) void gate_dg_reduce_kernel(const float* __restrict__ part, int chunks,
                                                                      int64_t n, float* __restrict__ dg) {
  for (int64_t i = int64_t(blockIdx.x) * kGateThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kGateThreads) {
    float s = 0.f;
    for (int q = 0; q < chunks; ++q) s += part[int64_t(q) * n + i];
    dg[i] = s;
  }
}

// Token chunking of the dG partials: enough blocks to fill the chip (about
// 512), but at most T / (4 E) chunks, so that the partials (chunks * d * E
// floats) stay well under the size of x.
static void dg_chunking(int64_t T, int d, int E, int& chunks, int64_t& chunk) {
  const int64_t colblocks = (d + kDgCols - 1) / kDgCols;
  int64_t c = (512 + colblocks - 1) / colblocks;
  c = std::max<int64_t>(std::min<int64_t>(c, T / (4 * int64_t(E))), 1);
  chunk = std::max<int64_t>((T + c - 1) / c, 1);
  chunks = int(std::max<int64_t>((T + chunk - 1) / chunk, 1));
}

static size_t dlog_bytes(int64_t T) { return (size_t(T) * kGateMaxK * 4 + 255) & ~size_t(255); }

// scratch: dlog [T][8] floats, then the partials
size_t gate_bwd_ws_bytes(int64_t T, int d, int E) {
  int chunks;
  int64_t chunk;
  dg_chunking(T, d, E, chunks, chunk);
  return dlog_bytes(T) + size_t(chunks) * size_t(d) * size_t(E) * 4;
}

static unsigned grid_cap(int64_t blocks, int64_t cap) {
  return unsigned(std::min<int64_t>(std::max<int64_t>(blocks, 1), cap));
}

template <class InT>
static void go_gate_fwd(const void* x, const void* g, int64_t T, int d, int E, int k, int* idx, float* gates,
                        float* logits, hipStream_t st) {
  const InT* xp = static_cast<const InT*>(x);
  const InT* gp = static_cast<const InT*>(g);
  const int g4 = E % 4 == 0;
  const dim3 block(kGateThreads);
  auto grid = [&](int emax) {
    const int64_t groups = (T + kWave / emax - 1) / (kWave / emax);
    return dim3(grid_cap((groups + kGateWaves - 1) / kGateWaves, 8192));
  };
  if (E <= 8)
    hipLaunchKernelGGL((gate_fwd_kernel<InT, 8>), grid(8), block, 0, st, xp, gp, T, d, E, k, g4, idx, gates, logits);
  else if (E <= 16)
    hipLaunchKernelGGL((gate_fwd_kernel<InT, 16>), grid(16), block, 0, st, xp, gp, T, d, E, k, g4, idx, gates,
                       logits);
  else if (E <= 32)
    hipLaunchKernelGGL((gate_fwd_kernel<InT, 32>), grid(32), block, 0, st, xp, gp, T, d, E, k, g4, idx, gates,
                       logits);
  else
    hipLaunchKernelGGL((gate_fwd_kernel<InT, 64>), grid(64), block, 0, st, xp, gp, T, d, E, k, g4, idx, gates,
                       logits);
}

hipError_t launch_gate_fwd(const void* x, const void* g, int64_t T, int d, int E, int k, int bf16, int* idx,
                           float* gates, float* logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (bf16) go_gate_fwd<uint16_t>(x, g, T, d, E, k, idx, gates, logits, st);
  else go_gate_fwd<float>(x, g, T, d, E, k, idx, gates, logits, st);
  return hipGetLastError();
}

template <class InT>
static void go_gate_bwd(const void* x, const void* g, int64_t T, int d, int E, int k, const int* idx,
                        const float* gates, const float* dgates, float* dg, void* dx, int accumulate, void* ws,
                        hipStream_t st) {
  const InT* xp = static_cast<const InT*>(x);
  const InT* gp = static_cast<const InT*>(g);
  float* dlog = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + dlog_bytes(T));
  hipLaunchKernelGGL(gate_dlogit_kernel, dim3(grid_cap((T + kGateThreads - 1) / kGateThreads, 4096)),
                     dim3(kGateThreads), 0, st, T, E, k, idx, gates, dgates, dlog);
  const dim3 dxgrid(unsigned((d + kDxCols - 1) / kDxCols), unsigned((T + kDxTokChunk - 1) / kDxTokChunk));
  hipLaunchKernelGGL((gate_dx_kernel<InT>), dxgrid, dim3(kGateThreads), size_t(E) * kDxCols * 4, st, gp, T, d, E, k,
                     idx, dlog, static_cast<InT*>(dx), accumulate);
  int chunks;
  int64_t chunk;
  dg_chunking(T, d, E, chunks, chunk);
  const dim3 pgrid(unsigned((d + kDgCols - 1) / kDgCols), unsigned(chunks));
  hipLaunchKernelGGL((gate_dg_partial_kernel<InT>), pgrid, dim3(kGateThreads), size_t(E) * kDgPitch * 4, st, xp, T,
                     d, E, k, idx, dlog, chunk, part);
  const int64_t n = int64_t(d) * E;
  hipLaunchKernelGGL(gate_dg_reduce_kernel, dim3(grid_cap((n + kGateThreads - 1) / kGateThreads, 4096)),
                     dim3(kGateThreads), 0, st, part, chunks, n, dg);
}

hipError_t launch_gate_bwd(const void* x, const void* g, int64_t T, int d, int E, int k, int bf16, const int* idx,
                           const float* gates, const float* dgates, float* dg, void* dx, int accumulate, void* ws,
                           hipStream_t st) {
  if (T == 0) return launch_zero(dg, size_t(d) * E * 4, st);
  if (bf16)
    go_gate_bwd<uint16_t>(x, g, T, d, E, k, idx, gates, dgates, dg, dx, accumulate, ws, st);
  else
    go_gate_bwd<float>(x, g, T, d, E, k, idx, gates, dgates, dg, dx, accumulate, ws, st);
  return hipGetLastError();
}

}  // namespace smoe
