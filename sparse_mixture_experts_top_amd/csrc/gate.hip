// The SMoE router on the GPU: the gate product logits = x w^T (w [E][d], a
// linear layer's weight), each token's k largest logits (descending, ties
// to the lower expert id) and the softmax over them (article "This Machine
// Learning Research Presents ScatterMoE", body, para. 1: a token goes to k of
// E experts and its output is their gate-weighted sum), and the backward of
// that softmax: dw = dlogits^T x and the router's part of dx = dlogits w.
// E <= 64 and k <= 8; d is a multiple of 8.  Every pass streams x (or dx)
// once from HBM; w is small and stays in cache.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace smoe {

constexpr int kGateThreads = 256;   // 4 waves
constexpr int kGateWaves = kGateThreads / kWave;
constexpr int kGateMaxK = 8;

// ---- forward -------------------------------------------------------------
// The gate weight is w [E][d] (a linear layer's layout: logits = x w^T), so
// one expert's weights run along d like a token's x.

// fp32 inputs, plain FMA.  A wave takes TT = 64 / EMAX tokens at once, so
// every lane holds 64 partial sums (TT tokens x EMAX experts) and each w
// value it loads serves TT tokens.  Lane l sums the products of columns
// 4l..4l+3, 4l+256, ... in column order.

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

// Top k of the logits of one token held by a group of L adjacent lanes,
// EL logits per lane (lane p of the group holds experts p*EL .. p*EL+EL-1;
// experts >= E are absent): k rounds of a group argmax, larger value first,
// equal values to the lower expert id, the winner leaving the race.  Then
// the softmax over the chosen logits (max subtracted).  Lane p of the group
// writes choices p, p+L, ...
template <int L, int EL>
SMOE_DEV void group_topk_softmax(const float (&z)[EL], int p, int E, int k, bool real, int64_t t,
                                 int* __restrict__ idx_out, float* __restrict__ gates_out) {
  uint32_t gone = 0;
  float zsel[kGateMaxK];
  int esel[kGateMaxK];
#pragma unroll
  for (int j = 0; j < kGateMaxK; ++j) {
    zsel[j] = 0.f;
    esel[j] = 0;
    if (j < k) {
      float bv = -INFINITY;
      int bi = 1 << 30;
#pragma unroll
      for (int i = 0; i < EL; ++i) {
        const int e = p * EL + i;
        if (e < E && !((gone >> i) & 1u) && (z[i] > bv || bi == (1 << 30))) {
          bv = z[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 1; o < L; o <<= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      zsel[j] = bv;
      esel[j] = bi;
      const int own = bi - p * EL;
      if (own >= 0 && own < EL) gone |= 1u << own;
    }
  }
  float w[kGateMaxK], s = 0.f;
#pragma unroll
  for (int j = 0; j < kGateMaxK; ++j) {
    w[j] = j < k ? __expf(zsel[j] - zsel[0]) : 0.f;
    s += w[j];
  }
  if (real) {
#pragma unroll
    for (int j = 0; j < kGateMaxK; ++j) {
      if (j < k && j % L == p) {
        idx_out[t * k + j] = esel[j];
        gates_out[t * k + j] = w[j] / s;
      }
    }
  }
}

template <int EMAX>
__global__ __launch_bounds__(kGateThreads) void gate_fwd_f32_kernel(const float* __restrict__ x,
                                                                    const float* __restrict__ wg, int64_t T, int d,
                                                                    int E, int k, int* __restrict__ idx_out,
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
          ld4<float>(x + (t0 + tt) * int64_t(d) + c0, xv[tt]);
        } else {
          xv[tt][0] = xv[tt][1] = xv[tt][2] = xv[tt][3] = 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (e < E) {
          float gq[4];
          ld4<float>(wg + int64_t(e) * d + c0, gq);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[tt * EMAX + e] += xv[tt][i] * gq[i];
        }
      }
    }
    // lane l: token t0 + l / EMAX, expert l % EMAX
    const float z[1] = {wave_transpose_sum(acc)};
    const int tt = lane / EMAX, e = lane % EMAX;
    const bool real = tt < nt;
    if (logits_out && real && e < E) logits_out[(t0 + tt) * E + e] = z[0];
    group_topk_softmax<EMAX, 1>(z, e, E, k, real, t0 + tt, idx_out, gates_out);
  }
}

// bf16 inputs, on the matrix cores: a block takes 32 tokens and all experts
// (NT tiles of 32), its 8 waves splitting d (wave w takes the 16-wide k
// steps w, w+8, ...; each wave keeps U steps of loads in flight, and two
// blocks share a CU, so 16 waves stream x through each CU).  The
// v_mfma_f32_32x32x16_bf16 fragments come straight from global memory: a
// lane loads 8 consecutive k of one token row (x) and of one expert row
// (w).  The wave partials meet in LDS, summed in wave order; then groups of
// 16 lanes per token pick the top k.
typedef __bf16 gate_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float gate_f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kFwdThreads = 512;
constexpr int kFwdWaves = kFwdThreads / kWave;
constexpr int kGateBT = 32;   // tokens per block
constexpr int kGateU = 8;     // k steps per wave per batch of loads

SMOE_DEV gate_bf16x8_t load_frag(const uint16_t* p, bool ok) {
  uint4 v = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(gate_bf16x8_t, v);
}

template <int NT>
__global__ __launch_bounds__(kFwdThreads) void gate_fwd_mfma_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ wg, int64_t T, int d,
                                                                    int E, int k, int* __restrict__ idx_out,
                                                                    float* __restrict__ gates_out,
                                                                    float* __restrict__ logits_out) {
  constexpr int EP = 32 * NT;
  constexpr int PITCH = EP + 1;
  __shared__ float red[kFwdWaves][kGateBT][PITCH];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  const int nsteps = (d + 15) / 16;
  for (int64_t t0 = int64_t(blockIdx.x) * kGateBT; t0 < T; t0 += int64_t(gridDim.x) * kGateBT) {
    const int64_t tok = t0 + (lane & 31);
    const bool tok_ok = tok < T;
    const uint16_t* xr = x + (tok_ok ? tok : 0) * int64_t(d) + 8 * half;
    const uint16_t* wr[NT];
    bool e_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = nt * 32 + (lane & 31);
      e_ok[nt] = e < E;
      wr[nt] = wg + int64_t(e_ok[nt] ? e : 0) * d + 8 * half;
    }
    gate_f32x16_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nt][i] = 0.f;
    for (int s0 = w; s0 < nsteps; s0 += kFwdWaves * kGateU) {
      gate_bf16x8_t a[kGateU], b[kGateU][NT];
#pragma unroll
      for (int u = 0; u < kGateU; ++u) {
        const int kk = 16 * (s0 + kFwdWaves * u);
        const bool k_ok = kk + 8 * half < d;
        a[u] = load_frag(xr + kk, k_ok && tok_ok);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b[u][nt] = load_frag(wr[nt] + kk, k_ok && e_ok[nt]);
      }
#pragma unroll
      for (int u = 0; u < kGateU; ++u)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[u][nt], a[u], acc[nt], 0, 0, 0);
    }
    // lane holds token (lane & 31), experts 32 nt + 8q + 4 half + i in
    // acc[nt][4q + i]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][lane & 31][32 * nt + 8 * q + 4 * half + i] = acc[nt][4 * q + i];
    __syncthreads();
    // 16 lanes per token: lane p of the group sums experts p*EL .. +EL-1
    constexpr int EL = EP / 16;
    const int tl = threadIdx.x / 16, p = threadIdx.x % 16;
    float z[EL];
#pragma unroll
    for (int i = 0; i < EL; ++i) {
      const int e = p * EL + i;
      float v = red[0][tl][e];
#pragma unroll
      for (int ww = 1; ww < kFwdWaves; ++ww) v += red[ww][tl][e];
      z[i] = v;
    }
    const int64_t t = t0 + tl;
    const bool real = t < T;
    if (logits_out && real) {
#pragma unroll
      for (int i = 0; i < EL; ++i)
        if (p * EL + i < E) logits_out[t * E + p * EL + i] = z[i];
    }
    group_topk_softmax<16, EL>(z, p, E, k, real, t, idx_out, gates_out);
    __syncthreads();
  }
}

// ---- backward ------------------------------------------------------------
// Router dx: dx[t][c] (+)= sum_j dlog[t][j] w[e_j][c], with
//   dlog[t][j] = g_j (dg_j - sum_i g_i dg_i)
// for choice j of token t (the sum over all k choices; 0 where the expert
// id is outside [0, E)).  Block (column tile of 256, token chunks of 128,
// strided by the grid's y extent):
// the tile's slice of every expert row, w[e][c0 .. c0+255], sits in LDS as
// fp32, and so do the chunk's expert ids and dlogits, formed in the
// prologue by one thread per token; lane l of each wave owns columns
// c0+4l..c0+4l+3, the four waves take every fourth token.
//
// The blocks of the first column tile also write what the dw product reads:
// the dense dlogits D [T][ncol] (bf16 inputs: D[t][e] = hi, D[t][ep + e] =
// lo with hi = bf16(v), lo = bf16(v - hi), so that the bf16 matrix-core
// product of x with both halves carries v to about 16 significant bits;
// fp32 inputs: D[t][e] = v; unchosen entries 0), the identity row index
// rows[t] = t (its rows are read in place) and the single-group row offsets
// {0, T}.
constexpr int kDxCols = 4 * kWave;
constexpr int kDxTokChunk = 128;
template <class InT, int EMAX>
__global__ __launch_bounds__(kGateThreads) void gate_dx_kernel(const InT* __restrict__ wg, int64_t T, int d, int E,
                                                               int k, const int* __restrict__ idx,
                                                               const float* __restrict__ gates,
                                                               const float* __restrict__ dgates, InT* __restrict__ dx,
                                                               int accumulate, int ep, int ncol_d,
                                                               InT* __restrict__ D, int* __restrict__ rows,
                                                               int* __restrict__ offsets) {
  __shared__ __attribute__((aligned(16))) float ws_tile[EMAX * kDxCols];
  __shared__ int ch_e[kDxTokChunk * kGateMaxK];
  __shared__ float ch_v[kDxTokChunk * kGateMaxK];
  const int c0 = blockIdx.x * kDxCols;
  const int ncol = min(kDxCols, d - c0);   // a multiple of 8
  constexpr int VW = sizeof(InT) == 2 ? 8 : 4;   // elements per 16-byte load
  for (int i = threadIdx.x; i < E * (kDxCols / VW); i += kGateThreads) {
    const int e = i / (kDxCols / VW), c = (i - e * (kDxCols / VW)) * VW;
    float v[VW];
    if (c < ncol) {
      const InT* src = wg + int64_t(e) * d + c0 + c;
      ld4<InT>(src, v);
      if constexpr (VW == 8) ld4<InT>(src + 4, v + 4);
    } else {
#pragma unroll
      for (int q = 0; q < VW; ++q) v[q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < VW; q += 4)
      *reinterpret_cast<float4*>(ws_tile + e * kDxCols + c + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
  }
  const bool first = blockIdx.x == 0;
  if (first && blockIdx.y == 0 && threadIdx.x == 0) {
    offsets[0] = 0;
    offsets[1] = int(T);
  }
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int cl = 4 * lane;
  const bool mine = cl < ncol;
  // token chunks y, y + gridDim.y, ... (the grid's y extent is capped)
  for (int64_t t0 = int64_t(blockIdx.y) * kDxTokChunk; t0 < T; t0 += int64_t(gridDim.y) * kDxTokChunk) {
    const int nt = int(T - t0 < kDxTokChunk ? T - t0 : kDxTokChunk);
    __syncthreads();   // the previous chunk's choices are no longer read
    for (int i = threadIdx.x; i < nt; i += kGateThreads) {
      const int64_t t = t0 + i;
      float gv[kGateMaxK], dv[kGateMaxK];
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < kGateMaxK; ++j) {
        gv[j] = j < k ? gates[t * k + j] : 0.f;
        dv[j] = j < k ? dgates[t * k + j] : 0.f;
        s += gv[j] * dv[j];
      }
      InT* drow = D + t * ncol_d;
      if (first) {
        rows[t] = int(t);
        for (int c = 0; c < ncol_d; c += 16 / int(sizeof(InT)))
          *reinterpret_cast<uint4*>(drow + c) = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < kGateMaxK; ++j) {
        if (j < k) {
          const int e = idx[t * k + j];
          const bool ok = e >= 0 && e < E;
          const float v = ok ? gv[j] * (dv[j] - s) : 0.f;
          ch_e[i * k + j] = ok ? e : 0;
          ch_v[i * k + j] = v;
          if (first && ok) {
            if constexpr (sizeof(InT) == 2) {
              const uint16_t hi = f2bf(v);
              drow[e] = hi;
              drow[ep + e] = f2bf(v - bf2f(hi));
            } else {
              drow[e] = v;
            }
          }
        }
      }
    }
    __syncthreads();
    for (int tl = w; tl < nt; tl += kGateWaves) {
      float r[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const int e = ch_e[tl * k + j];
        const float dl = ch_v[tl * k + j];
        const float4 gv = *reinterpret_cast<const float4*>(ws_tile + e * kDxCols + cl);
        r[0] += dl * gv.x;
        r[1] += dl * gv.y;
        r[2] += dl * gv.z;
        r[3] += dl * gv.w;
      }
      if (mine) {
        InT* p = dx + (t0 + tl) * int64_t(d) + c0 + cl;
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
}

// dw[e][c] from the product's tmp [d][ncol]: tmp[c][e] (+ tmp[c][ep + e]
// for the bf16 halves)
__global__ __launch_bounds__(kGateThreads) void gate_dw_finish_kernel(const float* __restrict__ tmp, int d, int E,
                                                                      int ep, int ncol, int two,
                                                                      float* __restrict__ dw) {
  const int64_t n = int64_t(E) * d;
  for (int64_t i = int64_t(blockIdx.x) * kGateThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kGateThreads) {
    const int e = int(i / d);
    const int64_t c = i - int64_t(e) * d;
    const float* r = tmp + c * ncol;
    dw[i] = two ? r[e] + r[ep + e] : r[e];
  }
}

static unsigned grid_cap(int64_t blocks, int64_t cap) {
  return unsigned(std::min<int64_t>(std::max<int64_t>(blocks, 1), cap));
}

hipError_t launch_gate_fwd(const void* x, const void* wg, int64_t T, int d, int E, int k, int bf16, int* idx,
                           float* gates, float* logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 block(kGateThreads);
  if (bf16) {
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(wg);
    const dim3 grid(grid_cap((T + kGateBT - 1) / kGateBT, 1 << 20)), fblock(kFwdThreads);
    if (E <= 32)
      hipLaunchKernelGGL((gate_fwd_mfma_kernel<1>), grid, fblock, 0, st, xp, wp, T, d, E, k, idx, gates, logits);
    else
      hipLaunchKernelGGL((gate_fwd_mfma_kernel<2>), grid, fblock, 0, st, xp, wp, T, d, E, k, idx, gates, logits);
  } else {
    const float* xp = static_cast<const float*>(x);
    const float* wp = static_cast<const float*>(wg);
    auto grid = [&](int emax) {
      const int64_t groups = (T + kWave / emax - 1) / (kWave / emax);
      return dim3(grid_cap((groups + kGateWaves - 1) / kGateWaves, 8192));
    };
    if (E <= 8)
      hipLaunchKernelGGL((gate_fwd_f32_kernel<8>), grid(8), block, 0, st, xp, wp, T, d, E, k, idx, gates, logits);
    else if (E <= 16)
      hipLaunchKernelGGL((gate_fwd_f32_kernel<16>), grid(16), block, 0, st, xp, wp, T, d, E, k, idx, gates, logits);
    else if (E <= 32)
      hipLaunchKernelGGL((gate_fwd_f32_kernel<32>), grid(32), block, 0, st, xp, wp, T, d, E, k, idx, gates, logits);
    else
      hipLaunchKernelGGL((gate_fwd_f32_kernel<64>), grid(64), block, 0, st, xp, wp, T, d, E, k, idx, gates, logits);
  }
  return hipGetLastError();
}

// Columns of the dense dlogits D: ep = E rounded up to 8; bf16 keeps the
// two halves side by side.
void gate_dlogit_cols(int E, int bf16, int& ep, int& ncol) {
  ep = (E + 7) / 8 * 8;
  ncol = bf16 ? 2 * ep : ep;
}

template <class InT>
static void go_gate_dx(const void* wg, int64_t T, int d, int E, int k, const int* idx, const float* gates,
                       const float* dgates, void* dx, int accumulate, void* D, int* rows, int* offsets,
                       hipStream_t st) {
  int ep, ncol;
  gate_dlogit_cols(E, sizeof(InT) == 2, ep, ncol);
  const dim3 grid(unsigned((d + kDxCols - 1) / kDxCols),
                  unsigned(std::min<int64_t>((T + kDxTokChunk - 1) / kDxTokChunk, 65535)));
  const InT* wp = static_cast<const InT*>(wg);
  InT* dp = static_cast<InT*>(dx);
  InT* Dp = static_cast<InT*>(D);
#define SMOE_GO_DX(EM)                                                                                            \
  hipLaunchKernelGGL((gate_dx_kernel<InT, EM>), grid, dim3(kGateThreads), 0, st, wp, T, d, E, k, idx, gates, dgates, \
                     dp, accumulate, ep, ncol, Dp, rows, offsets)
  if (E <= 8) SMOE_GO_DX(8);
  else if (E <= 16) SMOE_GO_DX(16);
  else if (E <= 32) SMOE_GO_DX(32);
  else SMOE_GO_DX(64);
#undef SMOE_GO_DX
}

hipError_t launch_gate_dx(const void* wg, int64_t T, int d, int E, int k, int bf16, const int* idx,
                          const float* gates, const float* dgates, void* dx, int accumulate, void* D, int* rows,
                          int* offsets, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (bf16) go_gate_dx<uint16_t>(wg, T, d, E, k, idx, gates, dgates, dx, accumulate, D, rows, offsets, st);
  else go_gate_dx<float>(wg, T, d, E, k, idx, gates, dgates, dx, accumulate, D, rows, offsets, st);
  return hipGetLastError();
}

hipError_t launch_gate_dw_finish(const float* tmp, int d, int E, int bf16, float* dw, hipStream_t st) {
  int ep, ncol;
  gate_dlogit_cols(E, bf16, ep, ncol);
  const int64_t n = int64_t(E) * d;
  hipLaunchKernelGGL(gate_dw_finish_kernel, dim3(grid_cap((n + kGateThreads - 1) / kGateThreads, 4096)),
                     dim3(kGateThreads), 0, st, tmp, d, E, ep, ncol, bf16, dw);
  return hipGetLastError();
}

}  // namespace smoe
