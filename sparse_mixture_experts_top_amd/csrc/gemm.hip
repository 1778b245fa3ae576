// Segmented grouped GEMM over scattered rows for gfx950 (CDNA4): the fp32
// kernel, and the host side (tile choice, grid sizing, dispatch) of both.
//
// The bf16 MFMA kernel is the template in gemm_kernel.h; its instances are
// compiled in groups in gemm_store_k.hip, gemm_store_mn.hip,
// gemm_act_fwd.hip, gemm_act_bwd.hip and gemm_dw.hip.
//
// fp32 kernel: the same contract with plain FMA on 64x64 tiles, used for
// fp32 runs (a small, launch-bound regime).
#include "gemm_kernel.h"

namespace smoe {

// ============================================================================
// fp32 kernel: 64x64 tiles, K step 16, 256 threads each owning 4x4 outputs
// (rows ty*4+i, columns tx*4+j).  Element-wise operand access through the
// same contract as the bf16 kernel.
// ============================================================================
constexpr int kFThreads = 256;
constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <int MODE, int EPI, int BNK, bool DUAL>
__global__ __launch_bounds__(kFThreads) void gemm_f32_kernel(GemmArgs p) {
  __shared__ float As[kFBK][kFBM + 4];
  __shared__ float Bs[kFBK][kFBN + 4];
  __shared__ float B3s[DUAL ? kFBK : 1][kFBN + 4];
  TileInfo T;
  if (!tile_of_block<kFBM, kFBN * (DUAL ? 2 : 1), MODE, DUAL>(p, T)) return;
  const Item& it = T.it;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float* a0 = static_cast<const float*>(p.a0);
  const float* a1 = static_cast<const float*>(p.a1);
  const float* b0 = static_cast<const float*>(p.b0);
  const float* b1 = static_cast<const float*>(p.b1);
  const int Kloop = MODE == SEG_M ? p.K : it.row1 - it.row0;

  auto Aval = [&](int m, int k) SMOE_INL -> float {  // m tile-local, k absolute (SEG_M) / chunk-local (SEG_K)
    if constexpr (MODE == SEG_M) {
      const int gr = it.row0 + m;
      if (gr >= it.row1 || k >= p.K) return 0.f;
      const int src = p.a_scat ? p.sidx[gr] / p.a_fan : gr;
      return k < p.K0 ? a0[int64_t(src) * p.lda + k] : a1[int64_t(src) * p.lda + (k - p.K0)];
    } else {
      const int r = it.row0 + k, i = T.m0 + m;
      if (r >= it.row1 || i >= p.Mo) return 0.f;
      const int src = p.a_scat ? p.sidx[r] / p.a_fan : r;
      const float v = a0[int64_t(src) * p.lda + i];
      return p.kscale ? p.kscale[r] * v : v;
    }
  };
  auto Bval = [&](int k, int n, int which) SMOE_INL -> float {  // n tile-local
    if constexpr (MODE == SEG_M) {
      const int col = T.n0 + n;
      if (col >= p.N || k >= p.K) return 0.f;
      const int64_t e = it.e;
      if constexpr (BNK) {
        return k < p.K0 ? b0[e * p.b_es + int64_t(col) * p.ldb + k]
                        : b1[e * p.b_es + int64_t(col) * p.ldb + (k - p.K0)];
      } else {
        return (which ? b1 : b0)[e * p.b_es + int64_t(k) * p.ldb + col];
      }
    } else {
      const int r = it.row0 + k, j = T.n0 + n;
      if (r >= it.row1 || j >= p.N) return 0.f;
      const int src = p.b_scat ? p.sidx[r] / p.b_fan : r;
      return b0[int64_t(src) * p.ldb + j];
    }
  };

  float acc[4][4] = {}, acc3[4][4] = {};
  for (int k0 = 0; k0 < Kloop; k0 += kFBK) {
    for (int l = tid; l < kFBK * kFBM; l += kFThreads) {
      const int m = l / kFBK, kk = l % kFBK;
      As[kk][m] = Aval(m, k0 + kk);
    }
    for (int l = tid; l < kFBK * kFBN; l += kFThreads) {
      const int n = l % kFBN, kk = l / kFBN;
      Bs[kk][n] = Bval(k0 + kk, n, 0);
      if constexpr (DUAL) B3s[kk][n] = Bval(k0 + kk, n, 1);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float av[4], bv[4], b3v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty * 4 + i];
        bv[i] = Bs[kk][tx * 4 + i];
        if constexpr (DUAL) b3v[i] = B3s[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
          if constexpr (DUAL) acc3[i][j] = fmaf(av[i], b3v[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }

  if constexpr (MODE == SEG_K) {
    float* dst = (it.nitems == 1 && !p.dw_all_partial) ? static_cast<float*>(p.c0) + int64_t(it.e) * p.Mo * p.N
                                                       : p.partial + int64_t(T.chunk) * p.Mo * p.N;
    for (int i = 0; i < 4; ++i) {
      const int r = T.m0 + ty * 4 + i;
      const int j = T.n0 + tx * 4;
      if (r < p.Mo && j < p.N) st4<float>(dst + int64_t(r) * p.N + j, acc[i]);
    }
  } else {
    float* c0 = static_cast<float*>(p.c0);
    float* c1 = static_cast<float*>(p.c1);
    float* c2 = static_cast<float*>(p.c2);
    const float* x0 = static_cast<const float*>(p.aux0);
    const float* x1 = static_cast<const float*>(p.aux1);
    for (int i = 0; i < 4; ++i) {
      const int gr = it.row0 + ty * 4 + i;
      const bool rok = gr < it.row1;
      const int sp = rok ? p.sidx[gr] : 0;
      const float g = (p.gate && rok) ? p.gate[sp] : 1.f;
      const int64_t crow = p.c_scat ? sp : gr;
      const int64_t xrow = p.aux_scat ? sp / p.aux_fan : gr;
      const int n = T.n0 + tx * 4;
      float dgacc = 0.f;
      if (rok && n < p.N) {
        float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        if constexpr (EPI == EPI_STORE) {
          if (p.dgpart) {
            float xv[4];
            ld4<float>(x0 + xrow * p.ldaux + n, xv);
            dgacc = xv[0] * v[0] + xv[1] * v[1] + xv[2] * v[2] + xv[3] * v[3];
          }
          if (c0) {
            if (p.gate)
              for (int j = 0; j < 4; ++j) v[j] *= g;
            if (p.c_add_fan > 0) {
              float* dst = c0 + (crow / p.c_add_fan) * p.ldc + n;
              for (int j = 0; j < 4; ++j) unsafeAtomicAdd(dst + j, v[j]);
            } else {
              st4<float>(c0 + crow * p.ldc + n, v);
            }
          }
        } else if constexpr (EPI == EPI_GELU_FWD) {
          float a[4];
          for (int j = 0; j < 4; ++j) a[j] = gelu_f(v[j]);
          st4<float>(c0 + int64_t(gr) * p.ldc + n, v);
          st4<float>(c1 + int64_t(gr) * p.ldc + n, a);
        } else if constexpr (EPI == EPI_SWIGLU_FWD) {
          float a[4];
          for (int j = 0; j < 4; ++j) a[j] = silu_f(v[j]) * acc3[i][j];
          st4<float>(c0 + int64_t(gr) * p.ldc + n, v);
          st4<float>(c1 + int64_t(gr) * p.ldc + n, acc3[i]);
          st4<float>(c2 + int64_t(gr) * p.ldc + n, a);
        } else if constexpr (EPI == EPI_GELU_BWD) {
          float h[4], dh[4], ag[4];
          ld4<float>(x0 + int64_t(gr) * p.ldaux + n, h);
          for (int j = 0; j < 4; ++j) {
            const float a = gelu_f(h[j]);
            dgacc += a * v[j];
            dh[j] = g * v[j] * gelu_grad_f(h[j]);
            ag[j] = g * a;
          }
          st4<float>(c0 + int64_t(gr) * p.ldc + n, dh);
          st4<float>(c2 + int64_t(gr) * p.ldc + n, ag);
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
          float h1[4], h3[4], d1[4], d3[4], ag[4];
          ld4<float>(x0 + int64_t(gr) * p.ldaux + n, h1);
          ld4<float>(x1 + int64_t(gr) * p.ldaux + n, h3);
          for (int j = 0; j < 4; ++j) {
            const float sg = silu_f(h1[j]);
            const float a = sg * h3[j];
            dgacc += a * v[j];
            d1[j] = g * v[j] * h3[j] * silu_grad_f(h1[j]);
            d3[j] = g * v[j] * sg;
            ag[j] = g * a;
          }
          st4<float>(c0 + int64_t(gr) * p.ldc + n, d1);
          st4<float>(c1 + int64_t(gr) * p.ldc + n, d3);
          st4<float>(c2 + int64_t(gr) * p.ldc + n, ag);
        }
      }
      if (p.dgpart) {
        // the 16 lanes sharing this row are consecutive lanes of one wave
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) dgacc += __shfl_xor(dgacc, o, kWave);
        if (tx == 0 && rok) p.dgpart[int64_t(T.nt) * p.M + gr] = dgacc;
      }
    }
  }
}

// ============================================================================
// host side: tile choice, grid sizing, instance dispatch
// ============================================================================
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t pad8(int64_t n) { return (n + 7) & ~int64_t(7); }

bool plan_gemm(GemmArgs& a, GemmPlan& pl, int mode, int epi, int dual, int bf16, int out_f32) {
  pl.mode = mode;
  pl.epi = epi;
  pl.dual = dual;
  pl.bf16 = bf16;
  pl.out_f32 = out_f32;
  pl.nw = 8;
  fastdiv_magic(std::max(a.a_fan, 1), a.a_fan_m, a.a_fan_s);
  fastdiv_magic(std::max(a.b_fan, 1), a.b_fan_m, a.b_fan_s);
  constexpr int kCUs = 256;
  if (!bf16) {
    pl.bm = kFBM;
    pl.bn = kFBN;
    if (mode == SEG_M) {
      a.mt_ub = int(ceil_div(a.M, pl.bm) + a.E);
      pl.n_tiles = int(ceil_div(a.N, pl.bn));
      pl.slots = pl.n_tiles;
      pl.grid = pad8(int64_t(a.mt_ub) * pl.n_tiles);
    } else {
      pl.n_tiles = int(ceil_div(a.Mo, pl.bm) * ceil_div(a.N, pl.bn));
      pl.slots = 0;
    }
  } else {
    if (mode == SEG_M) {
      const int64_t rows_per_expert = std::max<int64_t>(1, a.M / std::max(1, a.E));
      pl.bn = (dual || a.N >= 256) ? 256 : 128;
      pl.bm = (rows_per_expert >= 192) ? 256 : 128;
      // prefer smaller tiles when the big ones leave most CUs idle
      auto tiles = [&](int bm, int bn) SMOE_INL {
        const int ncols = dual ? bn / 2 : bn;
        return (ceil_div(a.M, bm) + a.E / 2) * ceil_div(a.N, ncols);
      };
      if (tiles(pl.bm, pl.bn) < 2 * kCUs && pl.bm == 256) pl.bm = 128;
      if (tiles(pl.bm, pl.bn) < 2 * kCUs && pl.bn == 256 && !dual) pl.bn = 128;
      a.mt_ub = int(ceil_div(a.M, pl.bm) + a.E);
      const int ncols = dual ? pl.bn / 2 : pl.bn;
      pl.n_tiles = int(ceil_div(a.N, ncols));
      // 256 x 256 tiles of the dual (W1 | W3) forward and of the W^T product
      // over long reductions run as 4 waves, one per SIMD, each 128 x 128: a
      // third fewer LDS fragment bytes per multiply than 8 waves of 128 x 64,
      // which the power-limited clock turns into speed.  Measured slower
      // with 4: epilogues that read operands (the activation backward), the
      // W2 forward, and short reductions (8 steps of 64: the tile's fill and
      // epilogue, with no second wave per SIMD, cost 0.16 ms against 0.12)
      if (pl.bm == 256 && pl.bn == 256 && a.K >= 4096 && (dual || (epi == EPI_STORE && a.b_nk))) pl.nw = 4;
      pl.slots = (pl.nw / 2) * pl.n_tiles;
      pl.grid = pad8(int64_t(a.mt_ub) * pl.n_tiles);
    } else {
      pl.bm = a.Mo >= 256 ? 256 : 128;
      pl.bn = a.N >= 256 ? 256 : 128;
      pl.n_tiles = int(ceil_div(a.Mo, pl.bm) * ceil_div(a.N, pl.bn));
      pl.slots = 0;
    }
  }
  if (mode == SEG_K) {
    // rows per chunk: enough chunks to give ~2 tiles per CU (more chunks
    // cost more in partials written and summed than they gain in balance),
    // at least one K step per chunk; experts with fewer rows form a single
    // chunk.
    const int64_t want_chunks = std::max<int64_t>(1, ceil_div(2 * kCUs, pl.n_tiles));
    int64_t ks = ceil_div(std::max(a.M, 1), want_chunks);
    ks = std::max<int64_t>(256, ceil_div(ks, 64) * 64);
    a.KS = int(std::min<int64_t>(ks, int64_t(1) << 30));
    a.mt_ub = int(ceil_div(a.M, a.KS) + a.E);
    pl.grid = pad8(int64_t(a.mt_ub) * pl.n_tiles);
  }
  return true;
}


template <int MODE, int EPI, int BNK, bool DUAL>
static void go_f32(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL((gemm_f32_kernel<MODE, EPI, BNK, DUAL>), dim3(unsigned(pl.grid)), dim3(kFThreads), 0, st, a);
}

// out_f32: 1 when c0 is fp32 (scattered pairs, weight gradients)
static bool dispatch(const GemmArgs& a, const GemmPlan& pl, int out_f32, hipStream_t st) {
  if (!pl.bf16) {
    if (pl.mode == SEG_K) { go_f32<SEG_K, EPI_PARTIAL, 0, false>(a, pl, st); return true; }   // reads kscale itself
    switch (pl.epi) {
      case EPI_STORE:
        if (a.b_nk) go_f32<SEG_M, EPI_STORE, 1, false>(a, pl, st);
        else go_f32<SEG_M, EPI_STORE, 0, false>(a, pl, st);
        return true;
      case EPI_GELU_FWD: go_f32<SEG_M, EPI_GELU_FWD, 0, false>(a, pl, st); return true;
      case EPI_SWIGLU_FWD: go_f32<SEG_M, EPI_SWIGLU_FWD, 0, true>(a, pl, st); return true;
      case EPI_GELU_BWD: go_f32<SEG_M, EPI_GELU_BWD, 1, false>(a, pl, st); return true;
      case EPI_SWIGLU_BWD: go_f32<SEG_M, EPI_SWIGLU_BWD, 1, false>(a, pl, st); return true;
    }
    return false;
  }
  if (pl.mode == SEG_K) return dispatch_bf16_dw(a, pl, st);
  switch (pl.epi) {
    case EPI_STORE:
      return a.b_nk ? dispatch_bf16_store_k(a, pl, out_f32, st) : dispatch_bf16_store_mn(a, pl, out_f32, st);
    case EPI_GELU_FWD:
    case EPI_SWIGLU_FWD: return dispatch_bf16_act_fwd(a, pl, st);
    case EPI_GELU_BWD:
    case EPI_SWIGLU_BWD: return dispatch_bf16_act_bwd(a, pl, st);
  }
  return false;
}

int64_t whole_round_tiles(const GemmArgs& a, const GemmPlan& pl) {
  constexpr int kCUs = 256, kGM = 8;
  if (!pl.bf16 || pl.mode != SEG_M) return 0;
  // every expert's rows fill at least ceil(M / bm) m-tiles in all; tiles
  // come in groups of kGM m-tiles by all n-tiles, so whole groups below that
  // count are real
  const int64_t mt_real = ceil_div(a.M, pl.bm);
  const int64_t t = (mt_real / kGM) * kGM * pl.n_tiles;
  return (t / kCUs) * kCUs;
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if (pl.grid <= 0) return hipSuccess;
  if (pl.grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  // the bf16 weight-gradient kernel copies row indices for both operands,
  // gathered or not: it needs a readable index array of M entries
  if (pl.mode == SEG_K && pl.bf16 && a.sidx == nullptr) return hipErrorInvalidValue;
  if (!dispatch(a, pl, pl.mode == SEG_K ? 1 : pl.out_f32, st)) return hipErrorInvalidConfiguration;
  return hipGetLastError();
}

}  // namespace smoe
