// Segmented grouped GEMM over scattered rows for gfx950 (CDNA4).
//
// One kernel family serves every product of the hot path (ParallelLinear /
// scatter2scatter forward in the four layouts, its dX against W^T, and the
// per-expert weight gradient "groupXtY"); see the SEG_M / SEG_K contract in
// kernels.h.  Rows are read straight from their scattered positions through
// sorted_scattered_idxs and results are written grouped or scattered, so no
// padded or copied grouped input ever exists (catalogue record "Scattered
// Mixture-of-Experts Implementation", abstract; review page, second review,
// Summary: grouped GEMM fused with scattered reads and writes).
//
// bf16 kernel (MFMA):
//  - 256 threads = 4 waves in a 2x2 grid; block tile BM x BN (128 or 256),
//    K step 64; each wave owns (BM/2) x (BN/2) as 32x32 fragments of
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
//  - LDS holds both operands as [row][64 k] bf16 (128-byte rows), 16-byte
//    chunk c of row j stored at chunk c ^ (j & 7): MFMA fragment reads,
//    direct row loads and the 8x8 transposing stores are all free of bank
//    conflicts.  Two stages; one barrier per K step.
//  - Operands whose K axis is contiguous in memory (gathered token rows,
//    W[e] read as W^T) are copied 16 bytes per lane.  Operands whose K axis
//    is strided (W[e] in the forward, both operands of the weight gradient)
//    are read as 8 K-rows x 16 bytes per lane and transposed 8x8 in
//    registers on the way into LDS.
//  - The MFMA is issued with the B fragment first, so each lane ends up
//    holding one output row and runs of 4 consecutive columns: epilogue
//    stores are 8 bytes (bf16) or 16 bytes (fp32) wide.
//  - Workgroups are renumbered so that each XCD (blockIdx % 8 on MI355X)
//    receives a contiguous range of tiles, and tiles are ordered in groups
//    of 8 m-tiles sweeping n, so the tiles resident on one XCD share their
//    A rows and weight panels in that XCD's L2.
//
// fp32 kernel: the same contract with plain FMA on 64x64 tiles, used for
// fp32 runs (a small, launch-bound regime).
#include "common.h"
#include "kernels.h"

namespace smoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kRowBytes = kBK * 2;

SMOE_DEV int xcd_remap(int b, int nblk) {
  const int per = nblk >> 3;  // the host pads the grid to a multiple of 8
  return (b & 7) * per + (b >> 3);
}

SMOE_DEV uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// 8x8 transpose of bf16 held as 8 rows of 8 (two per dword).
SMOE_DEV void transpose8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t s[32], o[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i * 4 + 0] = in[i].x; s[i * 4 + 1] = in[i].y; s[i * 4 + 2] = in[i].z; s[i * 4 + 3] = in[i].w;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t a = s[(2 * d) * 4 + j / 2], b = s[(2 * d + 1) * 4 + j / 2];
      o[j * 4 + d] = (j & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u) : __builtin_amdgcn_perm(b, a, 0x05040100u);
    }
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = make_uint4(o[j * 4 + 0], o[j * 4 + 1], o[j * 4 + 2], o[j * 4 + 3]);
}

// multiply the 8 bf16 values of a row by g and round back to bf16
SMOE_DEV uint4 scale8(uint4 v, float g) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float lo = __uint_as_float(w[d] << 16) * g, hi = __uint_as_float(w[d] & 0xffff0000u) * g;
    w[d] = uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int BM, int BN, int MODE, int EPI, int BNK, bool DUAL>
struct TileShape {
  static constexpr int FM = BM / 64, FN = BN / 64;
  static constexpr int NCOLS = DUAL ? BN / 2 : BN;  // real output columns per tile
};

// Which tile this workgroup computes.  Returns false if none.
struct TileInfo {
  Item it;
  int chunk;  // SEG_K chunk index
  int m0;     // SEG_K: first output row;  SEG_M: unused
  int n0;     // first output column (real)
  int nt;     // SEG_M n-tile index
};

template <int BM, int BN, int MODE, bool DUAL>
SMOE_DEV bool tile_of_block(const GemmArgs& p, TileInfo& t) {
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  if constexpr (MODE == SEG_M) {
    constexpr int NCOLS = DUAL ? BN / 2 : BN;
    const int ntn = (p.N + NCOLS - 1) / NCOLS;
    if (g >= p.mt_ub * ntn) return false;
    constexpr int GM = 8;
    const int group = g / (GM * ntn);
    const int gs = min(GM, p.mt_ub - group * GM);
    const int local = g - group * GM * ntn;
    const int mt = group * GM + local % gs;
    t.nt = local / gs;
    t.n0 = t.nt * NCOLS;
    t.m0 = 0;
    t.chunk = 0;
    return find_item(p.offsets, p.E, BM, mt, t.it);
  } else {
    const int ti = (p.Mo + BM - 1) / BM, tj = (p.N + BN - 1) / BN, tpc = ti * tj;
    if (g >= p.mt_ub * tpc) return false;
    t.chunk = g / tpc;
    const int rem = g - t.chunk * tpc;
    t.m0 = (rem / tj) * BM;
    t.n0 = (rem % tj) * BN;
    t.nt = 0;
    return find_item(p.offsets, p.E, p.KS, t.chunk, t.it);
  }
}

template <int BM, int BN, int MODE, int EPI, int BNK, bool DUAL, class OutT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes, STAGE = A_BYTES + B_BYTES;
  static_assert(!DUAL || (MODE == SEG_M && BNK == 0 && BN >= 128), "dual B layout");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  TileInfo T;
  if (!tile_of_block<BM, BN, MODE, DUAL>(p, T)) return;
  const Item& it = T.it;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int kb = tid & 7;    // 16-byte chunk (8 k) this thread moves
  const int rb = tid >> 3;   // row / 8-column block this thread moves

  // ---------------- per-thread operand addressing --------------------------
  const uint16_t* a0 = static_cast<const uint16_t*>(p.a0);
  const uint16_t* a1 = static_cast<const uint16_t*>(p.a1);
  const uint16_t* b0 = static_cast<const uint16_t*>(p.b0);
  const uint16_t* b1 = static_cast<const uint16_t*>(p.b1);

  constexpr int AR = BM / 32;                    // SEG_M: A rows per thread
  constexpr int BR = BN / 32;                    // SEG_M, BNK: B rows per thread
  int64_t a_off[MODE == SEG_M ? AR : 1];
  bool a_ok[MODE == SEG_M ? AR : 1];
  int64_t b_off[(MODE == SEG_M && BNK) ? BR : 1];
  bool b_ok[(MODE == SEG_M && BNK) ? BR : 1];
  const uint16_t* bt_base = nullptr;             // SEG_M, W[k][n]: column block base
  bool bt_ok = false;
  int Kloop;

  if constexpr (MODE == SEG_M) {
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      const int gr = it.row0 + rb + 32 * i;
      a_ok[i] = gr < it.row1;
      const int src = a_ok[i] ? (p.a_scat ? p.sidx[gr] / p.a_fan : gr) : 0;
      a_off[i] = int64_t(src) * p.lda;
    }
    if constexpr (BNK) {
#pragma unroll
      for (int i = 0; i < BR; ++i) {
        const int n = T.n0 + rb + 32 * i;
        b_ok[i] = n < p.N;
        b_off[i] = int64_t(it.e) * p.b_es + int64_t(b_ok[i] ? n : 0) * p.ldb;
      }
    } else {
      if (rb < BN / 8) {
        const int j = rb * 8;  // tile column block
        int col;
        const uint16_t* base = b0;
        if constexpr (DUAL) {
          const int wnp = j / (BN / 2), jj = j % (BN / 2);
          base = (jj / (BN / 4)) ? b1 : b0;
          col = T.n0 + wnp * (BN / 4) + jj % (BN / 4);
        } else {
          col = T.n0 + j;
        }
        bt_ok = col < p.N;
        bt_base = base + int64_t(it.e) * p.b_es + (bt_ok ? col : 0);
      }
    }
    Kloop = p.K;
  } else {
    Kloop = it.row1 - it.row0;
  }
  const int KT = (Kloop + kBK - 1) / kBK;

  // ---------------- global -> register prefetch ----------------------------
  uint4 ra[MODE == SEG_M ? AR : 8];
  uint4 rbv[(MODE == SEG_M && BNK) ? BR : 8];

  auto load = [&](int kt) {
    const int k0 = kt * kBK;
    if constexpr (MODE == SEG_M) {
      const int kk = k0 + kb * 8;
      const bool kok = kk < p.K;
      const uint16_t* abase = kk < p.K0 ? a0 + kk : a1 + (kk - p.K0);
#pragma unroll
      for (int i = 0; i < AR; ++i) ra[i] = (a_ok[i] && kok) ? ldg16(abase + a_off[i]) : make_uint4(0, 0, 0, 0);
      if constexpr (BNK) {
        const uint16_t* bbase = kk < p.K0 ? b0 + kk : b1 + (kk - p.K0);
#pragma unroll
        for (int i = 0; i < BR; ++i) rbv[i] = (b_ok[i] && kok) ? ldg16(bbase + b_off[i]) : make_uint4(0, 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + kb * 8 + i;
          rbv[i] = (bt_ok && k < p.K) ? ldg16(bt_base + int64_t(k) * p.ldb) : make_uint4(0, 0, 0, 0);
        }
      }
    } else {
      // eight consecutive grouped rows of this chunk feed both operands
      const int ia = T.m0 + rb * 8, jb = T.n0 + rb * 8;
      const bool aok = rb < BM / 8 && ia < p.Mo;
      const bool bok = rb < BN / 8 && jb < p.N;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = it.row0 + k0 + kb * 8 + i;
        const bool rok = r < it.row1;
        int s = 0;
        if (rok && (p.a_scat || p.b_scat || p.b_gate)) s = p.sidx[r];
        const int arow = p.a_scat ? s / p.a_fan : r;
        const int brow = p.b_scat ? s / p.b_fan : r;
        ra[i] = (rok && aok) ? ldg16(a0 + int64_t(arow) * p.lda + ia) : make_uint4(0, 0, 0, 0);
        uint4 v = (rok && bok) ? ldg16(b0 + int64_t(brow) * p.ldb + jb) : make_uint4(0, 0, 0, 0);
        if (p.b_gate) v = scale8(v, rok ? p.b_gate[s] : 0.f);
        rbv[i] = v;
      }
    }
  };

  // ---------------- register -> LDS --------------------------------------
  auto store = [&](int stage) {
    char* As = smem + stage * STAGE;
    char* Bs = As + A_BYTES;
    if constexpr (MODE == SEG_M) {
#pragma unroll
      for (int i = 0; i < AR; ++i) {
        const int row = rb + 32 * i;
        *reinterpret_cast<uint4*>(As + row * kRowBytes + ((kb ^ (row & 7)) << 4)) = ra[i];
      }
      if constexpr (BNK) {
#pragma unroll
        for (int i = 0; i < BR; ++i) {
          const int row = rb + 32 * i;
          *reinterpret_cast<uint4*>(Bs + row * kRowBytes + ((kb ^ (row & 7)) << 4)) = rbv[i];
        }
      } else if (rb < BN / 8) {
        uint4 t[8];
        transpose8(rbv, t);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(Bs + (rb * 8 + j) * kRowBytes + ((kb ^ j) << 4)) = t[j];
      }
    } else {
      uint4 t[8];
      if (rb < BM / 8) {
        transpose8(ra, t);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(As + (rb * 8 + j) * kRowBytes + ((kb ^ j) << 4)) = t[j];
      }
      if (rb < BN / 8) {
        transpose8(rbv, t);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(Bs + (rb * 8 + j) * kRowBytes + ((kb ^ j) << 4)) = t[j];
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (KT > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  const int rsw = lane & 7;  // fragment rows are 32-aligned, so row & 7 == lane & 7
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load(kt + 1);
    const char* As = smem + cur * STAGE;
    const char* Bs = As + A_BYTES;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int coff = ((2 * s + (lane >> 5)) ^ rsw) << 4;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const bf16x8_t*>(As + (wm * (BM / 2) + fm * 32 + (lane & 31)) * kRowBytes + coff);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bfr[fn] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * (BN / 2) + fn * 32 + (lane & 31)) * kRowBytes + coff);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fn], af[fm], acc[fm][fn], 0, 0, 0);
    }
    if (kt + 1 < KT) store(cur ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue ----------------------------------------------
  // lane holds, for fragment (fm, fn): row (lane & 31) and columns
  // 8q + 4*(lane >> 5) + {0..3}, q = 0..3, values acc[fm][fn][4q + i].
  const int csub = 4 * (lane >> 5);
  if constexpr (MODE == SEG_K) {
    float* dst = (it.nitems == 1) ? static_cast<float*>(p.c0) + int64_t(it.e) * p.Mo * p.N
                                  : p.partial + int64_t(T.chunk) * p.Mo * p.N;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = T.m0 + wm * (BM / 2) + fm * 32 + (lane & 31);
      if (i >= p.Mo) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = T.n0 + wn * (BN / 2) + fn * 32 + 8 * q + csub;
          if (j < p.N) {
            const float v[4] = {acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                                acc[fm][fn][4 * q + 3]};
            st4<float>(dst + int64_t(i) * p.N + j, v);
          }
        }
    }
  } else {
    OutT* c0 = static_cast<OutT*>(p.c0);
    OutT* c1 = static_cast<OutT*>(p.c1);
    OutT* c2 = static_cast<OutT*>(p.c2);
    const uint16_t* x0 = static_cast<const uint16_t*>(p.aux0);
    const uint16_t* x1 = static_cast<const uint16_t*>(p.aux1);
    constexpr int FNR = DUAL ? FN / 2 : FN;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int gr = it.row0 + wm * (BM / 2) + fm * 32 + (lane & 31);
      const bool rok = gr < it.row1;
      const int sp = rok ? p.sidx[gr] : 0;
      const float g = (p.gate && rok) ? p.gate[sp] : 1.f;
      const int64_t crow = p.c_scat ? sp : gr;
      const int64_t xrow = p.aux_scat ? sp / p.aux_fan : gr;
      float dgacc = 0.f;
#pragma unroll
      for (int fn = 0; fn < FNR; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = T.n0 + (DUAL ? wn * (BN / 4) : wn * (BN / 2)) + fn * 32 + 8 * q + csub;
          if (!rok || n >= p.N) continue;
          float v[4] = {acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]};
          if constexpr (EPI == EPI_STORE) {
            if (p.dgpart) {
              float xv[4];
              ld4<uint16_t>(x0 + xrow * p.ldaux + n, xv);
              dgacc += xv[0] * v[0] + xv[1] * v[1] + xv[2] * v[2] + xv[3] * v[3];
            }
            if (c0) {
              if (p.gate) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] *= g;
              }
              st4<OutT>(c0 + crow * p.ldc + n, v);
            }
          } else if constexpr (EPI == EPI_GELU_FWD) {
            float h[4], a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              h[i] = stored<OutT>(v[i]);
              a[i] = gelu_f(h[i]);
            }
            st4<OutT>(c0 + int64_t(gr) * p.ldc + n, h);
            st4<OutT>(c1 + int64_t(gr) * p.ldc + n, a);
          } else if constexpr (EPI == EPI_SWIGLU_FWD) {
            float h1[4], h3[4], a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              h1[i] = stored<OutT>(v[i]);
              h3[i] = stored<OutT>(acc[fm][fn + FN / 2][4 * q + i]);
              a[i] = silu_f(h1[i]) * h3[i];
            }
            st4<OutT>(c0 + int64_t(gr) * p.ldc + n, h1);
            st4<OutT>(c1 + int64_t(gr) * p.ldc + n, h3);
            st4<OutT>(c2 + int64_t(gr) * p.ldc + n, a);
          } else if constexpr (EPI == EPI_GELU_BWD) {
            float h[4], dh[4];
            ld4<uint16_t>(x0 + int64_t(gr) * p.ldaux + n, h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dgacc += stored<OutT>(gelu_f(h[i])) * v[i];
              dh[i] = g * v[i] * gelu_grad_f(h[i]);
            }
            st4<OutT>(c0 + int64_t(gr) * p.ldc + n, dh);
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            float h1[4], h3[4], d1[4], d3[4];
            ld4<uint16_t>(x0 + int64_t(gr) * p.ldaux + n, h1);
            ld4<uint16_t>(x1 + int64_t(gr) * p.ldaux + n, h3);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sg = silu_f(h1[i]);
              dgacc += stored<OutT>(sg * h3[i]) * v[i];
              const float dA = g * v[i];
              d1[i] = dA * h3[i] * silu_grad_f(h1[i]);
              d3[i] = dA * sg;
            }
            st4<OutT>(c0 + int64_t(gr) * p.ldc + n, d1);
            st4<OutT>(c1 + int64_t(gr) * p.ldc + n, d3);
          }
        }
      if (p.dgpart) {
        dgacc += __shfl_xor(dgacc, 32, kWave);
        if (lane < 32 && rok) p.dgpart[int64_t(T.nt * 2 + wn) * p.M + gr] = dgacc;
      }
    }
  }
}

// ============================================================================
// fp32 kernel: 64x64 tiles, K step 16, 256 threads each owning 4x4 outputs
// (rows ty*4+i, columns tx*4+j).  Element-wise operand access through the
// same contract as the bf16 kernel.
// ============================================================================
constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <int MODE, int EPI, int BNK, bool DUAL>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs p) {
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

  auto Aval = [&](int m, int k) -> float {  // m tile-local, k absolute (SEG_M) / chunk-local (SEG_K)
    if constexpr (MODE == SEG_M) {
      const int gr = it.row0 + m;
      if (gr >= it.row1 || k >= p.K) return 0.f;
      const int src = p.a_scat ? p.sidx[gr] / p.a_fan : gr;
      return k < p.K0 ? a0[int64_t(src) * p.lda + k] : a1[int64_t(src) * p.lda + (k - p.K0)];
    } else {
      const int r = it.row0 + k, i = T.m0 + m;
      if (r >= it.row1 || i >= p.Mo) return 0.f;
      const int src = p.a_scat ? p.sidx[r] / p.a_fan : r;
      return a0[int64_t(src) * p.lda + i];
    }
  };
  auto Bval = [&](int k, int n, int which) -> float {  // n tile-local
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
      int s = (p.b_scat || p.b_gate) ? p.sidx[r] : 0;
      const int src = p.b_scat ? s / p.b_fan : r;
      const float g = p.b_gate ? p.b_gate[s] : 1.f;
      return g * b0[int64_t(src) * p.ldb + j];
    }
  };

  float acc[4][4] = {}, acc3[4][4] = {};
  for (int k0 = 0; k0 < Kloop; k0 += kFBK) {
    for (int l = tid; l < kFBK * kFBM; l += kThreads) {
      const int m = l / kFBK, kk = l % kFBK;
      As[kk][m] = Aval(m, k0 + kk);
    }
    for (int l = tid; l < kFBK * kFBN; l += kThreads) {
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
    float* dst = (it.nitems == 1) ? static_cast<float*>(p.c0) + int64_t(it.e) * p.Mo * p.N
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
            st4<float>(c0 + crow * p.ldc + n, v);
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
          float h[4], dh[4];
          ld4<float>(x0 + int64_t(gr) * p.ldaux + n, h);
          for (int j = 0; j < 4; ++j) {
            dgacc += gelu_f(h[j]) * v[j];
            dh[j] = g * v[j] * gelu_grad_f(h[j]);
          }
          st4<float>(c0 + int64_t(gr) * p.ldc + n, dh);
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
          float h1[4], h3[4], d1[4], d3[4];
          ld4<float>(x0 + int64_t(gr) * p.ldaux + n, h1);
          ld4<float>(x1 + int64_t(gr) * p.ldaux + n, h3);
          for (int j = 0; j < 4; ++j) {
            const float sg = silu_f(h1[j]);
            dgacc += sg * h3[j] * v[j];
            d1[j] = g * v[j] * h3[j] * silu_grad_f(h1[j]);
            d3[j] = g * v[j] * sg;
          }
          st4<float>(c0 + int64_t(gr) * p.ldc + n, d1);
          st4<float>(c1 + int64_t(gr) * p.ldc + n, d3);
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
  pl.out_f32 = out_f32;
  pl.epi = epi;
  pl.dual = dual;
  pl.bf16 = bf16;
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
      const int ncols_needed = dual ? 2 * a.N : a.N;
      const int64_t rows_per_expert = std::max<int64_t>(1, a.M / std::max(1, a.E));
      pl.bn = (ncols_needed >= 256) ? 256 : 128;
      pl.bm = (rows_per_expert >= 192) ? 256 : 128;
      // prefer smaller tiles when the big ones leave most CUs idle
      auto tiles = [&](int bm, int bn) {
        const int ncols = dual ? bn / 2 : bn;
        return (ceil_div(a.M, bm) + a.E / 2) * ceil_div(a.N, ncols);
      };
      if (tiles(pl.bm, pl.bn) < 2 * kCUs && pl.bm == 256) pl.bm = 128;
      if (tiles(pl.bm, pl.bn) < 2 * kCUs && pl.bn == 256) pl.bn = 128;
      a.mt_ub = int(ceil_div(a.M, pl.bm) + a.E);
      const int ncols = dual ? pl.bn / 2 : pl.bn;
      pl.n_tiles = int(ceil_div(a.N, ncols));
      pl.slots = 2 * pl.n_tiles;
      pl.grid = pad8(int64_t(a.mt_ub) * pl.n_tiles);
    } else {
      pl.bm = a.Mo >= 256 ? 256 : 128;
      pl.bn = a.N >= 256 ? 256 : 128;
      pl.n_tiles = int(ceil_div(a.Mo, pl.bm) * ceil_div(a.N, pl.bn));
      pl.slots = 0;
    }
  }
  if (mode == SEG_K) {
    // rows per chunk: enough chunks to give ~4 tiles per CU, at least one K
    // step per chunk; experts with fewer rows form a single chunk.
    const int64_t want_chunks = std::max<int64_t>(1, ceil_div(4 * kCUs, pl.n_tiles));
    int64_t ks = ceil_div(std::max(a.M, 1), want_chunks);
    ks = std::max<int64_t>(256, ceil_div(ks, 64) * 64);
    a.KS = int(std::min<int64_t>(ks, int64_t(1) << 30));
    a.mt_ub = int(ceil_div(a.M, a.KS) + a.E);
    pl.grid = pad8(int64_t(a.mt_ub) * pl.n_tiles);
  }
  return true;
}

template <int BM, int BN, int MODE, int EPI, int BNK, bool DUAL, class OutT>
static void go_bf16(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, MODE, EPI, BNK, DUAL, OutT>), dim3(unsigned(pl.grid)),
                     dim3(kThreads), 0, st, a);
}

template <int MODE, int EPI, int BNK, bool DUAL, class OutT>
static bool dispatch_tiles(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if (pl.bm == 256 && pl.bn == 256) go_bf16<256, 256, MODE, EPI, BNK, DUAL, OutT>(a, pl, st);
  else if (pl.bm == 256 && pl.bn == 128) go_bf16<256, 128, MODE, EPI, BNK, DUAL, OutT>(a, pl, st);
  else if (pl.bm == 128 && pl.bn == 256) go_bf16<128, 256, MODE, EPI, BNK, DUAL, OutT>(a, pl, st);
  else if (pl.bm == 128 && pl.bn == 128) go_bf16<128, 128, MODE, EPI, BNK, DUAL, OutT>(a, pl, st);
  else return false;
  return true;
}

template <int MODE, int EPI, int BNK, bool DUAL>
static void go_f32(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL((gemm_f32_kernel<MODE, EPI, BNK, DUAL>), dim3(unsigned(pl.grid)), dim3(kThreads), 0, st, a);
}

// out_f32: 1 when c0 is fp32 (scattered pairs, weight gradients)
static bool dispatch(const GemmArgs& a, const GemmPlan& pl, int out_f32, hipStream_t st) {
  if (!pl.bf16) {
    if (pl.mode == SEG_K) { go_f32<SEG_K, EPI_PARTIAL, 0, false>(a, pl, st); return true; }
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
  if (pl.mode == SEG_K) return dispatch_tiles<SEG_K, EPI_PARTIAL, 0, false, float>(a, pl, st);
  switch (pl.epi) {
    case EPI_STORE:
      if (a.b_nk) {
        return out_f32 ? dispatch_tiles<SEG_M, EPI_STORE, 1, false, float>(a, pl, st)
                       : dispatch_tiles<SEG_M, EPI_STORE, 1, false, uint16_t>(a, pl, st);
      }
      return out_f32 ? dispatch_tiles<SEG_M, EPI_STORE, 0, false, float>(a, pl, st)
                     : dispatch_tiles<SEG_M, EPI_STORE, 0, false, uint16_t>(a, pl, st);
    case EPI_GELU_FWD: return dispatch_tiles<SEG_M, EPI_GELU_FWD, 0, false, uint16_t>(a, pl, st);
    case EPI_SWIGLU_FWD: return dispatch_tiles<SEG_M, EPI_SWIGLU_FWD, 0, true, uint16_t>(a, pl, st);
    case EPI_GELU_BWD: return dispatch_tiles<SEG_M, EPI_GELU_BWD, 1, false, uint16_t>(a, pl, st);
    case EPI_SWIGLU_BWD: return dispatch_tiles<SEG_M, EPI_SWIGLU_BWD, 1, false, uint16_t>(a, pl, st);
  }
  return false;
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if (pl.grid <= 0) return hipSuccess;
  if (pl.grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (!dispatch(a, pl, pl.mode == SEG_K ? 1 : pl.out_f32, st)) return hipErrorInvalidConfiguration;
  return hipGetLastError();
}

}  // namespace smoe
