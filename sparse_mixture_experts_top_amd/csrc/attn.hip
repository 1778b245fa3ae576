// Mixture-of-Attention core on the matrix cores (article "This Machine
// Learning Research Presents ScatterMoE", body, para. 4: the head experts
// of Mixture-of-Attention run on the same grouped products, with no extra
// memory).  Query row r is in grouped order (as the scattered-in /
// grouped-out Q projection writes it) and belongs to token t = s_r / k; it
// attends causally within its sequence (keys t' of the same sequence with
// t' <= t, sequences of S tokens) to keys and values shared by all experts;
// the output row stays in grouped order, ready for the grouped-in O
// projection.  bf16 operands, fp32 accumulation, head_dim 128.
//
// Matrix-core layout.  v_mfma_f32_32x32x16_bf16 is issued with the
// 32-row "column" operand first, as in the grouped products, so a lane ends
// up holding one row (lane & 31) of the result and columns 8q + 4h + i
// (h = lane >> 5) in acc[4q + i].  The scores of a 32-key block are formed
// with the key rows loaded in the order pi(c) (bits 2 and 3 of the column
// index swapped): a lane's scores for k-step s of the following product then
// cover keys 16s + 8h + 0..7 in register order, which is exactly the A
// operand layout that product needs, so the probabilities feed P V (and, in
// the backward, dS K) with no shuffle.  V (and the backward's other
// right-hand operands) are read from LDS with gfx950's transposing read.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace smoe {

typedef __bf16 at_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float at_f32x16_t __attribute__((ext_vector_type(16)));
typedef short at_i16x4_t __attribute__((ext_vector_type(4)));
typedef short at_i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void at_lds_void_t;
typedef __attribute__((address_space(3))) at_i16x4_t at_lds_i16x4_t;

constexpr int kHD = 128;          // head dim
constexpr int kRowB = kHD * 2;    // bytes per row of a bf16 tile
constexpr int kKB = 32;           // keys per block
constexpr int kAttnThreads = 256;
constexpr int kAttnRows = 128;    // query rows per block (32 per wave)

SMOE_DEV int key_perm(int c) { return (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1); }

// Row tiles [32 rows][128] bf16 in LDS, 16 chunks of 16 bytes per row.
// Row-read layout (a lane reads one row's chunk): chunk c of row r at
// c ^ (r & 15), so 16 consecutive rows put a given chunk on 16 distinct
// bank groups.  Transposing-read layout (a lane gathers one column over 4
// rows): chunk c at c ^ ((r & 3) << 2).
SMOE_DEV int swz_row(int r) { return r & 15; }
SMOE_DEV int swz_tr(int r) { return (r & 3) << 2; }

// 8 consecutive head-dim values of tile row `row`, k-step s, half h, from a
// row-read (TR = false) or transposing-read (TR = true) layout tile
template <bool TR = false>
SMOE_DEV at_bf16x8_t row_frag(const char* tile, int row, int s, int h) {
  const int c = (2 * s + h) ^ (TR ? swz_tr(row) : swz_row(row));
  return *reinterpret_cast<const at_bf16x8_t*>(tile + row * kRowB + (c << 4));
}

// MFMA operand from a transposing-layout tile [k-rows][128 cols]: lane gets
// column m0 + (lane & 31) at k-rows 16s + 8h + 0..7 (h = lane >> 5).  Within
// each 16-lane group, lane i addresses k-row kb + (i >> 2), columns
// mb + 4 (i & 3) .. +3 and receives column mb + i at k-rows kb .. kb+3.
SMOE_DEV at_bf16x8_t tr_frag(const char* tile, int m0, int s, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int mn = m0 + 16 * (grp & 1) + 4 * (i & 3);
  const int kr = 16 * s + 8 * (grp >> 1) + (i >> 2);
  const int c = mn >> 3, within = (mn & 7) * 2;
  const char* p0 = tile + kr * kRowB + ((c ^ swz_tr(kr)) << 4) + within;
  const char* p1 = tile + (kr + 4) * kRowB + ((c ^ swz_tr(kr + 4)) << 4) + within;
  const at_i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_i16x4_t*)(const at_lds_void_t*)p0);
  const at_i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_i16x4_t*)(const at_lds_void_t*)p1);
  const at_i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(at_bf16x8_t, v);
}

// bf16 A operands of k-step s from a lane's 16 accumulator values (keys or
// queries in the pi order, see the file comment), as two halves hi =
// bf16(v) and lo = bf16(v - hi): the product with both carries v to about
// 16 significant bits (one bf16 rounding of the probabilities alone would
// cost up to 2^-9 of each term)
SMOE_DEV void acc_frags(const float (&p)[16], int s, at_bf16x8_t& hi, at_bf16x8_t& lo) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float v = p[8 * s + m];
    const __bf16 b = static_cast<__bf16>(v);
    hi[m] = b;
    lo[m] = static_cast<__bf16>(v - static_cast<float>(b));
  }
}

// A 32-row tile (rows row0 .. row0+31 of a [n][128] tensor, zeros past n)
// moved by 256 threads: two 16-byte pieces per thread, held in registers
// between the load and the LDS store so the load can run ahead.
struct TileRegs {
  uint4 v[2];
};
SMOE_DEV void tile_load(TileRegs& r, const uint16_t* src, int64_t row0, int64_t n) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = threadIdx.x + u * kAttnThreads;
    const int row = i >> 4, c = i & 15;
    const int64_t g = row0 + row;
    r.v[u] = g < n ? *reinterpret_cast<const uint4*>(src + g * kHD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
}
template <bool TR>
SMOE_DEV void tile_store(const TileRegs& r, char* tile) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = threadIdx.x + u * kAttnThreads;
    const int row = i >> 4, c = i & 15;
    const int pc = c ^ (TR ? swz_tr(row) : swz_row(row));
    *reinterpret_cast<uint4*>(tile + row * kRowB + (pc << 4)) = r.v[u];
  }
}

// Block-wide [min lo, max t] over the block's rows (t = -1, lo = big for
// rows past M); every thread gets the result.
SMOE_DEV void block_range(int lo, int t, int* red, int& blo, int& bhi) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o, kWave));
    t = max(t, __shfl_xor(t, o, kWave));
  }
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) {
    red[2 * w] = lo;
    red[2 * w + 1] = t;
  }
  __syncthreads();
  blo = red[0];
  bhi = red[1];
#pragma unroll
  for (int i = 1; i < kAttnThreads / kWave; ++i) {
    blo = min(blo, red[2 * i]);
    bhi = max(bhi, red[2 * i + 1]);
  }
}

// ---- forward ---------------------------------------------------------------
// Block: 128 query rows and 8 waves, wave w = (row tile w & 3, key half
// w >> 2); lane: row lane & 31 of its tile.  Per step of 64 keys the block
// stages two 32-key K and V tiles in LDS and each wave takes the tile of its
// half, so K and V cross from L2 once per 128 rows.  Each wave keeps its own
// online-softmax state (base 2); at the end the second half's state goes
// through LDS to the first: O = (2^(m0-M) O0 + 2^(m1-M) O1) / (2^(m0-M) l0 +
// 2^(m1-M) l1).
constexpr int kFwdThreads = 512;
constexpr int kFwdWaves = kFwdThreads / kWave;
constexpr int kFwdRows = 128;
constexpr int kStepKeys = 2 * kKB;   // keys staged per step
__global__ __launch_bounds__(kFwdThreads) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kk,
                                                               const uint16_t* __restrict__ v,
                                                               const int* __restrict__ sidx, int64_t M, int64_t T,
                                                               int ktop, int64_t S, uint16_t* __restrict__ o,
                                                               float* __restrict__ lse) {
  // staging: K tiles [2][32 rows], V tiles [2][32 rows]; merge: the second
  // half's O as [row tile][16 float4 slots][64 lanes]
  __shared__ __attribute__((aligned(16))) char smem[4 * 16 * kWave * 16];
  __shared__ float st_m[4][kWave], st_l[4][kWave];
  __shared__ int red[2 * kFwdWaves];
  const int lane = lane_id(), h = lane >> 5;
  const int w = threadIdx.x / kWave;
  const int rt = w & 3, kh = w >> 2;
  const int64_t r = int64_t(blockIdx.x) * kFwdRows + 32 * rt + (lane & 31);
  const bool real = r < M;
  const int t = real ? sidx[r] / ktop : -1;
  const int lo = real ? int(int64_t(t) / S * S) : 0x7fffffff;
  // block and row-tile ranges
  int wlo = lo, whi = t, wlo_max = real ? lo : -1, whi_min = real ? t : 0x7fffffff;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    wlo = min(wlo, __shfl_xor(wlo, off, kWave));
    whi = max(whi, __shfl_xor(whi, off, kWave));
    wlo_max = max(wlo_max, __shfl_xor(wlo_max, off, kWave));
    whi_min = min(whi_min, __shfl_xor(whi_min, off, kWave));
  }
  if (lane == 0) {
    red[2 * w] = wlo;
    red[2 * w + 1] = whi;
  }
  __syncthreads();
  int blo = red[0], bhi = red[1];
#pragma unroll
  for (int i = 1; i < kFwdWaves; ++i) {
    blo = min(blo, red[2 * i]);
    bhi = max(bhi, red[2 * i + 1]);
  }
  if (bhi < 0) return;   // no real rows (uniform over the block)

  at_bf16x8_t qf[8];
  const uint16_t* qr = q + (real ? r : 0) * kHD + 8 * h;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint4 x = real ? *reinterpret_cast<const uint4*>(qr + 16 * s) : make_uint4(0u, 0u, 0u, 0u);
    qf[s] = __builtin_bit_cast(at_bf16x8_t, x);
  }
  at_f32x16_t acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[nt][i] = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf(float(kHD));   // scale * log2(e)
  float m2 = -INFINITY, l = 0.f;
  // two staging buffers of 64 keys (K tiles then V tiles), alternating by
  // step, so one barrier per step both publishes a step and frees the other
  constexpr int kBufBytes = 2 * kStepKeys * kRowB;
  const int krow = key_perm(lane & 31);
  // 64 keys of K and V per step, two 16-byte pieces of each per thread,
  // loaded ahead into registers
  uint4 kv[2], vv[2];
  auto step_load = [&](int sb) SMOE_INL {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * kFwdThreads;   // 0 .. 1023: 64 rows x 16 chunks
      const int64_t g = int64_t(sb) + (i >> 4);
      const bool ok = g < T;
      kv[u] = ok ? *reinterpret_cast<const uint4*>(kk + g * kHD + (i & 15) * 8) : make_uint4(0u, 0u, 0u, 0u);
      vv[u] = ok ? *reinterpret_cast<const uint4*>(v + g * kHD + (i & 15) * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // K in the row-read layout, V in the transposing layout
  auto step_store = [&](char* buf) SMOE_INL {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * kFwdThreads;
      const int row = i >> 4, c = i & 15, tr = row & 31;
      *reinterpret_cast<uint4*>(buf + row * kRowB + ((c ^ swz_row(tr)) << 4)) = kv[u];
      *reinterpret_cast<uint4*>(buf + kStepKeys * kRowB + row * kRowB + ((c ^ swz_tr(tr)) << 4)) = vv[u];
    }
  };
  const int first = blo / kKB * kKB;
  const int nsteps = (bhi - first) / kStepKeys + 1;
  step_load(first);
  step_store(smem);
  if (nsteps > 1) step_load(first + kStepKeys);
  __syncthreads();
  for (int j = 0; j < nsteps; ++j) {
    const int sb0 = first + j * kStepKeys;
    const char* ks = smem + (j & 1) * kBufBytes + kh * kKB * kRowB;
    const char* vs = smem + (j & 1) * kBufBytes + kStepKeys * kRowB + kh * kKB * kRowB;
    const int kb0 = sb0 + kKB * kh;
    if (!(kb0 > whi || kb0 + kKB <= wlo)) {   // this wave's tile has keys for its rows (uniform)
      // scores for keys kb0 + pi(c), two accumulation chains
      at_f32x16_t sa, sb;
#pragma unroll
      for (int i = 0; i < 16; ++i) sa[i] = sb[i] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; s += 2) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(ks, krow, s, h), qf[s], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(ks, krow, s + 1, h), qf[s + 1], sb, 0, 0, 0);
      }
      // V fragments now, so their LDS reads overlap the softmax below
      at_bf16x8_t vfr[4][2];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        vfr[nt][0] = tr_frag(vs, 32 * nt, 0, lane);
        vfr[nt][1] = tr_frag(vs, 32 * nt, 1, lane);
      }
      float z[16];
      float bm = -INFINITY;
      // a tile inside every row's range of this wave needs no mask (uniform)
      const bool inner = kb0 >= wlo_max && kb0 + kKB - 1 <= whi_min;
      if (inner) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          z[i] = (sa[i] + sb[i]) * sl2;
          bm = fmaxf(bm, z[i]);
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb0 + key_perm(8 * q4 + 4 * h + i);
            const bool ok = key >= lo && key <= t;
            const float zz = ok ? (sa[4 * q4 + i] + sb[4 * q4 + i]) * sl2 : -INFINITY;
            z[4 * q4 + i] = zz;
            bm = fmaxf(bm, zz);
          }
      }
      bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
      // The reference m2 moves only when a row's max exceeds it by more than
      // 8 (base 2), so the probabilities stay below 2^8 and O and l are
      // rescaled only on those steps (for the whole wave, when any row
      // needs it).  A row with no key so far keeps m = -inf, l = 0, O = 0.
      const bool grow = bm > m2 + 8.f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float mn = fmaxf(m2, bm);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m2 - mn);
        l *= alpha;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nt][i] *= alpha;
        m2 = mn;
      }
      const bool none = m2 == -INFINITY;
      float p[16], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = none ? 0.f : __builtin_amdgcn_exp2f(z[i] - m2);
        ps += p[i];
      }
      ps += __shfl_xor(ps, 32, kWave);
      l += ps;
      at_bf16x8_t a0h, a0l, a1h, a1l;
      acc_frags(p, 0, a0h, a0l);
      acc_frags(p, 1, a1h, a1l);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const at_bf16x8_t v0 = vfr[nt][0], v1 = vfr[nt][1];
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, a0h, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, a1h, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, a0l, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, a1l, acc[nt], 0, 0, 0);
      }

    }
    if (j + 1 < nsteps) {
      step_store(smem + ((j + 1) & 1) * kBufBytes);   // read at step j - 1, freed by its barrier
      if (j + 2 < nsteps) step_load(first + (j + 2) * kStepKeys);
    }
    __syncthreads();
  }
  // the second key half hands its state to the first
  __syncthreads();
  float4* slots = reinterpret_cast<float4*>(smem) + rt * 16 * kWave;
  if (kh == 1) {
    st_m[rt][lane] = m2;
    st_l[rt][lane] = l;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        slots[(4 * nt + q4) * kWave + lane] =
            make_float4(acc[nt][4 * q4], acc[nt][4 * q4 + 1], acc[nt][4 * q4 + 2], acc[nt][4 * q4 + 3]);
  }
  __syncthreads();
  if (kh == 1 || !real) return;
  const float m1 = st_m[rt][lane], l1 = st_l[rt][lane];
  const float mx = fmaxf(m2, m1);
  const float f0 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mx);
  const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
  const float L = f0 * l + f1 * l1;
  const float inv = 1.f / L;
  uint16_t* orow = o + r * kHD;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x = slots[(4 * nt + q4) * kWave + lane];
      const float vals[4] = {(f0 * acc[nt][4 * q4] + f1 * x.x) * inv, (f0 * acc[nt][4 * q4 + 1] + f1 * x.y) * inv,
                             (f0 * acc[nt][4 * q4 + 2] + f1 * x.z) * inv, (f0 * acc[nt][4 * q4 + 3] + f1 * x.w) * inv};
      *reinterpret_cast<uint2*>(orow + 32 * nt + 8 * q4 + 4 * h) = pack4_bf16(vals);
    }
  if (h == 0) lse[r] = mx * 0.69314718055994531f + logf(L);
}

hipError_t launch_attn_fwd(const void* q, const void* kk, const void* v, const int* sidx, int64_t M, int64_t T,
                           int ktop, int64_t S, void* o, float* lse, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const unsigned grid = unsigned((M + kFwdRows - 1) / kFwdRows);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(grid), dim3(kFwdThreads), 0, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(kk), static_cast<const uint16_t*>(v), sidx, M, T, ktop, S,
                     static_cast<uint16_t*>(o), lse);
  return hipGetLastError();
}

// ---- backward ----------------------------------------------------------
// With p the probabilities of row r (recomputed from lse), dp_t' = do_r . v_t'
// and D_r = do_r . o_r (= sum_t' p dp): dz = p (dp - D_r) is the gradient of
// the scaled score; dq_r = scale dz K, dK += scale dz^T q, dV += p^T do.

// D_r, and each 32-row query tile's [lowest sequence start, highest token]
// (one wave per tile; two lanes per row, 64 head-dim values each)
__global__ __launch_bounds__(kAttnThreads) void attn_bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                                     const uint16_t* __restrict__ dout,
                                                                     const int* __restrict__ sidx, int64_t M,
                                                                     int ktop, int64_t S, float* __restrict__ D,
                                                                     int* __restrict__ tile_lo,
                                                                     int* __restrict__ tile_hi, int64_t ntiles) {
  // tile_lo / tile_hi hold, per tile: [0, ntiles) the lowest sequence start
  // and the highest token, [ntiles, 2 ntiles) the highest sequence start and
  // the lowest token (a key inside both of the latter is in every row's range)
  const int lane = lane_id();
  const int64_t tile = int64_t(blockIdx.x) * (kAttnThreads / kWave) + threadIdx.x / kWave;
  if (tile >= ntiles) return;
  const int64_t r = tile * 32 + (lane >> 1);
  const int half = lane & 1;
  const bool real = r < M;
  float sum = 0.f;
  if (real) {
    const uint4* a = reinterpret_cast<const uint4*>(o + r * kHD + 64 * half);
    const uint4* b = reinterpret_cast<const uint4*>(dout + r * kHD + 64 * half);
#pragma unroll 2
    for (int c = 0; c < 8; ++c) {
      const uint4 x = a[c], y = b[c];
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
      for (int j = 0; j < 4; ++j) {
        sum += __uint_as_float(xs[j] << 16) * __uint_as_float(ys[j] << 16);
        sum += __uint_as_float(xs[j] & 0xffff0000u) * __uint_as_float(ys[j] & 0xffff0000u);
      }
    }
  }
  sum += __shfl_xor(sum, 1, kWave);
  if (real && half == 0) D[r] = sum;
  int t = real ? sidx[r] / ktop : -1;
  int lo = real ? int(int64_t(t) / S * S) : 0x7fffffff;
  int lo_max = real ? lo : -1, t_min = real ? t : 0x7fffffff;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off, kWave));
    t = max(t, __shfl_xor(t, off, kWave));
    lo_max = max(lo_max, __shfl_xor(lo_max, off, kWave));
    t_min = min(t_min, __shfl_xor(t_min, off, kWave));
  }
  if (lane == 0) {
    tile_lo[tile] = lo;
    tile_hi[tile] = t;
    tile_lo[ntiles + tile] = lo_max;
    tile_hi[ntiles + tile] = t_min;
  }
}

// dq: blocks of 128 query rows in 8 waves, wave w = (row tile w & 3, key
// half w >> 2), as in the forward; per step of 64 keys the scores (keys in
// the pi order) and dp = do V^T (V rows in the same order) give dz in the A
// operand layout of dz K, K read back transposed from LDS.  The two halves'
// dq partials are added through LDS at the end.
__global__ __launch_bounds__(kFwdThreads) void attn_dq_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ kk,
                                                              const uint16_t* __restrict__ v,
                                                              const int* __restrict__ sidx, int64_t M, int64_t T,
                                                              int ktop, int64_t S, const float* __restrict__ lse,
                                                              const float* __restrict__ D,
                                                              const uint16_t* __restrict__ dout,
                                                              uint16_t* __restrict__ dq) {
  // staging: K tiles [2][32] (transposing layout), V tiles [2][32] (row-read
  // layout); merge: the second half's dq as [row tile][16 float4][64 lanes]
  __shared__ __attribute__((aligned(16))) char smem[4 * 16 * kWave * 16];
  __shared__ int red[2 * kFwdWaves];
  const int lane = lane_id(), h = lane >> 5;
  const int w = threadIdx.x / kWave;
  const int rt = w & 3, kh = w >> 2;
  const int64_t r = int64_t(blockIdx.x) * kFwdRows + 32 * rt + (lane & 31);
  const bool real = r < M;
  const int t = real ? sidx[r] / ktop : -1;
  const int lo = real ? int(int64_t(t) / S * S) : 0x7fffffff;
  int wlo = lo, whi = t, wlo_max = real ? lo : -1, whi_min = real ? t : 0x7fffffff;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    wlo = min(wlo, __shfl_xor(wlo, off, kWave));
    whi = max(whi, __shfl_xor(whi, off, kWave));
    wlo_max = max(wlo_max, __shfl_xor(wlo_max, off, kWave));
    whi_min = min(whi_min, __shfl_xor(whi_min, off, kWave));
  }
  if (lane == 0) {
    red[2 * w] = wlo;
    red[2 * w + 1] = whi;
  }
  __syncthreads();
  int blo = red[0], bhi = red[1];
#pragma unroll
  for (int i = 1; i < kFwdWaves; ++i) {
    blo = min(blo, red[2 * i]);
    bhi = max(bhi, red[2 * i + 1]);
  }
  if (bhi < 0) return;
  const float l2e = 1.4426950408889634f;
  const float sl2 = l2e / sqrtf(float(kHD));
  const float lse2 = real ? lse[r] * l2e : 0.f;
  const float Dr = real ? D[r] : 0.f;
  at_bf16x8_t qf[8], df[8];
  const uint16_t* qr = q + (real ? r : 0) * kHD + 8 * h;
  const uint16_t* dr = dout + (real ? r : 0) * kHD + 8 * h;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint4 a = real ? *reinterpret_cast<const uint4*>(qr + 16 * s) : make_uint4(0u, 0u, 0u, 0u);
    uint4 b = real ? *reinterpret_cast<const uint4*>(dr + 16 * s) : make_uint4(0u, 0u, 0u, 0u);
    qf[s] = __builtin_bit_cast(at_bf16x8_t, a);
    df[s] = __builtin_bit_cast(at_bf16x8_t, b);
  }
  at_f32x16_t acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[nt][i] = 0.f;
  char* ktiles = smem;
  char* vtiles = smem + kStepKeys * kRowB;
  const char* ks = ktiles + kh * kKB * kRowB;
  const char* vs = vtiles + kh * kKB * kRowB;
  const int krow = key_perm(lane & 31);
  uint4 kv[2], vv[2];
  auto step_load = [&](int sb) SMOE_INL {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * kFwdThreads;
      const int64_t g = int64_t(sb) + (i >> 4);
      const bool ok = g < T;
      kv[u] = ok ? *reinterpret_cast<const uint4*>(kk + g * kHD + (i & 15) * 8) : make_uint4(0u, 0u, 0u, 0u);
      vv[u] = ok ? *reinterpret_cast<const uint4*>(v + g * kHD + (i & 15) * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  step_load(blo / kKB * kKB);
  for (int sb0 = blo / kKB * kKB; sb0 <= bhi; sb0 += kStepKeys) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * kFwdThreads;
      const int row = i >> 4, c = i & 15, tr = row & 31;
      *reinterpret_cast<uint4*>(ktiles + row * kRowB + ((c ^ swz_tr(tr)) << 4)) = kv[u];
      *reinterpret_cast<uint4*>(vtiles + row * kRowB + ((c ^ swz_row(tr)) << 4)) = vv[u];
    }
    __syncthreads();
    if (sb0 + kStepKeys <= bhi) step_load(sb0 + kStepKeys);
    const int kb0 = sb0 + kKB * kh;
    if (kb0 > whi || kb0 + kKB <= wlo) continue;   // nothing for this wave (uniform)
    at_f32x16_t sc, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<true>(ks, krow, s, h), qf[s], sc, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<false>(vs, krow, s, h), df[s], dp, 0, 0, 0);
    }
    float ds[16];
    if (kb0 >= wlo_max && kb0 + kKB - 1 <= whi_min) {   // inside every row's range (uniform)
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = __builtin_amdgcn_exp2f(sc[i] * sl2 - lse2) * (dp[i] - Dr);
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb0 + key_perm(8 * q4 + 4 * h + i);
          const bool ok = key >= lo && key <= t;
          const float p = ok ? __builtin_amdgcn_exp2f(sc[4 * q4 + i] * sl2 - lse2) : 0.f;
          ds[4 * q4 + i] = p * (dp[4 * q4 + i] - Dr);
        }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      at_bf16x8_t ah, al;
      acc_frags(ds, s, ah, al);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const at_bf16x8_t kf = tr_frag(ks, 32 * nt, s, lane);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, ah, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, al, acc[nt], 0, 0, 0);
      }
    }
  }
  // the second key half adds its partial to the first
  __syncthreads();
  float4* slots = reinterpret_cast<float4*>(smem) + rt * 16 * kWave;
  if (kh == 1) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        slots[(4 * nt + q4) * kWave + lane] =
            make_float4(acc[nt][4 * q4], acc[nt][4 * q4 + 1], acc[nt][4 * q4 + 2], acc[nt][4 * q4 + 3]);
  }
  __syncthreads();
  if (kh == 1 || !real) return;
  const float scale = 1.f / sqrtf(float(kHD));
  uint16_t* out = dq + r * kHD;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x = slots[(4 * nt + q4) * kWave + lane];
      const float vals[4] = {(acc[nt][4 * q4] + x.x) * scale, (acc[nt][4 * q4 + 1] + x.y) * scale,
                             (acc[nt][4 * q4 + 2] + x.z) * scale, (acc[nt][4 * q4 + 3] + x.w) * scale};
      *reinterpret_cast<uint2*>(out + 32 * nt + 8 * q4 + 4 * h) = pack4_bf16(vals);
    }
}

// dK, dV: block (128 keys, query split q) of 8 waves, wave w = (key tile
// w & 3, head-dim half w >> 2); lane: key lane & 31 of its tile, its K and V
// rows in registers.  The block walks the query tiles q, q + QS, ... whose
// key range meets its keys, each tile's q and do rows shared through LDS
// (the next relevant tile loading into registers meanwhile).  Transposed
// scores (queries in the pi order) and dp^T give p^T and dz^T in the A
// operand layout of p^T do and dz^T q; each wave forms the columns of its
// head-dim half.  Partial sums per split, fp32: part[q][key][128].
constexpr int kDkvThreads = 512;
__global__ __launch_bounds__(kDkvThreads) void attn_dkv_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kk,
                                                               const uint16_t* __restrict__ v,
                                                               const int* __restrict__ sidx, int64_t M, int64_t T,
                                                               int ktop, int64_t S, const float* __restrict__ lse,
                                                               const float* __restrict__ D,
                                                               const uint16_t* __restrict__ dout,
                                                               const int* __restrict__ tile_lo,
                                                               const int* __restrict__ tile_hi, int64_t ntiles,
                                                               int QS, float* __restrict__ pdk,
                                                               float* __restrict__ pdv) {
  __shared__ __attribute__((aligned(16))) char qs[32 * kRowB];
  __shared__ __attribute__((aligned(16))) char dos[32 * kRowB];
  __shared__ __attribute__((aligned(16))) char kall[kAttnRows * kRowB];   // the block's K rows
  __shared__ __attribute__((aligned(16))) char vall[kAttnRows * kRowB];   // and V rows
  __shared__ float4 xch[4][2][4 * kWave];   // per key tile: p (from half 0), dp (from half 1)
  __shared__ int q_lo[32], q_t[32];
  __shared__ float q_lse2[32], q_D[32];
  const int lane = lane_id(), h = lane >> 5;
  const int w = threadIdx.x / kWave;
  const int kt = w & 3, hh = w >> 2;
  const int64_t k0 = int64_t(blockIdx.x) * kAttnRows;
  const int64_t k1 = min(T, k0 + kAttnRows) - 1;
  const int64_t kw0 = k0 + 32 * kt;
  const int64_t key = kw0 + (lane & 31);
  const int split = blockIdx.y;
  const float l2e = 1.4426950408889634f;
  const float sl2 = l2e / sqrtf(float(kHD));
  // the block's 128 K and V rows, row-read layout (rows past T zero)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x + u * kDkvThreads;   // 0 .. 2047: 128 rows x 16 chunks
    const int row = i >> 4, c = i & 15;
    const int64_t g = k0 + row;
    const bool ok = g < T;
    const int pc = c ^ swz_row(row & 31);
    *reinterpret_cast<uint4*>(kall + row * kRowB + (pc << 4)) =
        ok ? *reinterpret_cast<const uint4*>(kk + g * kHD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(vall + row * kRowB + (pc << 4)) =
        ok ? *reinterpret_cast<const uint4*>(v + g * kHD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
  const char* kmine = kall + kt * 32 * kRowB;
  const char* vmine = vall + kt * 32 * kRowB;
  at_f32x16_t adk[2], adv[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) adk[n][i] = adv[n][i] = 0.f;

  // next query tile at or after i (step QS) whose range meets [k0, k1]
  auto next_tile = [&](int64_t i) -> int64_t {
    for (; i < ntiles; i += QS)
      if (tile_hi[i] >= k0 && tile_lo[i] <= k1) return i;
    return ntiles;
  };
  // a query tile's q and do rows: one 16-byte piece of each per thread
  uint4 qv, dv_;
  auto piece_load = [&](int64_t i) {
    const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
    const int64_t g = i * 32 + row;
    qv = g < M ? *reinterpret_cast<const uint4*>(q + g * kHD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    dv_ = g < M ? *reinterpret_cast<const uint4*>(dout + g * kHD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
  };
  // per-row values of a query tile, one row per thread 0..31
  int pr_lo = 0x7fffffff, pr_t = -1;
  float pr_lse2 = 0.f, pr_D = 0.f;
  auto row_load = [&](int64_t i) {
    if (threadIdx.x < 32) {
      const int64_t r = i * 32 + threadIdx.x;
      if (r < M) {
        pr_t = sidx[r] / ktop;
        pr_lo = int(int64_t(pr_t) / S * S);
        pr_lse2 = lse[r] * l2e;
        pr_D = D[r];
      } else {
        pr_t = -1;
        pr_lo = 0x7fffffff;
        pr_lse2 = 0.f;
        pr_D = 0.f;
      }
    }
  };
  int64_t i = next_tile(split);
  if (i < ntiles) {
    piece_load(i);
    row_load(i);
  }
  while (i < ntiles) {
    __syncthreads();
    {
      const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
      const int pc = c ^ swz_tr(row);
      *reinterpret_cast<uint4*>(qs + row * kRowB + (pc << 4)) = qv;
      *reinterpret_cast<uint4*>(dos + row * kRowB + (pc << 4)) = dv_;
    }
    if (threadIdx.x < 32) {
      q_lo[threadIdx.x] = pr_lo;
      q_t[threadIdx.x] = pr_t;
      q_lse2[threadIdx.x] = pr_lse2;
      q_D[threadIdx.x] = pr_D;
    }
    const int tlo = tile_lo[i], thi = tile_hi[i];
    const int tlo_max = tile_lo[ntiles + i], thi_min = tile_hi[ntiles + i];
    __syncthreads();
    const int64_t inext = next_tile(i + QS);
    if (inext < ntiles) {
      piece_load(inext);
      row_load(inext);
    }
    // half 0 forms p^T, half 1 dp^T; they swap them through LDS
    const bool active = !(thi < kw0 || tlo > kw0 + 31);   // uniform per key tile
    float pt[16], dz[16];
    if (active) {
      at_f32x16_t acc_;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc_[j] = 0.f;
      const int qrow = key_perm(lane & 31);
      const char* src = hh == 0 ? qs : dos;
      const char* mine = hh == 0 ? kmine : vmine;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<true>(src, qrow, s, h),
                                                       row_frag<false>(mine, lane & 31, s, h), acc_, 0, 0, 0);
      float mineval[16];
      if (hh == 0) {
        const bool inner = kw0 >= tlo_max && kw0 + 31 <= thi_min;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int qi = key_perm(8 * q4 + 4 * h + j);
            const bool ok = inner || (key >= q_lo[qi] && key <= q_t[qi]);
            mineval[4 * q4 + j] = ok ? __builtin_amdgcn_exp2f(acc_[4 * q4 + j] * sl2 - q_lse2[qi]) : 0.f;
          }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) mineval[j] = acc_[j];
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        xch[kt][hh][q4 * kWave + lane] =
            make_float4(mineval[4 * q4], mineval[4 * q4 + 1], mineval[4 * q4 + 2], mineval[4 * q4 + 3]);
#pragma unroll
      for (int j = 0; j < 16; ++j) pt[j] = mineval[j];
    }
    __syncthreads();
    if (active) {
      float other[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = xch[kt][1 - hh][q4 * kWave + lane];
        other[4 * q4] = x.x;
        other[4 * q4 + 1] = x.y;
        other[4 * q4 + 2] = x.z;
        other[4 * q4 + 3] = x.w;
      }
      // pt: p^T, dz = p (dp - D)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qi = key_perm(8 * q4 + 4 * h + j);
          const float p = hh == 0 ? pt[4 * q4 + j] : other[4 * q4 + j];
          const float dpv = hh == 0 ? other[4 * q4 + j] : pt[4 * q4 + j];
          pt[4 * q4 + j] = p;
          dz[4 * q4 + j] = p * (dpv - q_D[qi]);
        }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        at_bf16x8_t ph, pl, zh, zl;
        acc_frags(pt, s, ph, pl);
        acc_frags(dz, s, zh, zl);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int nt = 2 * hh + n;
          const at_bf16x8_t fo = tr_frag(dos, 32 * nt, s, lane);
          const at_bf16x8_t fq = tr_frag(qs, 32 * nt, s, lane);
          adv[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo, ph, adv[n], 0, 0, 0);
          adk[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq, zh, adk[n], 0, 0, 0);
          adv[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo, pl, adv[n], 0, 0, 0);
          adk[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq, zl, adk[n], 0, 0, 0);
        }
      }
    }
    i = inext;
  }
  if (key >= T) return;
  const float scale = 1.f / sqrtf(float(kHD));
  float* ok_ = pdk + (int64_t(split) * T + key) * kHD;
  float* ov_ = pdv + (int64_t(split) * T + key) * kHD;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c = 32 * (2 * hh + n) + 8 * q4 + 4 * h;
      *reinterpret_cast<float4*>(ok_ + c) = make_float4(adk[n][4 * q4] * scale, adk[n][4 * q4 + 1] * scale,
                                                        adk[n][4 * q4 + 2] * scale, adk[n][4 * q4 + 3] * scale);
      *reinterpret_cast<float4*>(ov_ + c) =
          make_float4(adv[n][4 * q4], adv[n][4 * q4 + 1], adv[n][4 * q4 + 2], adv[n][4 * q4 + 3]);
    }
}

// dK, dV [T][128] in bf16 from the QS partials, summed in split order
__global__ __launch_bounds__(kAttnThreads) void attn_dkv_reduce_kernel(const float* __restrict__ pdk,
                                                                       const float* __restrict__ pdv, int QS,
                                                                       int64_t n, uint16_t* __restrict__ dk,
                                                                       uint16_t* __restrict__ dv) {
  for (int64_t i = (int64_t(blockIdx.x) * kAttnThreads + threadIdx.x) * 4; i < n;
       i += int64_t(gridDim.x) * kAttnThreads * 4) {
    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < QS; ++sp) {
      const float4 x = *reinterpret_cast<const float4*>(pdk + int64_t(sp) * n + i);
      const float4 y = *reinterpret_cast<const float4*>(pdv + int64_t(sp) * n + i);
      a[0] += x.x; a[1] += x.y; a[2] += x.z; a[3] += x.w;
      b[0] += y.x; b[1] += y.y; b[2] += y.z; b[3] += y.w;
    }
    *reinterpret_cast<uint2*>(dk + i) = pack4_bf16(a);
    *reinterpret_cast<uint2*>(dv + i) = pack4_bf16(b);
  }
}

// query splits of the dK/dV pass: about 512 blocks in all, at most 16
int attn_query_splits(int64_t T) {
  const int64_t kb = (T + kAttnRows - 1) / kAttnRows;
  return int(std::min<int64_t>(16, std::max<int64_t>(1, (512 + kb - 1) / std::max<int64_t>(kb, 1))));
}

hipError_t launch_attn_bwd(const void* q, const void* kk, const void* v, const int* sidx, int64_t M, int64_t T,
                           int ktop, int64_t S, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, float* D, int* tile_lo, int* tile_hi, float* pdk, float* pdv, hipStream_t st,
                           hipEvent_t dq_start, hipEvent_t dq_stop, hipEvent_t dkv_start, hipEvent_t dkv_stop) {
  if (M == 0) return hipSuccess;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(kk);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  const uint16_t* dp = static_cast<const uint16_t*>(dout);
  const int64_t ntiles = (M + 31) / 32;
  hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3(unsigned((ntiles + 3) / 4)), dim3(kAttnThreads), 0, st,
                     static_cast<const uint16_t*>(o), dp, sidx, M, ktop, S, D, tile_lo, tile_hi, ntiles);
  if (dq_start) (void)hipEventRecord(dq_start, st);
  hipLaunchKernelGGL(attn_dq_kernel, dim3(unsigned((M + kFwdRows - 1) / kFwdRows)), dim3(kFwdThreads), 0, st, qp,
                     kp, vp, sidx, M, T, ktop, S, lse, D, dp, static_cast<uint16_t*>(dq));
  if (dq_stop) (void)hipEventRecord(dq_stop, st);
  const int QS = attn_query_splits(T);
  if (dkv_start) (void)hipEventRecord(dkv_start, st);
  hipLaunchKernelGGL(attn_dkv_kernel, dim3(unsigned((T + kAttnRows - 1) / kAttnRows), unsigned(QS)),
                     dim3(kDkvThreads), 0, st, qp, kp, vp, sidx, M, T, ktop, S, lse, D, dp, tile_lo, tile_hi, ntiles,
                     QS, pdk, pdv);
  if (dkv_stop) (void)hipEventRecord(dkv_stop, st);
  const int64_t n = T * kHD;
  hipLaunchKernelGGL(attn_dkv_reduce_kernel, dim3(unsigned(std::min<int64_t>((n / 4 + kAttnThreads - 1) / kAttnThreads, 4096))),
                     dim3(kAttnThreads), 0, st, pdk, pdv, QS, n, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
  return hipGetLastError();
}

}  // namespace smoe
