// Internal interface between the host orchestration (api.hip) and the
// gfx950 kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace smoe {

constexpr int kMaxExperts = 1024;

// Segmented grouped GEMM over scattered rows.
//
// SEG_M (rows mode, the scatter2scatter product and its dX):
//   for every grouped row r of expert e (offsets[e] <= r < offsets[e+1]):
//     C[r][n] = sum_{k<K} A(r,k) * B_e(k,n),   n < N
//   A(r,k) = (k < K0 ? a0 : a1)[arow(r) * lda + k (- K0)]
//            arow(r) = a_scat ? sidx[r] / a_fan : r
//   B_e(k,n): b_nk == 0: W[k][n] layout, (dual ? b0 for W1 / b1 for W3)
//                        b0 + e*b_es + k*ldb + n
//             b_nk == 1: W[n][k] layout (W^T product), concat along K:
//                        (k < K0 ? b0 : b1) + e*b_es + n*ldb + k (- K0)
// SEG_K (weights mode, groupXtY):
//   for every expert e, row chunk [r0, r1) of its grouped rows (chunks of
//   KS rows):  C_e[i][j] += sum_{r in chunk} A(r,i) * B(r,j),  i < Mo, j < N
//   A(r,i) = a0[arow(r) * lda + i],  B(r,j) = b0[brow(r) * ldb + j]
//   brow(r) = b_scat ? sidx[r] / b_fan : r
//   An expert with one chunk writes c0 + e*Mo*N directly (unless
//   dw_all_partial); otherwise each chunk writes partial + chunk*Mo*N and
//   reduce_dw() sums them.
enum Mode { SEG_M = 0, SEG_K = 1 };

// Epilogues (SEG_M).  v is the fp32 product; "stored" means rounded to the
// storage type of the outputs (bf16 or fp32).
enum Epi {
  EPI_STORE = 0,   // c0[crow(r)][n] = (gate ? g*v : v); dg partial <aux row, v>
  EPI_GELU_FWD,    // h = stored(v) -> c0; a = stored(gelu(h)) -> c1
  EPI_SWIGLU_FWD,  // h1 = stored(v1) -> c0; h3 = stored(v3) -> c1; a = stored(silu(h1) h3) -> c2
  EPI_GELU_BWD,    // v = dA/g; h = aux0; a = stored(gelu(h)); dg += <a, v>;
                   // c0 = stored(g v gelu'(h)); c2 = stored(g a)
  EPI_SWIGLU_BWD,  // v = dA/g; h1,h3 = aux0,aux1; a = stored(silu(h1) h3); dg += <a, v>;
                   // c0 = stored(g v h3 silu'(h1)); c1 = stored(g v silu(h1)); c2 = stored(g a)
  EPI_PARTIAL,     // SEG_K fp32 tile store
  EPI_PARTIAL_GATED  // SEG_K fp32 tile store, A(r,i) scaled by kscale[r] first (bf16: the
                     // scaled value rounded to bf16 before it enters the contraction)
};

struct GemmArgs {
  const int* offsets;  // [E+1]
  const int* sidx;     // sorted_scattered_idxs [M]
  int E;
  int M;    // T*k: grouped-row count upper bound, stride of dg partials
  int N;    // output columns
  int K;    // SEG_M reduction length (with concat)
  int K0;   // SEG_M concat split (== K when single)
  int Mo;   // SEG_K output rows
  int KS;   // SEG_K rows per chunk
  int mt_ub;   // SEG_M: upper bound on m-tiles; SEG_K: upper bound on chunks
  int g_base;  // SEG_M: index of this launch's first tile (a launch may cover a range)
  int g_count; // SEG_M: tiles in this launch (0: all from g_base on)
  int b_nk;
  const void* a0;
  const void* a1;
  int64_t lda;
  int64_t a_rows;      // rows of the A tensor(s) (bounds of the buffer loads)
  int a_scat, a_fan;
  const void* b0;
  const void* b1;
  int64_t ldb, b_es;
  int64_t b_rows;      // SEG_K: rows of the B tensor (bounds of the buffer loads)
  int b_scat, b_fan;
  void* c0;
  void* c1;
  void* c2;
  int64_t ldc;
  int c_scat;
  int c_add_fan;       // SEG_M EPI_STORE, fp32 out: 0 stores row crow; f > 0 adds
                       // (atomically) into row crow / f (the combine fused in)
  const float* gate;   // SEG_M epilogue gate, indexed by p = sidx[r]
  const void* aux0;    // SEG_M epilogue loads
  const void* aux1;
  int64_t ldaux;
  int aux_scat, aux_fan;
  float* dgpart;       // [slots][M]
  float* partial;      // SEG_K partial tiles [mt_ub][Mo*N]
  int dw_all_partial;  // SEG_K: every chunk writes its partial (reduce_dw writes dw)
  const float* kscale; // SEG_K EPI_PARTIAL_GATED: per grouped row scale of A
  // x / fan == (x * fan_m) >> fan_s for 0 <= x < 2^31 (set by plan_gemm)
  uint32_t a_fan_m, b_fan_m;
  int a_fan_s, b_fan_s;
};

// Multiply-shift constants for exact division by d (1 <= d < 2^16) of
// non-negative 31-bit integers: l = ceil(log2 d), m = ceil(2^(31+l) / d).
inline void fastdiv_magic(int d, uint32_t& m, int& s) {
  int l = 0;
  while ((1 << l) < d) ++l;
  const uint64_t num = uint64_t(1) << (31 + l);
  m = uint32_t((num + uint64_t(d) - 1) / uint64_t(d));
  s = 31 + l;
}

// Launch descriptions chosen on the host.
struct GemmPlan {
  int mode;
  int epi;
  int dual;      // SwiGLU dual B (W1 and W3 share the A tile)
  int bf16;      // 1: MFMA bf16 kernel; 0: fp32 kernel
  int bm, bn;    // tile (bf16 kernel: 128 or 256 each)
  int nw;        // bf16 kernel: waves per workgroup (8, or 4 for 256 x 256 rows-mode tiles)
  int slots;     // dg partial slots written per row
  int n_tiles;   // tiles along N (SEG_M) or tiles per chunk (SEG_K)
  int out_f32;   // SEG_M EPI_STORE: c0 is fp32 (else the storage type)
  int64_t grid;  // workgroups launched
};

// Chooses tiles, sizes the grid and fills plan; returns false if no kernel
// instance exists for the request.
bool plan_gemm(GemmArgs& a, GemmPlan& plan, int mode, int epi, int dual, int bf16, int out_f32);
// SEG_M, bf16: the number of leading tiles that are certainly real (whatever
// the per-expert row counts) and fill whole rounds of the chip; 0 if none.
int64_t whole_round_tiles(const GemmArgs& a, const GemmPlan& plan);

// Router (gate.hip): top-k softmax gates from logits = x w^T (w [E][d]);
// the backward's pieces: the router's dx (written or added) from the
// per-choice dlogits, which it also leaves as a dense D [T][ncol] for the dw
// product together with that product's identity row index and single-group
// offsets {0, T}; and dw [E][d] from the product's [d][ncol] result.
hipError_t launch_gate_fwd(const void* x, const void* wg, int64_t T, int d, int E, int k, int bf16, int* idx,
                           float* gates, float* logits, hipStream_t st);
void gate_dlogit_cols(int E, int bf16, int& ep, int& ncol);
hipError_t launch_gate_dx(const void* wg, int64_t T, int d, int E, int k, int bf16, const int* idx,
                          const float* gates, const float* dgates, void* dx, int accumulate, void* D, int* rows,
                          int* offsets, hipStream_t st);
hipError_t launch_gate_dw_finish(const float* tmp, int d, int E, int bf16, float* dw, hipStream_t st);

// Mixture-of-Attention core (attn.hip), bf16, head_dim 128: o and lse of
// grouped query rows against shared K/V, causal within sequences of S.
hipError_t launch_attn_fwd(const void* q, const void* kk, const void* v, const int* sidx, int64_t M, int64_t T,
                           int ktop, int64_t S, void* o, float* lse, hipStream_t st);
// backward: D [M], per-32-row query tile ranges [ceil(M/32)] x 4, and fp32
// dK/dV partials [attn_query_splits(T)][T][128] each
int attn_query_splits(int64_t T);
hipError_t launch_attn_bwd(const void* q, const void* kk, const void* v, const int* sidx, int64_t M, int64_t T,
                           int ktop, int64_t S, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, float* D, int* tile_lo, int* tile_hi, float* pdk, float* pdv, hipStream_t st,
                           hipEvent_t dq_start, hipEvent_t dq_stop, hipEvent_t dkv_start, hipEvent_t dkv_stop);

// Matrix-core rate probe (probe.hip): blocks x 256 threads, each wave
// iters rounds of 16 bf16 32x32x16 multiplies on registers.
hipError_t launch_mfma_loop(float* out, int blocks, int iters, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& plan, hipStream_t st);

// routing
size_t route_ws_bytes(int64_t M, int E);
// device address (this device) and size in ints of the routing kernels'
// static scratch, for the allocation-free entry point
hipError_t route_static_scratch(int** ptr, size_t* ints);
size_t route_static_scratch_ints();
hipError_t launch_route(const int* eidx, int M, int E, int* s_exp, int* s_sct, int* counts, int* offsets,
                        void* ws, hipStream_t st);

// elementwise / reductions
// out[t][c] = sum_j w(t,j) * pairs[t*k + j][c]; w = gates or 1.  pairs fp32.
hipError_t launch_combine(const float* pairs, const float* gates, int64_t T, int k, int64_t d, void* out,
                          int out_bf16, hipStream_t st);
// dg[sidx[r]] = sum_s part[s*M + r] for r < offsets[E]
hipError_t launch_reduce_dg(const float* part, int slots, int M, const int* offsets, int E, const int* sidx,
                            float* dg, hipStream_t st);
// expert e with 0 chunks: dw[e] = 0; with >= 2 chunks (every expert if
// all_partial): dw[e] = sum of its partials, in chunk order; accumulate adds
// the sum to what dw holds; dw is fp32 or (out_bf16) bf16, rounded once
hipError_t launch_reduce_dw(const float* partial, const int* offsets, int E, int KS, int64_t elems, void* dw,
                            int all_partial, int accumulate, int out_bf16, hipStream_t st);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);
// gg[r] = gates[sidx[r]] for grouped rows r < offsets[E], 0 for r < M past
// them: the gates in grouped order (one float per assignment)
hipError_t launch_grouped_gates(const float* gates, const int* sidx, const int* offsets, int E, int M, float* gg,
                                hipStream_t st);

}  // namespace smoe
