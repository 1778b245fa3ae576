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
//  - 512 threads = 8 waves, two per SIMD, in a 2 (M) x 4 (N) grid over a
//    BM x BN tile (128 or 256 each), K step 64.  Each wave owns
//    (BM/2) x (BN/4) as 32x32 fragments of v_mfma_f32_32x32x16_bf16 with
//    fp32 accumulators; the second wave on a SIMD keeps the matrix core busy
//    while the first waits on LDS, copies or the barrier.
//  - Every operand moves global -> LDS with buffer loads that write LDS
//    directly (no register staging); out-of-range offsets read as zero,
//    which pads ragged rows, columns and K without branches.  Two LDS stages.
//  - An operand whose K axis is contiguous in memory (gathered token rows,
//    W[e] read as W^T) is stored [row][64 k] (128-byte rows) and fragments
//    are 128-bit LDS reads.  An operand whose K axis is strided (W[e] in the
//    forward, both operands of the weight gradient) is stored [64 k][mn] as
//    it sits in memory and fragments come from gfx950's transposing LDS read
//    (ds_read_b64_tr_b16), which hands each lane four consecutive k of one
//    mn: no transpose is ever done in registers.
//  - Both layouts XOR-swizzle 16-byte chunks per row so that the 16 lanes
//    served together by the 64-bank LDS hit distinct banks.
//  - The MFMA is issued with the B fragment first, so each lane ends up
//    holding one output row and runs of 4 consecutive columns: epilogue
//    stores are 8 bytes (bf16) or 16 bytes (fp32) wide.
//  - Workgroups are renumbered so that each XCD (blockIdx % 8 on MI355X)
//    receives an equal, contiguous run of the tiles that exist (counted on
//    the device from the expert row counts), ordered in groups of 8 m-tiles
//    sweeping n, so concurrent tiles on one XCD share A rows and weight
//    panels in that XCD's L2 and no XCD idles on the grid's empty tail.
//
// fp32 kernel: the same contract with plain FMA on 64x64 tiles, used for
// fp32 runs (a small, launch-bound regime).
#include "common.h"
#include "kernels.h"

namespace smoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kThreads = 512;   // bf16 kernel
#ifndef SMOE_BK
#define SMOE_BK 32
#endif
#ifndef SMOE_NS
#define SMOE_NS 4
#endif
#ifndef SMOE_SCHED
#define SMOE_SCHED 0
#endif
constexpr int kBK = SMOE_BK;    // K of one pipeline stage (32 or 64)
constexpr int kNS = SMOE_NS;    // LDS stages in flight
static_assert(kBK == 32 || kBK == 64, "K step");
static_assert(kNS >= 2, "stages");
constexpr uint32_t kOOB = 0xFFFFFFF0u;  // byte offset past every buffer: reads as 0

enum Lay { LAY_K = 0, LAY_MN = 1 };

SMOE_DEV int fdiv(int x, uint32_t m, int s) { return int((uint64_t(uint32_t(x)) * m) >> s); }

// K-layout tile: row j (one gathered token row, or one column of W read as
// W^T) holds the stage's kBK values of k, KC 16-byte chunks.  Chunk c of row
// j sits at chunk c ^ swz_k(j).  A 128-bit LDS read serves 16 lanes at a
// time, i.e. 16 consecutive rows at one logical chunk; the 64 banks cover
// 256 bytes = 2 rows of 128 bytes (kBK = 64) or 4 rows of 64 bytes (kBK =
// 32), and the swizzle gives the rows that share banks distinct chunks.
struct KGeom {
  static constexpr int RB = 2 * kBK;    // bytes per row
  static constexpr int KC = kBK / 8;    // 16-byte chunks per row
  static constexpr int RPL = 64 / KC;   // rows per wave copy
};
SMOE_DEV int swz_k(int row) {
  if constexpr (kBK == 64) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
// MN-layout: chunk c (8 mn) of k-row r is stored at chunk c ^ swz_mn(r).  A
// 64-bit LDS read is served 32 lanes at a time; for a transposing fragment
// read those 32 lanes take four aligned chunks from each of four consecutive
// k-rows, and the masks 0, 4, 8, 12 put the sixteen chunks on distinct banks.
SMOE_DEV int swz_mn(int krow) { return (krow & 3) << 2; }

// Buffer descriptor over [base, base + bytes) (raw buffer, no stride,
// out-of-range offsets read zero).  Base and size are the same on every
// lane; reading them through readfirstlane keeps the descriptor in scalar
// registers, as the buffer instructions require.
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));
SMOE_DEV rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const int64_t n = bytes < int64_t(kOOB) ? bytes : int64_t(kOOB);
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane(uint32_t(b));
  r.y = __builtin_amdgcn_readfirstlane(uint32_t(b >> 32) & 0xFFFFu);
  r.z = __builtin_amdgcn_readfirstlane(uint32_t(n));
  r.w = 0x00020000u;
  return r;
}
// The 64 lanes of the wave each copy 16 bytes (at byte offset voff of the
// buffer) to wave_lds + 16 * lane, straight into LDS.  Written as inline asm
// so that the compiler does not order later LDS reads of OTHER stages behind
// these copies (it cannot tell the stages apart); the kernel waits for the
// copies itself (wait_vmem) before the barrier that publishes a stage.  The
// asm has no register outputs; its inputs are read when it issues.
// The LDS address is the low 32 bits of the flat address of wave_lds (the
// LDS aperture starts at a multiple of 4 GiB).
SMOE_DEV uint32_t lds_addr(const char* p) { return uint32_t(reinterpret_cast<uintptr_t>(p)); }
SMOE_DEV void dma16(rsrc_t r, char* wave_lds, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(wave_lds));
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(m0v)
               : "memory", "m0");
}
// the same at byte offset voff + soff: soff is the wave-uniform part (the
// step's advance along k), so a copy inside the buffer needs no vector
// arithmetic per step.  Only used where voff + soff stays in range.
SMOE_DEV void dma16s(rsrc_t r, char* wave_lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(wave_lds));
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(r), "s"(m0v), "s"(soff)
               : "memory", "m0");
}
// the same with 4 bytes per lane (64 consecutive dwords)
SMOE_DEV void dma4(rsrc_t r, char* wave_lds, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(wave_lds));
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(m0v)
               : "memory", "m0");
}
// wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order): s_waitcnt vmcnt(N), other counters free
template <int N>
SMOE_DEV void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

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
  // The grid is sized for an upper bound on the tiles; how many exist
  // depends on the per-expert row counts and is counted here.  Blocks are
  // dealt to the XCDs round-robin (block b runs on XCD b % 8): each XCD
  // takes a contiguous run of this launch's real tiles, the runs as even as
  // the count divides, and the blocks past a run have no tile.  (Runs over
  // the upper-bound range would leave the last XCDs with the empty tail:
  // with 8 experts and 2 split-K chunks' room, 2 of 10 chunks are empty.)
  constexpr int kXcd = 8;
  constexpr int GM = 8;
  constexpr int NCOLS = DUAL ? BN / 2 : BN;
  int n_real, units = 0;
  const int ntn = (p.N + NCOLS - 1) / NCOLS;
  const int ti = (p.Mo + BM - 1) / BM, tj = (p.N + BN - 1) / BN, tpc = ti * tj;
  if constexpr (MODE == SEG_M) {
    units = total_items(p.offsets, p.E, BM);   // real m-tiles
    n_real = units * ntn;
  } else {
    n_real = total_items(p.offsets, p.E, p.KS) * tpc;
  }
  const int lo = MODE == SEG_M ? p.g_base : 0;
  const int hi = (MODE == SEG_M && p.g_count > 0) ? min(n_real, lo + p.g_count) : n_real;
  if (hi <= lo) return false;
  const int per = (hi - lo + kXcd - 1) / kXcd;
  const int j = int(blockIdx.x) / kXcd;
  if (j >= per) return false;
  const int g = lo + (int(blockIdx.x) % kXcd) * per + j;
  if (g >= hi) return false;
  if constexpr (MODE == SEG_M) {
    // groups of GM m-tiles sweeping the n-tiles: concurrent tiles on an XCD
    // share GM A panels and a few weight panels
    const int group = g / (GM * ntn);
    const int gs = min(GM, units - group * GM);
    const int local = g - group * GM * ntn;
    const int mt = group * GM + local % gs;
    t.nt = local / gs;
    t.n0 = t.nt * NCOLS;
    t.m0 = 0;
    t.chunk = 0;
    return find_item(p.offsets, p.E, BM, mt, t.it);
  } else {
    t.chunk = g / tpc;
    const int rem = g - t.chunk * tpc;
    // groups of 8 output row blocks sweeping the column blocks, as in rows
    // mode: concurrent tiles on an XCD then share 8 A panels and a few B
    // panels instead of one A panel and 32 distinct B panels
    const int group = rem / (GM * tj);
    const int gs = min(GM, ti - group * GM);
    const int local = rem - group * GM * tj;
    t.m0 = (group * GM + local % gs) * BM;
    t.n0 = (local / gs) * BN;
    t.nt = 0;
    return find_item(p.offsets, p.E, p.KS, t.chunk, t.it);
  }
}

// ---------------------------------------------------------------------------
// Operand tiles in LDS, one stage = kBK values of k.
//
// K-layout tile of R rows: row j at j*RB bytes.  The copy of one stage is
// R*kBK/4096 buffer loads per wave; load t of wave w fills rows
// (8t + w)*RPL .. +RPL, lane L taking row +(L / KC) and storing physical
// chunk L % KC, i.e. the logical chunk (L % KC) ^ swz_k(row) of that row.
//
// MN-layout tile of R mn (R = 128 or 256) by kBK k: k-row r at r*2R bytes,
// CPR = R/8 chunks per k-row, RPI = 64/CPR k-rows per wave load; load t of
// wave w fills k-rows (8t + w)*RPI .. +RPI, lane L taking k-row +(L / CPR)
// and physical chunk L % CPR (logical chunk (L % CPR) ^ swz_mn(k-row)).
// ---------------------------------------------------------------------------
template <int R>
struct MnGeom {
  static constexpr int RB = 2 * R;         // bytes per k-row
  static constexpr int CPR = R / 8;        // 16-byte chunks per k-row
  static constexpr int RPI = 64 / CPR;     // k-rows per wave load
  static constexpr int NI = R * kBK / 4096;  // loads per wave per stage
  static_assert(NI >= 1, "tile too small for one copy per wave");
};

// lane's k-row and logical chunk in MN-layout load t of wave `wave`
template <int R>
SMOE_DEV void mn_slot(int t, int wave, int lane, int& krow, int& chunk) {
  using G = MnGeom<R>;
  krow = (t * 8 + wave) * G::RPI + lane / G::CPR;
  chunk = (lane % G::CPR) ^ swz_mn(krow);
}

// 32x32x16 MFMA operand (lane: row lane&31, k = 16s + 8*(lane>>5) + 0..7)
// from a K-layout tile
SMOE_DEV bf16x8_t frag_k(const char* tile, int row0, int s, int lane) {
  const int row = row0 + (lane & 31);
  const int c = (2 * s + (lane >> 5)) ^ swz_k(row);
  return *reinterpret_cast<const bf16x8_t*>(tile + row * KGeom::RB + (c << 4));
}

// the same operand from an MN-layout tile, through two transposing reads:
// within each 16-lane group, lane i receives element i & 3 of the 8-byte
// pieces addressed by lanes (i >> 2) + 4j, j = 0..3; lane i therefore
// addresses k-row kb + (i >> 2), columns mb + 4*(i & 3) .. +3, and gets
// column mb + i at k-rows kb .. kb+3.
template <int R>
SMOE_DEV bf16x8_t frag_mn(const char* tile, int m0, int s, int lane) {
  using G = MnGeom<R>;
  const int grp = lane >> 4, i = lane & 15;
  const int mn = m0 + 16 * (grp & 1) + 4 * (i & 3);
  const int kr = 16 * s + 8 * (grp >> 1) + (i >> 2);
  const int c = mn >> 3, within = (mn & 7) * 2;
  const char* p0 = tile + kr * G::RB + ((c ^ swz_mn(kr)) << 4) + within;
  const char* p1 = tile + (kr + 4) * G::RB + ((c ^ swz_mn(kr + 4)) << 4) + within;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(const lds_void_t*)p0);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(const lds_void_t*)p1);
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int BM, int BN, int MODE, int EPI, int BLAY, bool DUAL, class OutT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int ALAY = MODE == SEG_M ? LAY_K : LAY_MN;
  constexpr int FM = BM / 64, FN = BN / 128;   // fragments per wave
  constexpr int WM = BM / 2, WN = BN / 4;      // wave tile
  constexpr int A_BYTES = BM * kBK * 2, B_BYTES = BN * kBK * 2, STAGE = A_BYTES + B_BYTES;
  static_assert(BN >= 128 && BM >= 128, "tile");
  static_assert(!DUAL || (MODE == SEG_M && BLAY == LAY_MN && BN == 256), "dual B layout");
  // one LDS object per stage, always named statically (the loop below is
  // unrolled by kNS): the compiler can then tell a stage being read from the
  // stages whose copies are still in flight
  __shared__ __attribute__((aligned(16))) char smem0[STAGE];
  __shared__ __attribute__((aligned(16))) char smem1[STAGE];
  __shared__ __attribute__((aligned(16))) char smem2[kNS > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) char smem3[kNS > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) char smem4[kNS > 4 ? STAGE : 16];
  static_assert(kNS <= 5, "stages");
  auto stage = [&](auto s) SMOE_INL -> char* {
    constexpr int S = decltype(s)::value % kNS;
    if constexpr (S == 0) return smem0;
    else if constexpr (S == 1) return smem1;
    else if constexpr (S == 2) return smem2;
    else if constexpr (S == 3) return smem3;
    else return smem4;
  };

  TileInfo T;
  if (!tile_of_block<BM, BN, MODE, DUAL>(p, T)) return;
  const Item& it = T.it;

  // wave index as a scalar: everything derived from it (LDS copy targets,
  // per-wave roles) stays wave-uniform for the compiler
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // ---------------- K steps ------------------------------------------------
  // SEG_M: K is [part 0: K0 columns of a0 / b0 | part 1: K-K0 of a1 / b1];
  // each kBK-wide step lies inside one part.  SEG_K: the chunk's rows.
  const int K0 = MODE == SEG_M ? p.K0 : it.row1 - it.row0;
  const int K1 = MODE == SEG_M ? p.K - p.K0 : 0;
  const int KT0 = (K0 + kBK - 1) / kBK;
  const int KT = KT0 + (K1 + kBK - 1) / kBK;

  // ---------------- per-lane copy addressing -------------------------------
  constexpr int NA = BM * kBK / 4096, NB = BN * kBK / 4096;   // buffer loads per wave per operand
  constexpr int LPS = NA + NB;                                // per stage
  static_assert(NA >= 1 && NB >= 1 && (!DUAL || NB % 2 == 0), "copy split");
  using GA = MnGeom<BM>;
  using GB = MnGeom<BN>;
  // buffer descriptors of the operands (part 0 / part 1 of K; dual: W1 / W3),
  // built from kernel arguments at each use
  auto descA = [&](auto part) SMOE_INL {
    const void* base;
    if constexpr (decltype(part)::value) base = p.a1;
    else base = p.a0;
    return make_rsrc(base, p.a_rows * p.lda * 2);
  };
  auto descB = [&](auto part) SMOE_INL {
    const uint16_t* base;
    if constexpr (decltype(part)::value) base = static_cast<const uint16_t*>(p.b1);
    else base = static_cast<const uint16_t*>(p.b0);
    int64_t bytes;
    if constexpr (MODE == SEG_K) {
      bytes = p.b_rows * p.ldb * 2;
    } else {
      base += int64_t(it.e) * p.b_es;
      bytes = int64_t(BLAY == LAY_K ? p.N : p.K0) * p.ldb * 2;
    }
    return make_rsrc(base, bytes);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // row pitches in bytes (every operand is under 4 GiB)
  const uint32_t lda2 = uint32_t(p.lda * 2), ldb2 = uint32_t(p.ldb * 2);
  // SEG_K: all-ones when the operand's rows are gathered (a mask rather
  // than a condition, so that the copies carry no branch)
  const int scat_a = -int(p.a_scat != 0), scat_b = -int(p.b_scat != 0);
  // Per copy and lane, the byte offset of the lane's 16 bytes at k = 0 of
  // the part (SEG_M) or chunk (SEG_K), and the lane's k within a step (ka,
  // kb: k offset of its chunk for K-layout, k-row for MN-layout).  A full
  // step then advances every copy by one wave-uniform scalar offset.  Rows
  // and columns outside the tile's valid range read other (in-range) data:
  // their products land only in outputs that are never stored.  Only k
  // beyond the end of the reduction must read zero, on both operands; the
  // step that crosses it takes a per-lane path.
  uint32_t a_off[NA], b_off[NB];
  int ka[NA], kb_[NB];
  // SEG_K: column byte offset of the lane (a_col / b_col) for gathered rows
  uint32_t a_col[MODE == SEG_K ? NA : 1], b_col[MODE == SEG_K ? NB : 1];

  if constexpr (MODE == SEG_M) {
    static_for<NA>([&](auto t) SMOE_INL {
      const int row = (int(t) * 8 + wave) * KGeom::RPL + lane / KGeom::KC;
      const int gr = it.row0 + row;
      const int src = gr < it.row1 ? (p.a_scat ? p.sidx[gr] / p.a_fan : gr) : -1;
      ka[t] = ((lane % KGeom::KC) ^ swz_k(row)) * 8;
      a_off[t] = (src >= 0 ? uint32_t(int64_t(src) * p.lda * 2) : 0u) + uint32_t(ka[t]) * 2;
    });
    if constexpr (BLAY == LAY_K) {
      // W[e] viewed [n][k]: N rows of ldb
      static_for<NB>([&](auto t) SMOE_INL {
        const int row = (int(t) * 8 + wave) * KGeom::RPL + lane / KGeom::KC;
        const int n = T.n0 + row;
        kb_[t] = ((lane % KGeom::KC) ^ swz_k(row)) * 8;
        b_off[t] = (n < p.N ? uint32_t(int64_t(n) * p.ldb * 2) : 0u) + uint32_t(kb_[t]) * 2;
      });
    } else {
      // W[e] viewed [k][n]: K rows of ldb.  Dual: the tile is two BN/2-column
      // sub-tiles, W1 columns then W3 columns (loads t < NB/2 fill the first)
      static_for<NB>([&](auto t) SMOE_INL {
        int krow, c;
        if constexpr (DUAL) mn_slot<BN / 2>(int(t) % (NB / 2), wave, lane, krow, c);
        else mn_slot<BN>(int(t), wave, lane, krow, c);
        const int col = T.n0 + 8 * c;
        kb_[t] = krow;
        b_off[t] = uint32_t(krow) * ldb2 + uint32_t(col) * 2;
      });
    }
  } else {
    static_for<NA>([&](auto t) SMOE_INL {
      int krow, c;
      mn_slot<BM>(int(t), wave, lane, krow, c);
      a_col[t] = uint32_t(T.m0 + 8 * c) * 2;
      ka[t] = (int(t) * 8 + wave) * GA::RPI + lane / GA::CPR;   // row within the step
      a_off[t] = uint32_t(ka[t]) * lda2 + a_col[t];
    });
    static_for<NB>([&](auto t) SMOE_INL {
      int krow, c;
      mn_slot<BN>(int(t), wave, lane, krow, c);
      b_col[t] = uint32_t(T.n0 + 8 * c) * 2;
      kb_[t] = (int(t) * 8 + wave) * GB::RPI + lane / GB::CPR;
      b_off[t] = uint32_t(kb_[t]) * ldb2 + b_col[t];
    });
  }
  // descriptors, built once
  const rsrc_t rA0 = descA(std::integral_constant<int, 0>{});
  const rsrc_t rA1 = descA(std::integral_constant<int, 1>{});
  const rsrc_t rB0 = descB(std::integral_constant<int, 0>{});
  const rsrc_t rB1 = descB(std::integral_constant<int, 1>{});

  // SEG_K: the source rows of the gathered operand come from
  // sorted_scattered_idxs.  The indices of the 32 grouped rows of step j are
  // copied into an LDS ring (slot j % kRing, 64 dwords: every wave copies the
  // same 64 indices, so each wave's count of copies per step is the same) in
  // step j-5, ahead of the copies of stage j-2; the stage waits therefore
  // also cover them, and the barrier of step j-3 publishes them before step
  // j-3 issues stage j.  The indices are read back with LDS reads, which keep
  // the LDS counter in order (no scalar loads in the loop).
  constexpr int kRing = 8, kIdxAhead = kNS + 1;
  constexpr int IDX = MODE == SEG_K ? 1 : 0;   // index copies per step
  __shared__ __attribute__((aligned(16))) int ring[MODE == SEG_K ? kRing * 64 : 1];
  auto idx_copy = [&](int j) SMOE_INL {
    if constexpr (MODE == SEG_K) {
      const uint32_t r = uint32_t(it.row0 + j * kBK + lane);
      dma4(make_rsrc(p.sidx, int64_t(p.M) * 4), reinterpret_cast<char*>(ring + (j % kRing) * 64), r * 4u);
    }
  };
  // the lane's raw indices for the copies of step j, read into registers
  // right after the barrier that published them, ahead of the fragment reads
  constexpr int SA = MODE == SEG_K ? NA : 1, SB = MODE == SEG_K ? NB : 1;
  int gia[SA], gib[SB];
  auto idx_fetch = [&](int j) SMOE_INL {
    if constexpr (MODE == SEG_K) {
      // read for both operands, gathered or not (no branch: the copies
      // select the index or the plain row)
      const int* slot = ring + (j % kRing) * 64;
      static_for<NA>([&](auto t) SMOE_INL { gia[t] = slot[(int(t) * 8 + wave) * GA::RPI + lane / GA::CPR]; });
      static_for<NB>([&](auto t) SMOE_INL { gib[t] = slot[(int(t) * 8 + wave) * GB::RPI + lane / GB::CPR]; });
    }
  };

  // ---------------- copy step kt into stage `stg` -------------------------
  // SEG_M: a uniform branch on the K part picks the buffer descriptors.  A
  // step inside the reduction advances every copy by one scalar offset; the
  // step that crosses its end (a uniform branch, at most one per part)
  // zero-fills the lanes past it.
  auto issue_part = [&](auto part, int kl, char* stg) SMOE_INL {
    constexpr int P = decltype(part)::value;
    char* As = stg;
    char* Bs = stg + A_BYTES;
    const int Kp = P ? K1 : K0;
    const rsrc_t& rA = P ? rA1 : rA0;
    const rsrc_t& rB = P ? rB1 : rB0;
    auto copies = [&](auto full) SMOE_INL {
      constexpr bool F = decltype(full)::value;
      // K-layout A: lane copies logical chunk (lane % KC) ^ swz_k(row)
      static_for<NA>([&](auto t) SMOE_INL {
        char* dst = As + (int(t) * 8 + wave) * KGeom::RPL * KGeom::RB;
        if constexpr (F) dma16s(rA, dst, a_off[t], uint32_t(kl) * 2);
        else dma16(rA, dst, kl + ka[t] < Kp ? a_off[t] + uint32_t(kl) * 2 : kOOB);
      });
      if constexpr (BLAY == LAY_K) {
        static_for<NB>([&](auto t) SMOE_INL {
          char* dst = Bs + (int(t) * 8 + wave) * KGeom::RPL * KGeom::RB;
          if constexpr (F) dma16s(rB, dst, b_off[t], uint32_t(kl) * 2);
          else dma16(rB, dst, kl + kb_[t] < Kp ? b_off[t] + uint32_t(kl) * 2 : kOOB);
        });
      } else {
        // one K part: W[e] viewed [k][n] has K0 rows
        static_for<NB>([&](auto t) SMOE_INL {
          char* dst;
          if constexpr (DUAL) {
            using G = MnGeom<BN / 2>;
            constexpr int tt = int(t) % (NB / 2);
            dst = Bs + (int(t) / (NB / 2)) * (BN / 2) * kBK * 2 + (tt * 8 + wave) * G::RPI * G::RB;
          } else {
            dst = Bs + (int(t) * 8 + wave) * GB::RPI * GB::RB;
          }
          // dual: loads t >= NB/2 read W3
          const rsrc_t& r = (DUAL && int(t) >= NB / 2) ? rB1 : rB0;
          if constexpr (F) dma16s(r, dst, b_off[t], uint32_t(kl) * ldb2);
          else dma16(r, dst, kl + kb_[t] < K0 ? b_off[t] + uint32_t(kl) * ldb2 : kOOB);
        });
      }
    };
    const bool full = kl + kBK <= Kp && (BLAY == LAY_K || kl + kBK <= K0);
    if (full) copies(std::true_type{});
    else copies(std::false_type{});
  };
  auto issue = [&](int kt, char* stg) SMOE_INL {
    if constexpr (MODE == SEG_M) {
      if (kt >= KT0) issue_part(P1{}, (kt - KT0) * kBK, stg);
      else issue_part(P0{}, kt * kBK, stg);
    } else {
      // SEG_K: a plain operand advances by the step's first row (a scalar
      // offset); a gathered one addresses each row from its index
      char* As = stg;
      char* Bs = stg + A_BYTES;
      const int r0 = it.row0 + kt * kBK;
      const uint32_t sa = (uint32_t(r0) * lda2) & uint32_t(~scat_a);
      const uint32_t sb = (uint32_t(r0) * ldb2) & uint32_t(~scat_b);
      auto copies = [&](auto full) SMOE_INL {
        constexpr bool F = decltype(full)::value;
        static_for<NA>([&](auto t) SMOE_INL {
          const uint32_t g = uint32_t(fdiv(gia[t], p.a_fan_m, p.a_fan_s)) * lda2 + a_col[t];
          const uint32_t vo = (g & uint32_t(scat_a)) | (a_off[t] & uint32_t(~scat_a));
          char* dst = As + (int(t) * 8 + wave) * GA::RPI * GA::RB;
          if constexpr (F) dma16s(rA0, dst, vo, sa);
          else dma16(rA0, dst, r0 + ka[t] < it.row1 ? vo + sa : kOOB);
        });
        static_for<NB>([&](auto t) SMOE_INL {
          const uint32_t g = uint32_t(fdiv(gib[t], p.b_fan_m, p.b_fan_s)) * ldb2 + b_col[t];
          const uint32_t vo = (g & uint32_t(scat_b)) | (b_off[t] & uint32_t(~scat_b));
          char* dst = Bs + (int(t) * 8 + wave) * GB::RPI * GB::RB;
          if constexpr (F) dma16s(rB0, dst, vo, sb);
          else dma16(rB0, dst, r0 + kb_[t] < it.row1 ? vo + sb : kOOB);
        });
      };
      if (r0 + kBK <= it.row1) copies(std::true_type{});
      else copies(std::false_type{});
    }
  };

  f32x16_t acc[FM][FN];
  static_for<FM>([&](auto i) SMOE_INL {
    static_for<FN>([&](auto j) SMOE_INL {
      static_for<16>([&](auto v) SMOE_INL { acc[i][j][int(v)] = 0.f; });
    });
  });

  auto frags = [&](const char* stg, int s, bf16x8_t (&af)[FM], bf16x8_t (&bf)[FN]) SMOE_INL {
    const char* As = stg;
    const char* Bs = stg + A_BYTES;
    static_for<FM>([&](auto fm) SMOE_INL {
      if constexpr (ALAY == LAY_K) af[fm] = frag_k(As, wm * WM + fm * 32, s, lane);
      else af[fm] = frag_mn<BM>(As, wm * WM + fm * 32, s, lane);
    });
    static_for<FN>([&](auto fn) SMOE_INL {
      if constexpr (MODE == SEG_M && BLAY == LAY_K) {
        bf[fn] = frag_k(Bs, wn * WN + fn * 32, s, lane);
      } else if constexpr (DUAL) {
        // fn 0: W1 sub-tile, fn 1: W3 sub-tile, same 32 columns
        bf[fn] = frag_mn<BN / 2>(Bs + int(fn) * (BN / 2) * kBK * 2, wn * (WN / 2), s, lane);
      } else {
        bf[fn] = frag_mn<BN>(Bs, wn * WN + fn * 32, s, lane);
      }
    });
  };
  // fragments of two 16-wide k slices: slot 0 / slot 1
  bf16x8_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto mfmas = [&](bf16x8_t (&A)[FM], bf16x8_t (&B)[FN]) SMOE_INL {
    static_for<FM>([&](auto fm) SMOE_INL {
      static_for<FN>([&](auto fn) SMOE_INL {
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B[fn], A[fm], acc[fm][fn], 0, 0, 0);
      });
    });
  };

  // ---------------- pipeline -----------------------------------------------
  // kNS stages.  At the top of step kt each wave waits until its own copies
  // of stages kt and kt+1 have landed (later stages may still be in flight);
  // the barrier then publishes every wave's copies and frees the stage
  // multiplied in step kt-1, which receives stage kt+kNS-1.  Because stage
  // kt+1 is published one step early, each wave reads the first fragments
  // of step kt+1 while the last multiplies of step kt run, and arrives at
  // the next barrier with them in registers.  The barrier is a bare
  // s_barrier: the fragment reads of step kt-1 were consumed by its
  // multiplies, which is all the ordering the stages need.
  static_assert(kNS >= 3, "the next stage is published one step early");
  constexpr int NSL = kBK / 16;   // k slices per stage (even)
  // LDS read instructions per slice: one per K-layout fragment, two per
  // transposed (MN-layout) fragment
  constexpr int kFragReads = FM * (ALAY == LAY_K ? 1 : 2) + FN * ((MODE == SEG_M && BLAY == LAY_K) ? 1 : 2);
  if constexpr (MODE == SEG_K) {
    // indices of the steps issued before the loop's own index copies land
    for (int j = 0; j < kIdxAhead; ++j) idx_copy(j);
    wait_vmem<0>();
    asm volatile("s_barrier" ::: "memory");
  }
  static_for<kNS - 1>([&](auto s) SMOE_INL {
    if (int(s) < KT) {
      if constexpr (MODE == SEG_K) idx_copy(int(s) + kIdxAhead);
      idx_fetch(int(s));
      issue(int(s), stage(s));
    }
  });
  // first fragments of step 0 (read before the loop, so that every step's
  // code sees the same outstanding LDS reads and the compiler's waits for
  // them stay exact)
  if (kNS - 2 < KT) wait_vmem<(kNS - 3) * (LPS + IDX)>();
  else wait_vmem<0>();
  asm volatile("s_barrier" ::: "memory");
  frags(stage(std::integral_constant<int, 0>{}), 0, fa0, fb0);
  for (int k0 = 0; k0 < KT; k0 += kNS) {
    static_for<kNS>([&](auto s) SMOE_INL {
      const int kt = k0 + int(s);
      if (kt < KT) {
        if (kt + kNS - 2 < KT) wait_vmem<(kNS - 3) * (LPS + IDX)>();
        else wait_vmem<0>();
        asm volatile("s_barrier" ::: "memory");
        if (kt + kNS - 1 < KT) idx_fetch(kt + kNS - 1);
        static_for<NSL>([&](auto j) SMOE_INL {
          constexpr int J = decltype(j)::value;
          auto& A = (J & 1) == 0 ? fa0 : fa1;
          auto& B = (J & 1) == 0 ? fb0 : fb1;
          auto& An = (J & 1) == 0 ? fa1 : fa0;
          auto& Bn = (J & 1) == 0 ? fb1 : fb0;
          // read the next slice (the next stage's first one after the last;
          // unconditionally, so the outstanding LDS reads are the same on
          // every path: after the last step the values are simply unused)
          if constexpr (J + 1 < NSL) frags(stage(s), J + 1, An, Bn);
          else frags(stage(std::integral_constant<int, int(s) + 1>{}), 0, An, Bn);
          mfmas(A, B);
#if SMOE_SCHED == 1
          // schedule: one multiply, then a share of the fragment reads, so
          // the reads of the next slice run under this slice's multiplies
          static_for<FM * FN>([&](auto i) SMOE_INL {
            constexpr int r0 = int(i) * kFragReads / (FM * FN), r1 = (int(i) + 1) * kFragReads / (FM * FN);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(0x100, r1 - r0, 0);
          });
#else
          // schedule: every fragment read of the next slice first, then this
          // slice's multiplies (a wave issues in order, so reads placed after
          // a multiply would wait for the matrix unit)
          __builtin_amdgcn_sched_group_barrier(0x100, kFragReads, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
#endif
          if constexpr (J == 0) {
            __builtin_amdgcn_sched_barrier(0);
            const int nk = kt + kNS - 1;
            if (nk < KT) {
              // the index copy precedes the stage copies, so the stage waits
              // cover it (see the ring above)
              if constexpr (MODE == SEG_K) idx_copy(nk + kIdxAhead - (kNS - 1));
              issue(nk, stage(std::integral_constant<int, int(s) + kNS - 1>{}));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        });
      }
    });
  }

  // ---------------- epilogue ----------------------------------------------
  // lane holds, for fragment (fm, fn): row (lane & 31) and columns
  // 8q + 4*(lane >> 5) + {0..3}, q = 0..3, values acc[fm][fn][4q + i].
  const int csub = 4 * (lane >> 5);

  // Results leave through LDS: each wave writes the 32 rows of one fragment
  // row (per output) into a private slot, then reads them back as whole
  // 16-byte chunks of consecutive columns, so that every global store
  // instruction writes complete 128-byte lines instead of 16 bytes into 32
  // lines.  The stage buffers are free once every wave is past the loop.
  using ST = typename std::conditional<MODE == SEG_K, float, OutT>::type;
  constexpr int OB = sizeof(ST);                           // bytes per element
  constexpr int WC = (MODE == SEG_M && DUAL) ? WN / 2 : WN;  // output columns per wave
  constexpr int RBE = WC * OB;                              // bytes per staged row
  constexpr int CH = RBE / 16;                              // 16-byte chunks per row
  constexpr int RPR = 64 / CH;                              // rows per read-back instruction
  constexpr int NOUT = (MODE == SEG_M && (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD)) ? 3
                       : (MODE == SEG_M && (EPI == EPI_GELU_FWD || EPI == EPI_GELU_BWD)) ? 2 : 1;
  static_assert((CH & (CH - 1)) == 0 && CH <= 64 && 32 % RPR == 0, "staging geometry");
  static_assert(NOUT * 32 * RBE <= STAGE / 2, "staging slot");
  asm volatile("s_barrier" ::: "memory");
  char* slot;
  {
    const int ob = (wave >> 1) & 3;
    char* base = ob == 0 ? smem0 : ob == 1 ? smem1 : ob == 2 ? smem2 : smem3;
    slot = base + (wave & 1) * (STAGE / 2);
  }
  // lane's 4 values of fragment (fn, q) of one fragment row -> output o
  auto put = [&](int o, auto fn, auto q, const float v[4]) SMOE_INL {
    const int row = lane & 31;
    char* rb = slot + o * 32 * RBE + row * RBE;
    if constexpr (OB == 2) {
      const int c = int(fn) * 4 + int(q);
      *reinterpret_cast<uint2*>(rb + ((c ^ (row & (CH - 1))) << 4) + (lane >> 5) * 8) = pack4_bf16(v);
    } else {
      const int c = int(fn) * 8 + 2 * int(q) + (lane >> 5);
      *reinterpret_cast<float4*>(rb + ((c ^ (row & (CH - 1))) << 4)) = make_float4(v[0], v[1], v[2], v[3]);
    }
  };
  // staged output o -> global: row j of the fragment row goes to
  // base + rowoff(j) + colbase; rowoff / ok are held by lane j
  // ADD: fp32 atomic adds of the four values instead of one store (the
  // fused combine; several assignments add into one token's row)
  auto flush = [&](int o, ST* base, int64_t rowoff, bool ok, int colbase, auto add) SMOE_INL {
    const uint32_t ro_lo = uint32_t(rowoff), ro_hi = uint32_t(uint64_t(rowoff) >> 32);
    static_for<32 / RPR>([&](auto i) SMOE_INL {
      const int j = int(i) * RPR + lane / CH, c = lane % CH;
      const uint4 d = *reinterpret_cast<const uint4*>(slot + o * 32 * RBE + j * RBE + ((c ^ (j & (CH - 1))) << 4));
      const int64_t ro = int64_t((uint64_t(uint32_t(__shfl(int(ro_hi), j, kWave))) << 32) |
                                 uint32_t(__shfl(int(ro_lo), j, kWave)));
      const bool rok_j = __shfl(int(ok), j, kWave) != 0;
      const int colc = colbase + c * (16 / OB);
      if (rok_j && colc < p.N) {
        if constexpr (decltype(add)::value && std::is_same<ST, float>::value) {
          float* dst = reinterpret_cast<float*>(base + ro + colc);
          unsafeAtomicAdd(dst, __uint_as_float(d.x));
          unsafeAtomicAdd(dst + 1, __uint_as_float(d.y));
          unsafeAtomicAdd(dst + 2, __uint_as_float(d.z));
          unsafeAtomicAdd(dst + 3, __uint_as_float(d.w));
        } else {
          *reinterpret_cast<uint4*>(base + ro + colc) = d;
        }
      }
    });
  };
  constexpr std::false_type kStore{};
  constexpr std::true_type kAdd{};

  if constexpr (MODE == SEG_K) {
    float* dst = (it.nitems == 1) ? static_cast<float*>(p.c0) + int64_t(it.e) * p.Mo * p.N
                                  : p.partial + int64_t(T.chunk) * p.Mo * p.N;
    static_for<FM>([&](auto fm) SMOE_INL {
      const int i = T.m0 + wm * WM + fm * 32 + (lane & 31);
      static_for<FN>([&](auto fn) SMOE_INL {
        static_for<4>([&](auto q) SMOE_INL {
          const float v[4] = {acc[fm][fn][4 * int(q)], acc[fm][fn][4 * int(q) + 1],
                              acc[fm][fn][4 * int(q) + 2], acc[fm][fn][4 * int(q) + 3]};
          put(0, fn, q, v);
        });
      });
      flush(0, dst, int64_t(i) * p.N, i < p.Mo, T.n0 + wn * WN, kStore);
    });
  } else {
    OutT* c0 = static_cast<OutT*>(p.c0);
    OutT* c1 = static_cast<OutT*>(p.c1);
    OutT* c2 = static_cast<OutT*>(p.c2);
    const uint16_t* x0 = static_cast<const uint16_t*>(p.aux0);
    const uint16_t* x1 = static_cast<const uint16_t*>(p.aux1);
    constexpr int FNR = DUAL ? FN / 2 : FN;
    // the epilogue reads bf16 operands (h / h1, h3 of the backward
    // epilogues; the input rows of the gate gradient) for every output
    constexpr bool AUX0 = EPI == EPI_GELU_BWD || EPI == EPI_SWIGLU_BWD || EPI == EPI_STORE;
    constexpr bool AUX1 = EPI == EPI_SWIGLU_BWD;
    const bool aux0_on = EPI == EPI_STORE ? p.dgpart != nullptr : AUX0;

    // row information of the lane's FM rows, read up front
    int gr[FM], sp[FM];
    bool rok[FM];
    float g[FM];
    static_for<FM>([&](auto fm) SMOE_INL {
      gr[fm] = it.row0 + wm * WM + fm * 32 + (lane & 31);
      rok[fm] = gr[fm] < it.row1;
      sp[fm] = rok[fm] ? p.sidx[gr[fm]] : 0;
    });
    static_for<FM>([&](auto fm) SMOE_INL { g[fm] = (p.gate && rok[fm]) ? p.gate[sp[fm]] : 1.f; });
    auto col = [&](auto fn, auto q) SMOE_INL {
      return T.n0 + (DUAL ? wn * (WN / 2) : wn * WN) + int(fn) * 32 + 8 * int(q) + csub;
    };
    // aux operands of one fragment row.  The lane needs 4 bf16 of each of
    // the four 8-column chunks of a fragment's 32 columns (half lane >> 5
    // of each chunk); lane half h reads chunks 2h and 2h+1 whole (16 bytes
    // each, half the load instructions and line accesses of 8-byte reads)
    // and the halves it lacks are swapped with lane l ^ 32 when the row is
    // used.  Double-buffered over fm so the reads of row fm+1 are in flight
    // while row fm is computed and stored.  Masked lanes read a clamped,
    // valid address.
    const int hh = lane >> 5;
    uint4 rx0[2][FNR][2], rx1[2][AUX1 ? FNR : 1][2];
    auto load_aux = [&](auto fm, auto buf) SMOE_INL {
      if constexpr (AUX0) {
        if (aux0_on) {
          const int64_t row = EPI == EPI_STORE ? (p.aux_scat ? sp[fm] / p.aux_fan : gr[fm]) : gr[fm];
          const int64_t rr = rok[fm] ? row : (EPI == EPI_STORE && p.aux_scat ? 0 : it.row0);
          static_for<FNR>([&](auto fn) SMOE_INL {
            static_for<2>([&](auto j) SMOE_INL {
              const int n = T.n0 + wn * WN + int(fn) * 32 + 8 * (2 * hh + int(j));
              const int nn = n < p.N ? n : 0;
              rx0[buf][fn][j] = *reinterpret_cast<const uint4*>(x0 + rr * p.ldaux + nn);
              if constexpr (AUX1) rx1[buf][fn][j] = *reinterpret_cast<const uint4*>(x1 + rr * p.ldaux + nn);
            });
          });
        }
      }
    };
    // the lane's 4 values of chunk q of fragment fn from the 16-byte reads
    auto aux_vals = [&](uint4 (&rx)[2], uint2 (&ax)[4]) SMOE_INL {
      static_for<2>([&](auto j) SMOE_INL {
        const uint2 lo = make_uint2(rx[j].x, rx[j].y), hi = make_uint2(rx[j].z, rx[j].w);
        const uint2 own = hh ? hi : lo, send = hh ? lo : hi;
        const uint2 recv = make_uint2(uint32_t(__shfl_xor(int(send.x), 32, kWave)),
                                      uint32_t(__shfl_xor(int(send.y), 32, kWave)));
        ax[int(j)] = hh ? recv : own;
        ax[2 + int(j)] = hh ? own : recv;
      });
    };
    auto unpack = [&](uint2 w, float v[4]) SMOE_INL { unpack4_bf16(w, v); };
    load_aux(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    static_for<FM>([&](auto fm) SMOE_INL {
      constexpr int BUF = int(fm) & 1;
      if constexpr (int(fm) + 1 < FM)
        load_aux(std::integral_constant<int, int(fm) + 1>{}, std::integral_constant<int, BUF ^ 1>{});
      const int64_t grow = gr[fm];
      const int64_t crow = p.c_scat ? sp[fm] : grow;
      float dgacc = 0.f;
      static_for<FNR>([&](auto fn) SMOE_INL {
        uint2 ax0[4], ax1[4];
        if constexpr (AUX0) {
          if (aux0_on) aux_vals(rx0[BUF][fn], ax0);
        }
        if constexpr (AUX1) aux_vals(rx1[BUF][fn], ax1);
        static_for<4>([&](auto q) SMOE_INL {
          const int n = col(fn, q);
          if (rok[fm] && n < p.N) {
            float v[4] = {acc[fm][fn][4 * int(q)], acc[fm][fn][4 * int(q) + 1], acc[fm][fn][4 * int(q) + 2],
                          acc[fm][fn][4 * int(q) + 3]};
            if constexpr (EPI == EPI_STORE) {
              if (p.dgpart) {
                float xv[4];
                unpack(ax0[q], xv);
                dgacc += xv[0] * v[0] + xv[1] * v[1] + xv[2] * v[2] + xv[3] * v[3];
              }
              if (p.gate) {
                static_for<4>([&](auto i) SMOE_INL { v[i] *= g[fm]; });
              }
              put(0, fn, q, v);
            } else if constexpr (EPI == EPI_GELU_FWD) {
              // h stored in bf16; a computed from the stored h
              static_assert(std::is_same<OutT, uint16_t>::value, "bf16 epilogue");
              const uint2 wh = pack4_bf16(v);
              float h[4], a[4];
              unpack4_bf16(wh, h);
              static_for<4>([&](auto i) SMOE_INL { a[i] = gelu_f(h[i]); });
              float hs[4];
              unpack4_bf16(wh, hs);
              put(0, fn, q, hs);
              put(1, fn, q, a);
            } else if constexpr (EPI == EPI_SWIGLU_FWD) {
              static_assert(std::is_same<OutT, uint16_t>::value, "bf16 epilogue");
              float v3[4], h1[4], h3[4], a[4];
              static_for<4>([&](auto i) SMOE_INL { v3[i] = acc[fm][fn + FN / 2][4 * int(q) + int(i)]; });
              const uint2 w1 = pack4_bf16(v), w3 = pack4_bf16(v3);
              unpack4_bf16(w1, h1);
              unpack4_bf16(w3, h3);
              static_for<4>([&](auto i) SMOE_INL { a[i] = silu_f(h1[i]) * h3[i]; });
              put(0, fn, q, h1);
              put(1, fn, q, h3);
              put(2, fn, q, a);
            } else if constexpr (EPI == EPI_GELU_BWD) {
              static_assert(std::is_same<OutT, uint16_t>::value, "bf16 epilogue");
              float h[4], a[4], dh[4], ag[4];
              unpack(ax0[q], h);
              static_for<4>([&](auto i) SMOE_INL { a[i] = gelu_f(h[i]); });
              unpack4_bf16(pack4_bf16(a), a);   // a as stored in the forward
              static_for<4>([&](auto i) SMOE_INL {
                dgacc += a[i] * v[i];
                dh[i] = g[fm] * v[i] * gelu_grad_f(h[i]);
                ag[i] = g[fm] * a[i];
              });
              put(0, fn, q, dh);
              put(1, fn, q, ag);
            } else if constexpr (EPI == EPI_SWIGLU_BWD) {
              static_assert(std::is_same<OutT, uint16_t>::value, "bf16 epilogue");
              float h1[4], h3[4], sg[4], si[4], a[4], d1[4], d3[4], ag[4];
              unpack(ax0[q], h1);
              unpack(ax1[q], h3);
              static_for<4>([&](auto i) SMOE_INL {
                sg[i] = sigmoid_f(h1[i]);
                si[i] = h1[i] * sg[i];
                a[i] = si[i] * h3[i];
              });
              unpack4_bf16(pack4_bf16(a), a);   // a as stored in the forward
              static_for<4>([&](auto i) SMOE_INL {
                dgacc += a[i] * v[i];
                const float dA = g[fm] * v[i];
                d1[i] = dA * h3[i] * (sg[i] * (1.0f + h1[i] * (1.0f - sg[i])));
                d3[i] = dA * si[i];
                ag[i] = g[fm] * a[i];
              });
              put(0, fn, q, d1);
              put(1, fn, q, d3);
              put(2, fn, q, ag);
            }
          }
        });
      });
      if (p.dgpart) {
        dgacc += __shfl_xor(dgacc, 32, kWave);
        if (lane < 32 && rok[fm]) p.dgpart[int64_t(T.nt * 4 + wn) * p.M + gr[fm]] = dgacc;
      }
      // staged rows -> global (grouped rows, or scattered for EPI_STORE)
      const int cb = T.n0 + (DUAL ? wn * (WN / 2) : wn * WN);
      if constexpr (EPI == EPI_STORE) {
        if (c0) {
          if (p.c_add_fan > 0)
            flush(0, c0, (crow / p.c_add_fan) * p.ldc, rok[fm], cb, kAdd);
          else
            flush(0, c0, crow * p.ldc, rok[fm], cb, kStore);
        }
      } else if constexpr (EPI == EPI_GELU_FWD) {
        flush(0, c0, grow * p.ldc, rok[fm], cb, kStore);
        flush(1, c1, grow * p.ldc, rok[fm], cb, kStore);
      } else if constexpr (EPI == EPI_SWIGLU_FWD) {
        flush(0, c0, grow * p.ldc, rok[fm], cb, kStore);
        flush(1, c1, grow * p.ldc, rok[fm], cb, kStore);
        flush(2, c2, grow * p.ldc, rok[fm], cb, kStore);
      } else if constexpr (EPI == EPI_GELU_BWD) {
        flush(0, c0, grow * p.ldc, rok[fm], cb, kStore);
        flush(1, c2, grow * p.ldc, rok[fm], cb, kStore);
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        flush(0, c0, grow * p.ldc, rok[fm], cb, kStore);
        flush(1, c1, grow * p.ldc, rok[fm], cb, kStore);
        flush(2, c2, grow * p.ldc, rok[fm], cb, kStore);
      }
    });
  }
}

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
      return a0[int64_t(src) * p.lda + i];
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
      pl.slots = 4 * pl.n_tiles;
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

template <int BM, int BN, int MODE, int EPI, int BLAY, bool DUAL, class OutT>
static void go_bf16(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, MODE, EPI, BLAY, DUAL, OutT>), dim3(unsigned(pl.grid)),
                     dim3(kThreads), 0, st, a);
}

template <int MODE, int EPI, int BLAY, bool DUAL, class OutT>
static bool dispatch_tiles(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if constexpr (DUAL) {
    if (pl.bm == 256 && pl.bn == 256) go_bf16<256, 256, MODE, EPI, BLAY, DUAL, OutT>(a, pl, st);
    else if (pl.bm == 128 && pl.bn == 256) go_bf16<128, 256, MODE, EPI, BLAY, DUAL, OutT>(a, pl, st);
    else return false;
  } else {
    if (pl.bm == 256 && pl.bn == 256) go_bf16<256, 256, MODE, EPI, BLAY, DUAL, OutT>(a, pl, st);
    else if (pl.bm == 256 && pl.bn == 128) go_bf16<256, 128, MODE, EPI, BLAY, DUAL, OutT>(a, pl, st);
    else if (pl.bm == 128 && pl.bn == 256) go_bf16<128, 256, MODE, EPI, BLAY, DUAL, OutT>(a, pl, st);
    else if (pl.bm == 128 && pl.bn == 128) go_bf16<128, 128, MODE, EPI, BLAY, DUAL, OutT>(a, pl, st);
    else return false;
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
  if (pl.mode == SEG_K) return dispatch_tiles<SEG_K, EPI_PARTIAL, LAY_MN, false, float>(a, pl, st);
  switch (pl.epi) {
    case EPI_STORE:
      if (a.b_nk) {
        return out_f32 ? dispatch_tiles<SEG_M, EPI_STORE, LAY_K, false, float>(a, pl, st)
                       : dispatch_tiles<SEG_M, EPI_STORE, LAY_K, false, uint16_t>(a, pl, st);
      }
      return out_f32 ? dispatch_tiles<SEG_M, EPI_STORE, LAY_MN, false, float>(a, pl, st)
                     : dispatch_tiles<SEG_M, EPI_STORE, LAY_MN, false, uint16_t>(a, pl, st);
    case EPI_GELU_FWD: return dispatch_tiles<SEG_M, EPI_GELU_FWD, LAY_MN, false, uint16_t>(a, pl, st);
    case EPI_SWIGLU_FWD: return dispatch_tiles<SEG_M, EPI_SWIGLU_FWD, LAY_MN, true, uint16_t>(a, pl, st);
    case EPI_GELU_BWD: return dispatch_tiles<SEG_M, EPI_GELU_BWD, LAY_K, false, uint16_t>(a, pl, st);
    case EPI_SWIGLU_BWD: return dispatch_tiles<SEG_M, EPI_SWIGLU_BWD, LAY_K, false, uint16_t>(a, pl, st);
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
