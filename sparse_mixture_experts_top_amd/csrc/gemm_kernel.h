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
//    while the first waits on LDS, copies or the barrier.  Or 256 threads =
//    4 waves, one per SIMD, in a 2 x 2 grid, each owning (BM/2) x (BN/2)
//    with its accumulators in the AGPRs: each multiply then takes 0.5 KB of
//    LDS fragment reads instead of 0.75 KB, and the clock, which the chip's
//    power limit sets, runs higher.
//  - The K loop runs a steady form while every stage lies whole inside the
//    reduction: the copies keep their lanes' offsets and each step sets one
//    scalar offset, so the loop carries ~1.5 other instructions per
//    multiply; the last steps, and reductions not a multiple of 64, take the
//    general form (masked copies, per-step conditions).
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
//  - Workgroups are renumbered over the tiles that exist (counted on the
//    device from the expert row counts), ordered in groups of 8 m-tiles
//    sweeping n.  Each XCD (blockIdx % 8 on MI355X) takes runs of 32
//    consecutive tiles, the 8 XCDs neighbouring runs at the same time: the
//    concurrent tiles on one XCD share A rows and weight panels in its L2,
//    the XCDs share them in the last-level cache, and no XCD idles on the
//    grid's empty tail.
//
// fp32 kernel: the same contract with plain FMA on 64x64 tiles, used for
// fp32 runs (a small, launch-bound regime).
#pragma once
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
constexpr int kBK = 64;         // K of one pipeline stage: 128-byte rows of a K-contiguous operand
constexpr int kNSL = kBK / 16;  // 16-wide k slices per stage
constexpr uint32_t kOOB = 0xFFFFFFF0u;  // byte offset past every buffer: reads as 0

enum Lay { LAY_K = 0, LAY_MN = 1 };

SMOE_DEV int fdiv(int x, uint32_t m, int s) { return int((uint64_t(uint32_t(x)) * m) >> s); }

// K-layout tile: row j (one gathered token row, or one column of W read as
// W^T) holds the stage's 64 values of k, 128 bytes = 8 chunks of 16 bytes;
// chunk c of row j sits at chunk c ^ swz_k(j).  A 128-bit LDS read serves
// 16 lanes at a time, i.e. 16 consecutive rows at one logical chunk; the 64
// banks cover 256 bytes = 2 rows, and the swizzle gives the 8 row pairs 8
// distinct chunks.  A wave's copy instruction fills 8 whole rows: every
// lane group of 8 reads one complete 128-byte line (whole lines move twice
// as fast from L2 into LDS as half lines).
struct KGeom {
  static constexpr int RB = 2 * kBK;    // bytes per row
  static constexpr int KC = kBK / 8;    // 16-byte chunks per row
  static constexpr int RPL = 64 / KC;   // rows per wave copy
};
SMOE_DEV int swz_k(int row) { return (row >> 1) & 7; }
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
// The 64 lanes of the wave each copy 16 bytes (at byte offset voff + soff
// of the buffer) to wave_lds + 16 * lane, straight into LDS.  soff is the
// wave-uniform part (a step's advance along k), so a copy inside the buffer
// needs no vector arithmetic per step.  Written as inline asm so that the
// compiler does not order later LDS reads of the OTHER stage behind these
// copies (it cannot tell the stages apart); the kernel waits for the copies
// itself (wait_vmem) before the barrier that publishes a stage.  The asm
// has no register outputs; its inputs are read when it issues.  The LDS
// address is the low 32 bits of the flat address of wave_lds (the LDS
// aperture starts at a multiple of 4 GiB).
SMOE_DEV uint32_t lds_addr(const char* p) { return uint32_t(reinterpret_cast<uintptr_t>(p)); }
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
// wait until every LDS access of this wave is done: s_waitcnt lgkmcnt(0)
SMOE_DEV void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

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
  // depends on the per-expert row counts and is counted here.  Block b runs
  // on XCD b % 8, and an XCD's blocks start in order, 32 at a time (one per
  // CU).  The real tiles are dealt in rounds of 8 x 32: XCD x takes the
  // x-th run of 32 consecutive tiles of each round, so the 8 XCDs work on
  // neighbouring tiles at the same time (the same A panels with different
  // n-tiles, or the same weight panels) and the copies they share come
  // from the last-level cache instead of HBM.  The tiles past the last
  // whole round are dealt in 8 even runs.  The blocks past an XCD's share
  // have no tile.  (Dealing over the upper-bound range would leave the
  // last XCDs with the empty tail.)
  constexpr int kXcd = 8, kRun = 32;
  constexpr int GM = 8;
  constexpr int NCOLS = DUAL ? BN / 2 : BN;
  int n_real, units = 0;
  const int ntn = (p.N + NCOLS - 1) / NCOLS;
  const int ti = (p.Mo + BM - 1) / BM, tj = (p.N + BN - 1) / BN, tpc = ti * tj;
  const int unit = MODE == SEG_M ? BM : p.KS;
  // up to 64 experts: one read and scan of the offsets for the count and the
  // lookup; more: a pass for each
  const bool one_pass = p.E <= kWave;
  ItemScan sc;
  if (one_pass) sc = scan_items(p.offsets, p.E, unit);
  const int items = one_pass ? sc.total : total_items(p.offsets, p.E, unit);
  if constexpr (MODE == SEG_M) {
    units = items;   // real m-tiles
    n_real = units * ntn;
  } else {
    n_real = items * tpc;
  }
  auto locate = [&](int item, Item& it) SMOE_INL {
    return one_pass ? pick_item(sc, p.E, unit, item, it) : find_item(p.offsets, p.E, unit, item, it);
  };
  const int lo = MODE == SEG_M ? p.g_base : 0;
  const int hi = (MODE == SEG_M && p.g_count > 0) ? min(n_real, lo + p.g_count) : n_real;
  if (hi <= lo) return false;
  const int n = hi - lo, x = int(blockIdx.x) % kXcd, j = int(blockIdx.x) / kXcd;
  const int full = n / (kXcd * kRun);
  int g;
  if (j < full * kRun) {
    g = lo + (j / kRun) * (kXcd * kRun) + x * kRun + j % kRun;
  } else {
    const int rem = n - full * kXcd * kRun;
    const int per = (rem + kXcd - 1) / kXcd;
    const int jj = j - full * kRun;
    if (jj >= per) return false;
    g = lo + full * kXcd * kRun + x * per + jj;
    if (g >= hi) return false;
  }
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
    return locate(mt, t.it);
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
    return locate(t.chunk, t.it);
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
template <int R, int NW>
SMOE_DEV void mn_slot(int t, int wave, int lane, int& krow, int& chunk) {
  using G = MnGeom<R>;
  krow = (t * NW + wave) * G::RPI + lane / G::CPR;
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

template <int BM, int BN, int NW, int MODE, int EPI, int BLAY, bool DUAL, class OutT>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int ALAY = MODE == SEG_M ? LAY_K : LAY_MN;
  static_assert(NW == 8 || NW == 4, "waves");
  constexpr int WGN = NW / 2;                  // wave columns (2 wave rows)
  constexpr int WM = BM / 2, WN = BN / WGN;    // wave tile
  constexpr int FM = WM / 32, FN = WN / 32;    // fragments per wave
  constexpr int A_BYTES = BM * kBK * 2, B_BYTES = BN * kBK * 2;
  static_assert(BN >= 128 && BM >= 128, "tile");
  static_assert(!DUAL || (MODE == SEG_M && BLAY == LAY_MN && BN == 256), "dual B layout");
  // Stage buffers of 64 k.  Rows mode keeps three A buffers and two B
  // buffers (160 KB at 256 x 256): the A copies of a stage then have two
  // steps to land and are spread over the first three slices of a step,
  // and only the B copies share the last slice.  Weights mode keeps two of
  // each (its index rings take the rest of the LDS).
  constexpr bool A3 = MODE == SEG_M;
  constexpr bool KSPLIT = MODE == SEG_K;   // weights mode: B copies one step later
  constexpr int NBA = A3 ? 3 : 2;
  constexpr int LDS_BYTES = NBA * A_BYTES + 2 * B_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  auto abuf = [&](auto s) SMOE_INL -> char* { return lds + (decltype(s)::value % NBA) * A_BYTES; };
  auto bbuf = [&](auto s) SMOE_INL -> char* { return lds + NBA * A_BYTES + (decltype(s)::value % 2) * B_BYTES; };
  constexpr int UNROLL = A3 ? 6 : 2;

  TileInfo T;
  if (!tile_of_block<BM, BN, MODE, DUAL>(p, T)) return;
  const Item& it = T.it;

  // wave index as a scalar: everything derived from it (LDS copy targets,
  // per-wave roles) stays wave-uniform for the compiler
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // ---------------- K steps ------------------------------------------------
  // SEG_M: K is [part 0: K0 columns of a0 / b0 | part 1: K-K0 of a1 / b1];
  // each kBK-wide step lies inside one part.  SEG_K: the chunk's rows.
  const int K0 = MODE == SEG_M ? p.K0 : it.row1 - it.row0;
  const int K1 = MODE == SEG_M ? p.K - p.K0 : 0;
  const int KT0 = (K0 + kBK - 1) / kBK;
  const int KT = KT0 + (K1 + kBK - 1) / kBK;

  // ---------------- per-lane copy addressing -------------------------------
  constexpr int NA = BM * kBK / (512 * NW), NB = BN * kBK / (512 * NW);   // buffer loads per wave per operand
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
  // step that crosses it masks the lanes past it.
  uint32_t a_off[NA], b_off[NB];
  int ka[NA], kb_[NB];
  // SEG_K: column byte offset of the lane (a_col / b_col) for gathered rows
  uint32_t a_col[MODE == SEG_K ? NA : 1], b_col[MODE == SEG_K ? NB : 1];

  if constexpr (MODE == SEG_M) {
    static_for<NA>([&](auto t) SMOE_INL {
      const int row = (int(t) * NW + wave) * KGeom::RPL + lane / KGeom::KC;
      const int gr = it.row0 + row;
      const int src = gr < it.row1 ? (p.a_scat ? p.sidx[gr] / p.a_fan : gr) : -1;
      ka[t] = ((lane % KGeom::KC) ^ swz_k(row)) * 8;
      a_off[t] = (src >= 0 ? uint32_t(int64_t(src) * p.lda * 2) : 0u) + uint32_t(ka[t]) * 2;
    });
    if constexpr (BLAY == LAY_K) {
      // W[e] viewed [n][k]: N rows of ldb
      static_for<NB>([&](auto t) SMOE_INL {
        const int row = (int(t) * NW + wave) * KGeom::RPL + lane / KGeom::KC;
        const int n = T.n0 + row;
        kb_[t] = ((lane % KGeom::KC) ^ swz_k(row)) * 8;
        b_off[t] = (n < p.N ? uint32_t(int64_t(n) * p.ldb * 2) : 0u) + uint32_t(kb_[t]) * 2;
      });
    } else {
      // W[e] viewed [k][n]: K rows of ldb.  Dual: the tile is two BN/2-column
      // sub-tiles, W1 columns then W3 columns (loads t < NB/2 fill the first)
      static_for<NB>([&](auto t) SMOE_INL {
        int krow, c;
        if constexpr (DUAL) mn_slot<BN / 2, NW>(int(t) % (NB / 2), wave, lane, krow, c);
        else mn_slot<BN, NW>(int(t), wave, lane, krow, c);
        const int col = T.n0 + 8 * c;
        kb_[t] = krow;
        b_off[t] = uint32_t(krow) * ldb2 + uint32_t(col) * 2;
      });
    }
  } else {
    static_for<NA>([&](auto t) SMOE_INL {
      int krow, c;
      mn_slot<BM, NW>(int(t), wave, lane, krow, c);
      a_col[t] = uint32_t(T.m0 + 8 * c) * 2;
      ka[t] = (int(t) * NW + wave) * GA::RPI + lane / GA::CPR;   // row within the step
      a_off[t] = uint32_t(ka[t]) * lda2 + a_col[t];
    });
    static_for<NB>([&](auto t) SMOE_INL {
      int krow, c;
      mn_slot<BN, NW>(int(t), wave, lane, krow, c);
      b_col[t] = uint32_t(T.n0 + 8 * c) * 2;
      kb_[t] = (int(t) * NW + wave) * GB::RPI + lane / GB::CPR;
      b_off[t] = uint32_t(kb_[t]) * ldb2 + b_col[t];
    });
  }
  // descriptors, built once
  const rsrc_t rA0 = descA(std::integral_constant<int, 0>{});
  const rsrc_t rA1 = descA(std::integral_constant<int, 1>{});
  const rsrc_t rB0 = descB(std::integral_constant<int, 0>{});
  const rsrc_t rB1 = descB(std::integral_constant<int, 1>{});

  // SEG_K: the source rows of the gathered operand come from
  // sorted_scattered_idxs.  The indices of the 64 grouped rows of step j are
  // copied into an LDS ring (slot j % kRing, one dword per lane) at the
  // barrier of step j-4, so the wait before the barrier of step j-3
  // covers them and that barrier publishes them; they are read into
  // registers right after it and address the copies of stage j, issued at
  // the barrier of step j-2.  Reading them back from LDS keeps the loop free
  // of scalar loads and data-dependent branches.
  // A gated weight gradient (EPI_PARTIAL_GATED) copies the rows' scales
  // into a second ring the same way; the fragments of A are scaled in
  // registers right before their multiplies, so no scaled copy of A exists.
  constexpr int kRing = 8, kIdxAhead = 4;
  constexpr bool GATED = MODE == SEG_K && EPI == EPI_PARTIAL_GATED;
  __shared__ __attribute__((aligned(16))) int ring[MODE == SEG_K ? kRing * 64 : 1];
  __shared__ __attribute__((aligned(16))) float gring[GATED ? kRing * 64 : 1];
  auto idx_copy = [&](int j) SMOE_INL {
    if constexpr (MODE == SEG_K) {
      const uint32_t r = uint32_t(it.row0 + j * kBK + lane);
      dma4(make_rsrc(p.sidx, int64_t(p.M) * 4), reinterpret_cast<char*>(ring + (j % kRing) * 64), r * 4u);
      if constexpr (GATED)
        dma4(make_rsrc(p.kscale, int64_t(p.M) * 4), reinterpret_cast<char*>(gring + (j % kRing) * 64), r * 4u);
    }
  };
  constexpr int SA = MODE == SEG_K ? NA : 1, SB = MODE == SEG_K ? NB : 1;
  int gia[SA], gib[SB];
  // reads for both operands, gathered or not (no branch: the general plans
  // select the index or the plain row); the steady plans read only the
  // gathered operand's
  auto idx_fetch_of = [&](int j, auto want_a, auto want_b) SMOE_INL {
    if constexpr (MODE == SEG_K) {
      const int* slot = ring + (j % kRing) * 64;
      if constexpr (decltype(want_a)::value) static_for<NA>([&](auto t) SMOE_INL { gia[t] = slot[ka[t]]; });
      if constexpr (decltype(want_b)::value) static_for<NB>([&](auto t) SMOE_INL { gib[t] = slot[kb_[t]]; });
    }
  };
  auto idx_fetch = [&](int j) SMOE_INL { idx_fetch_of(j, std::true_type{}, std::true_type{}); };

  // ---------------- copies of one stage ------------------------------------
  // planA(kt) / planB(kt) set, for every copy of an operand at step kt, the
  // lane's byte offset (cva / cvb), the operand's scalar offset and its
  // descriptor; copyA(c, buf) / copyB(c, buf) issue copy c into a stage
  // buffer.  A step inside the reduction adds the step's advance as the
  // scalar offset; the step that crosses the end of a part (a uniform
  // branch, at most one per part) masks the lanes past it instead.
  uint32_t cva[NA], cvb[NB];
  uint32_t csa = 0, csb = 0;
  rsrc_t cra = rA0, crb = rB0;
  auto planA = [&](int kt) SMOE_INL {
    if constexpr (MODE == SEG_M) {
      const bool p1 = kt >= KT0;
      const int kl = (p1 ? kt - KT0 : kt) * kBK;
      const int Kp = p1 ? K1 : K0;
      cra = p1 ? rA1 : rA0;
      const uint32_t sa = uint32_t(kl) * 2;
      if (kl + kBK <= Kp) {
        static_for<NA>([&](auto t) SMOE_INL { cva[t] = a_off[t]; });
        csa = sa;
      } else {
        static_for<NA>([&](auto t) SMOE_INL { cva[t] = kl + ka[t] < Kp ? a_off[t] + sa : kOOB; });
        csa = 0;
      }
    } else {
      // a plain operand advances by the step's first row (a scalar offset);
      // a gathered one addresses each row from its index
      const int r0 = it.row0 + kt * kBK;
      const uint32_t sa = (uint32_t(r0) * lda2) & uint32_t(~scat_a);
      static_for<NA>([&](auto t) SMOE_INL {
        const uint32_t g = uint32_t(fdiv(gia[t], p.a_fan_m, p.a_fan_s)) * lda2 + a_col[t];
        cva[t] = (g & uint32_t(scat_a)) | (a_off[t] & uint32_t(~scat_a));
      });
      if (r0 + kBK <= it.row1) {
        csa = sa;
      } else {
        static_for<NA>([&](auto t) SMOE_INL { cva[t] = r0 + ka[t] < it.row1 ? cva[t] + sa : kOOB; });
        csa = 0;
      }
    }
    // uniform by construction; say so, so that it stays a scalar operand
    csa = __builtin_amdgcn_readfirstlane(csa);
  };
  auto planB = [&](int kt) SMOE_INL {
    if constexpr (MODE == SEG_M) {
      const bool p1 = kt >= KT0;
      const int kl = (p1 ? kt - KT0 : kt) * kBK;
      const int Kp = p1 ? K1 : K0;
      crb = (BLAY == LAY_K && p1) ? rB1 : rB0;
      const uint32_t sb = BLAY == LAY_K ? uint32_t(kl) * 2 : uint32_t(kl) * ldb2;
      if (kl + kBK <= Kp) {
        static_for<NB>([&](auto t) SMOE_INL { cvb[t] = b_off[t]; });
        csb = sb;
      } else {
        static_for<NB>([&](auto t) SMOE_INL { cvb[t] = kl + kb_[t] < Kp ? b_off[t] + sb : kOOB; });
        csb = 0;
      }
    } else {
      const int r0 = it.row0 + kt * kBK;
      const uint32_t sb = (uint32_t(r0) * ldb2) & uint32_t(~scat_b);
      static_for<NB>([&](auto t) SMOE_INL {
        const uint32_t g = uint32_t(fdiv(gib[t], p.b_fan_m, p.b_fan_s)) * ldb2 + b_col[t];
        cvb[t] = (g & uint32_t(scat_b)) | (b_off[t] & uint32_t(~scat_b));
      });
      if (r0 + kBK <= it.row1) {
        csb = sb;
      } else {
        static_for<NB>([&](auto t) SMOE_INL { cvb[t] = r0 + kb_[t] < it.row1 ? cvb[t] + sb : kOOB; });
        csb = 0;
      }
    }
    csb = __builtin_amdgcn_readfirstlane(csb);
  };
  // Rows mode, a stage that lies inside one part of K with no lane past
  // its end (every stage, when the parts are whole multiples of the step):
  // the copies keep their lanes' offsets at k = 0 and the step sets only
  // the scalar offset and the part's descriptors, all scalar work.
  auto planA_steady = [&](int kt) SMOE_INL {
    const bool p1 = kt >= KT0;
    cra = p1 ? rA1 : rA0;
    csa = __builtin_amdgcn_readfirstlane(uint32_t((p1 ? kt - KT0 : kt) * kBK) * 2);
  };
  auto planB_steady = [&](int kt) SMOE_INL {
    const bool p1 = kt >= KT0;
    const uint32_t kl = uint32_t((p1 ? kt - KT0 : kt) * kBK);
    crb = (BLAY == LAY_K && p1) ? rB1 : rB0;
    csb = __builtin_amdgcn_readfirstlane(BLAY == LAY_K ? kl * 2 : kl * ldb2);
  };
  // Weights mode, a stage of 64 rows that all lie inside the chunk: the
  // gathered operand's copies take their rows' offsets from the indices,
  // the plain operand's keep their lanes' offsets and advance by a scalar
  // offset (no masks, no selects between the two forms).
  auto planA_k = [&](int kt, auto gathered) SMOE_INL {
    if constexpr (decltype(gathered)::value) {
      static_for<NA>([&](auto t) SMOE_INL { cva[t] = uint32_t(fdiv(gia[t], p.a_fan_m, p.a_fan_s)) * lda2 + a_col[t]; });
      csa = 0;
    } else {
      csa = __builtin_amdgcn_readfirstlane(uint32_t(it.row0 + kt * kBK) * lda2);
    }
  };
  auto planB_k = [&](int kt, auto gathered) SMOE_INL {
    if constexpr (decltype(gathered)::value) {
      static_for<NB>([&](auto t) SMOE_INL { cvb[t] = uint32_t(fdiv(gib[t], p.b_fan_m, p.b_fan_s)) * ldb2 + b_col[t]; });
      csb = 0;
    } else {
      // the copies that use it run at the next step's start, which may be
      // a general step: keep the general form's lane offsets
      static_for<NB>([&](auto t) SMOE_INL { cvb[t] = b_off[t]; });
      csb = __builtin_amdgcn_readfirstlane(uint32_t(it.row0 + kt * kBK) * ldb2);
    }
  };
  // every copy instruction fills 1 KB of its operand's tile: 8 K-layout
  // rows, or 64 / CPR MN-layout k-rows.  BASE: the lane offsets at k = 0.
  auto copyA = [&](auto c, char* buf, auto base) SMOE_INL {
    constexpr int C = decltype(c)::value;
    dma16s(cra, buf + (C * NW + wave) * 1024, decltype(base)::value ? a_off[C] : cva[C], csa);
  };
  auto copyB = [&](auto c, char* buf, auto steady) SMOE_INL {
    constexpr int t = decltype(c)::value;
    const uint32_t vo = decltype(steady)::value ? b_off[t] : cvb[t];
    if constexpr (DUAL) {
      // loads t >= NB/2 read W3 into the second sub-tile
      constexpr int tt = t % (NB / 2);
      dma16s(t >= NB / 2 ? rB1 : rB0, buf + (t / (NB / 2)) * (BN / 2) * kBK * 2 + (tt * NW + wave) * 1024, vo, csb);
    } else {
      dma16s(crb, buf + (t * NW + wave) * 1024, vo, csb);
    }
  };
  static_assert(KGeom::RPL * KGeom::RB == 1024 && GA::RPI * GA::RB == 1024 && GB::RPI * GB::RB == 1024,
                "1 KB per copy");

  f32x16_t acc[FM][FN];
  static_for<FM>([&](auto i) SMOE_INL {
    static_for<FN>([&](auto j) SMOE_INL {
      static_for<16>([&](auto v) SMOE_INL { acc[i][j][int(v)] = 0.f; });
    });
  });

  // fragment of row block fm (A) / column block fn (B) of k slice s, from
  // an A or B stage buffer
  auto frag_a = [&](const char* As, auto fm, int s) SMOE_INL {
    if constexpr (ALAY == LAY_K) return frag_k(As, wm * WM + int(fm) * 32, s, lane);
    else return frag_mn<BM>(As, wm * WM + int(fm) * 32, s, lane);
  };
  auto frag_b = [&](const char* Bs, auto fn, int s) SMOE_INL {
    if constexpr (MODE == SEG_M && BLAY == LAY_K) {
      return frag_k(Bs, wn * WN + int(fn) * 32, s, lane);
    } else if constexpr (DUAL) {
      // fn < FN/2: W1 sub-tile, the rest: W3 sub-tile, same columns
      constexpr int sub = int(fn) / (FN / 2), f = int(fn) % (FN / 2);
      return frag_mn<BN / 2>(Bs + sub * (BN / 2) * kBK * 2, wn * (WN / 2) + f * 32, s, lane);
    } else {
      return frag_mn<BN>(Bs, wn * WN + int(fn) * 32, s, lane);
    }
  };
  // GATED: A fragments of slice s of step kt times their rows' scales.  A
  // lane's fragment holds k-rows 16s + 8 (lane >> 5) + 0..7 of the step (one
  // column each); each product is rounded to bf16 (nearest even), the value
  // the contraction then takes.
  auto scale_a = [&](bf16x8_t (&af)[FM], int kt, int s) SMOE_INL {
    if constexpr (GATED) {
      const float* gs = gring + (kt % kRing) * 64 + 16 * s + 8 * (lane >> 5);
      const float4 g0 = *reinterpret_cast<const float4*>(gs);
      const float4 g1 = *reinterpret_cast<const float4*>(gs + 4);
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      static_for<FM>([&](auto fm) SMOE_INL {
        const uint4 w = __builtin_bit_cast(uint4, af[fm]);
        const uint32_t in[4] = {w.x, w.y, w.z, w.w};
        uint32_t o[4];
        static_for<4>([&](auto q) SMOE_INL {
          const float lo = __uint_as_float(in[q] << 16) * gv[2 * int(q)];
          const float hi = __uint_as_float(in[q] & 0xffff0000u) * gv[2 * int(q) + 1];
          o[q] = pack_bf16x2(lo, hi);
        });
        af[fm] = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
      });
    }
  };
  // fragments of two 16-wide k slices: slot 0 / slot 1
  bf16x8_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto mfma = [&](bf16x8_t (&A)[FM], bf16x8_t (&B)[FN], auto fm, auto fn) SMOE_INL {
    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B[fn], A[fm], acc[fm][fn], 0, 0, 0);
  };
  // One 16-wide k slice in a fixed order: each multiply, then the copies
  // placed after it (cp(I)), then one fragment read of the next slice (slice
  // ns of buffers na / nb), so that the reads and copies run under the
  // multiplies and no copy burst holds them up.
  constexpr int NM = FM * FN;
  auto slice = [&](bf16x8_t (&A)[FM], bf16x8_t (&B)[FN], bf16x8_t (&An)[FM], bf16x8_t (&Bn)[FN], const char* na,
                   const char* nb, int ns, auto cp) SMOE_INL {
    static_for<NM>([&](auto ii) SMOE_INL {
      constexpr int I = decltype(ii)::value;
      mfma(A, B, std::integral_constant<int, I / FN>{}, std::integral_constant<int, I % FN>{});
      cp(std::integral_constant<int, I>{});
      if constexpr (I < FM) An[I] = frag_a(na, std::integral_constant<int, I>{}, ns);
      else if constexpr (I < FM + FN) Bn[I - FM] = frag_b(nb, std::integral_constant<int, I - FM>{}, ns);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (NM < FM + FN) {
      // more fragments than multiplies in the slice (small tiles)
      static_for<FM + FN - NM>([&](auto rr) SMOE_INL {
        constexpr int I = NM + decltype(rr)::value;
        if constexpr (I < FM) An[I] = frag_a(na, std::integral_constant<int, I>{}, ns);
        else Bn[I - FM] = frag_b(nb, std::integral_constant<int, I - FM>{}, ns);
      });
    }
  };

  // Weights mode, slices 0-2 (no copies): the next slice's reads first in
  // program order, then the multiplies, and the scheduler interleaves them,
  // one multiply and a share of the reads at a time.
  constexpr int kFragReads = FM * (ALAY == LAY_K ? 1 : 2) + FN * ((MODE == SEG_M && BLAY == LAY_K) ? 1 : 2);
  auto slice_sched = [&](bf16x8_t (&A)[FM], bf16x8_t (&B)[FN], bf16x8_t (&An)[FM], bf16x8_t (&Bn)[FN],
                         const char* na, const char* nb, int ns) SMOE_INL {
    static_for<FM>([&](auto fm) SMOE_INL { An[fm] = frag_a(na, fm, ns); });
    static_for<FN>([&](auto fn) SMOE_INL { Bn[fn] = frag_b(nb, fn, ns); });
    static_for<FM>([&](auto fm) SMOE_INL { static_for<FN>([&](auto fn) SMOE_INL { mfma(A, B, fm, fn); }); });
    static_for<NM>([&](auto i) SMOE_INL {
      constexpr int r0 = int(i) * kFragReads / NM, r1 = (int(i) + 1) * kFragReads / NM;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(0x100, r1 - r0, 0);
    });
  };

  // ---------------- pipeline -----------------------------------------------
  // Step kt multiplies the four 16-wide slices of stage kt, reading the
  // fragments of slice j+1 while slice j multiplies.  Before the last slice
  // (whose fragments are then in registers) each wave waits until its LDS
  // reads are done and its copies of stage kt+1 have landed; one barrier per
  // step then publishes stage kt+1 and frees the buffers of stage kt.  The
  // last slice reads stage kt+1's first slice.  Rows mode: the A copies of
  // stage kt+2 go into the third A buffer during slices 0-2 (two steps to
  // land), the B copies of stage kt+2 into the freed B buffer during the
  // last slice (one step to land).  Weights mode: both operands' copies of
  // stage kt+2 go into the freed buffers during the last slice.
  if constexpr (MODE == SEG_K) {
    for (int j = 0; j < kIdxAhead; ++j)
      if (j < KT) idx_copy(j);
    wait_vmem<0>();
    asm volatile("s_barrier" ::: "memory");
    idx_fetch(0);
  }
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  constexpr std::false_type kMasked{};
  // step forms: general; steady rows mode; steady weights mode with the B
  // operand gathered (form 2, A gathered, is not instantiated)
  constexpr std::integral_constant<int, 0> kGeneral{};
  constexpr std::integral_constant<int, 1> kSteady{};
  constexpr std::integral_constant<int, 3> kSteadyGB{};
  planA(0);
  static_for<NA>([&](auto c) SMOE_INL { copyA(c, abuf(I0{}), kMasked); });
  planB(0);
  static_for<NB>([&](auto c) SMOE_INL { copyB(c, bbuf(I0{}), kMasked); });
  if (1 < KT) {
    idx_fetch(1);
    planA(1);
    static_for<NA>([&](auto c) SMOE_INL { copyA(c, abuf(I1{}), kMasked); });
    planB(1);
    static_for<NB>([&](auto c) SMOE_INL { copyB(c, bbuf(I1{}), kMasked); });
    wait_vmem<LPS>();
  } else {
    wait_vmem<0>();
  }
  asm volatile("s_barrier" ::: "memory");
  if (2 < KT) idx_fetch(2);
  static_for<FM>([&](auto fm) SMOE_INL { fa0[fm] = frag_a(abuf(I0{}), fm, 0); });
  static_for<FN>([&](auto fn) SMOE_INL { fb0[fn] = frag_b(bbuf(I0{}), fn, 0); });
  static_assert(kNSL == 4, "four slices per stage");
  // One step kt (s = kt mod UNROLL picks the buffers).  STEADY (rows mode,
  // K parts whole multiples of the step, and stage kt+2 inside the
  // reduction): no masking and no per-copy conditions.
  auto step = [&](auto s, const int kt, auto form, const bool more_rt) SMOE_INL {
        constexpr int SC = decltype(form)::value;
        constexpr bool STEADY = SC != 0;
        // copies of A from the lanes' base offsets: steady rows mode, and
        // steady weights mode with a plain A
        constexpr std::integral_constant<bool, SC == 1 || SC == 3> a_base{};
        constexpr std::integral_constant<bool, SC == 1> b_base{};
        using S1 = std::integral_constant<int, int(s) + 1>;
        using S2 = std::integral_constant<int, int(s) + 2>;
        const char* ca = abuf(s);
        const char* cb = bbuf(s);
        const char* na = abuf(S1{});
        const char* nb = bbuf(S1{});
        const bool more = STEADY || more_rt;
        // rows mode: A copies of stage kt+2, spread over slices 0-2
        if constexpr (A3) {
          if constexpr (STEADY) planA_steady(kt + 2);
          else if (more) planA(kt + 2);
        }
        auto acp = [&](auto sl) SMOE_INL {
          return [&](auto ii) SMOE_INL {
            if constexpr (A3) {
              constexpr int I = decltype(ii)::value;
              static_for<NA>([&](auto cc) SMOE_INL {
                constexpr int c = decltype(cc)::value, pos = c * 3 * NM / NA;
                if constexpr (pos / NM == decltype(sl)::value && pos % NM == I) {
                  if (more) copyA(cc, abuf(S2{}), a_base);
                }
              });
            }
          };
        };
        if constexpr (A3) {
          slice(fa0, fb0, fa1, fb1, ca, cb, 1, acp(std::integral_constant<int, 0>{}));
          slice(fa1, fb1, fa0, fb0, ca, cb, 2, acp(std::integral_constant<int, 1>{}));
          slice(fa0, fb0, fa1, fb1, ca, cb, 3, acp(std::integral_constant<int, 2>{}));
        } else {
          // weights mode: the B copies of stage kt+1 (planned in step kt-1,
          // into the B buffer that step freed) go first, apart from the A
          // copies issued in step kt-1's last slice
          if (KSPLIT && kt >= 1 && kt + 1 < KT) {
            static_for<NB>([&](auto cc) SMOE_INL { copyB(cc, bbuf(S1{}), kMasked); });
          }
          scale_a(fa0, kt, 0);
          slice_sched(fa0, fb0, fa1, fb1, ca, cb, 1);
          scale_a(fa1, kt, 1);
          slice_sched(fa1, fb1, fa0, fb0, ca, cb, 2);
          scale_a(fa0, kt, 2);
          slice_sched(fa0, fb0, fa1, fb1, ca, cb, 3);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SC == 1) {
          planB_steady(kt + 2);
        } else if constexpr (SC == 3) {
          planA_k(kt + 2, std::false_type{});
          planB_k(kt + 2, std::true_type{});
        } else if (more) {
          if constexpr (!A3) planA(kt + 2);
          planB(kt + 2);
        }
        wait_lds();
        // stage kt+1 must have landed; rows mode: this step's A copies of
        // stage kt+2 (the last issued) may still be in flight
        if (A3 && more) wait_vmem<A3 ? NA : 0>();
        else wait_vmem<0>();
        asm volatile("s_barrier" ::: "memory");
        if constexpr (MODE == SEG_K) {
          if (kt + kIdxAhead < KT) idx_copy(kt + kIdxAhead);
        }
        scale_a(fa1, kt, 3);
        __builtin_amdgcn_sched_barrier(0);
        // last slice: the copies of stage kt+2 into this step's freed buffers
        constexpr int LC = A3 ? NB : (KSPLIT ? NA : NA + NB);
        auto lcp = [&](auto ii) SMOE_INL {
          constexpr int I = decltype(ii)::value;
          static_for<LC>([&](auto cc) SMOE_INL {
            constexpr int c = decltype(cc)::value;
            if constexpr (c * NM / LC == I) {
              if (more) {
                if constexpr (A3) copyB(cc, bbuf(s), b_base);
                else if constexpr (c < NA) copyA(cc, abuf(s), a_base);
                else copyB(std::integral_constant<int, c - NA>{}, bbuf(s), kMasked);
              }
            }
          });
        };
        slice(fa1, fb1, fa0, fb0, na, nb, 0, lcp);
        if constexpr (MODE == SEG_K) {
          if (kt + 3 < KT) idx_fetch_of(kt + 3, std::integral_constant<bool, SC != 3>{}, std::integral_constant<bool, SC != 2>{});
        }
  };
  int k0 = 0;
  if constexpr (MODE == SEG_M) {
    if (K0 % kBK == 0 && K1 % kBK == 0) {
      for (; k0 + UNROLL + 2 <= KT; k0 += UNROLL)
        static_for<UNROLL>([&](auto s) SMOE_INL { step(s, k0 + int(s), kSteady, true); });
    }
  } else if constexpr (!GATED) {
    // steady while stage kt+2 holds 64 rows of the chunk, for a plain A and
    // a gathered B (the W2 weight gradient over the upstream gradient).  A
    // gathered A (the weight gradients over x) takes the general form: its
    // steady form measured 7 % slower (the extra registers it holds push an
    // LDS address into scratch, and the reload before the loop costs a
    // wait for every copy in flight on each pass)
    const int KTF = K0 / kBK;
    if (!p.a_scat && p.b_scat) {
      for (; k0 + UNROLL + 2 <= KTF; k0 += UNROLL)
        static_for<UNROLL>([&](auto s) SMOE_INL { step(s, k0 + int(s), kSteadyGB, true); });
    }
  }
  for (; k0 < KT; k0 += UNROLL) {
    static_for<UNROLL>([&](auto s) SMOE_INL {
      const int kt = k0 + int(s);
      if (kt < KT) step(s, kt, kGeneral, kt + 2 < KT);
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
  static_assert(NOUT * 32 * RBE <= LDS_BYTES / NW && (LDS_BYTES / NW) % 16 == 0, "staging slot");
  asm volatile("s_barrier" ::: "memory");
  // each wave stages into its share of the stage buffers
  char* const slot = lds + wave * (LDS_BYTES / NW);
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
  // staged output o -> global: row j (0..31) of the fragment row goes to
  // base + rowoff(j) + colbase, or nowhere when rowoff(j) < 0.
  // ADD: fp32 atomic adds of the four values instead of one store (the
  // fused combine; several assignments add into one token's row)
  auto flush = [&](int o, ST* base, auto rowoff, int colbase, auto add) SMOE_INL {
    static_for<32 / RPR>([&](auto i) SMOE_INL {
      const int j = int(i) * RPR + lane / CH, c = lane % CH;
      const uint4 d = *reinterpret_cast<const uint4*>(slot + o * 32 * RBE + j * RBE + ((c ^ (j & (CH - 1))) << 4));
      const int64_t ro = rowoff(j);
      const int colc = colbase + c * (16 / OB);
      if (ro >= 0 && colc < p.N) {
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
  // row offsets for flush: rows first + j of a dense range (stored below
  // end), computed by every lane; or rows held by the lanes of the fragment
  // row (lane j: row j, or -1), fetched with one shuffle
  auto dense_rows = [](int64_t first, int64_t end, int64_t ld) SMOE_INL {
    return [=](int j) SMOE_INL -> int64_t { return first + j < end ? (first + j) * ld : int64_t(-1); };
  };
  auto held_rows = [](int held, int64_t ld) SMOE_INL {
    return [=](int j) SMOE_INL -> int64_t {
      const int r = __shfl(held, j, kWave);
      return r >= 0 ? int64_t(r) * ld : int64_t(-1);
    };
  };
  constexpr std::false_type kStore{};
  constexpr std::true_type kAdd{};

  if constexpr (MODE == SEG_K) {
    float* dst = (it.nitems == 1 && !p.dw_all_partial) ? static_cast<float*>(p.c0) + int64_t(it.e) * p.Mo * p.N
                                                       : p.partial + int64_t(T.chunk) * p.Mo * p.N;
    static_for<FM>([&](auto fm) SMOE_INL {
      static_for<FN>([&](auto fn) SMOE_INL {
        static_for<4>([&](auto q) SMOE_INL {
          const float v[4] = {acc[fm][fn][4 * int(q)], acc[fm][fn][4 * int(q) + 1],
                              acc[fm][fn][4 * int(q) + 2], acc[fm][fn][4 * int(q) + 3]};
          put(0, fn, q, v);
        });
      });
      flush(0, dst, dense_rows(T.m0 + wm * WM + fm * 32, p.Mo, p.N), T.n0 + wn * WN, kStore);
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
    const int hh = lane >> 5;   // the half of the chunk pair a lane reads
    // 4 waves: twice the columns per lane, so one buffer (the accumulators
    // already fill the AGPRs)
    constexpr int NBUF = NW == 4 ? 1 : 2;
    uint4 rx0[NBUF][FNR][2], rx1[NBUF][AUX1 ? FNR : 1][2];
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
    // the lane's 4 values of chunk q of fragment fn from the 16-byte reads:
    // lane l < 32 keeps the low halves of its reads and takes the low halves
    // of lane l + 32's; lane l >= 32 keeps its high halves and takes lane
    // l - 32's.  gfx950's v_permlane32_swap exchanges the upper 32 lanes of
    // one register with the lower 32 lanes of another, which is exactly
    // that (a VALU operation, no LDS round trip).
    auto aux_vals = [&](uint4 (&rx)[2], uint2 (&ax)[4]) SMOE_INL {
      static_for<2>([&](auto j) SMOE_INL {
        const auto sx = __builtin_amdgcn_permlane32_swap(rx[j].x, rx[j].z, false, false);
        const auto sy = __builtin_amdgcn_permlane32_swap(rx[j].y, rx[j].w, false, false);
        ax[int(j)] = make_uint2(sx[0], sy[0]);
        ax[2 + int(j)] = make_uint2(sx[1], sy[1]);
      });
    };
    auto unpack = [&](uint2 w, float v[4]) SMOE_INL { unpack4_bf16(w, v); };
    if constexpr (NBUF == 2) load_aux(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    static_for<FM>([&](auto fm) SMOE_INL {
      constexpr int BUF = int(fm) % NBUF;
      if constexpr (NBUF == 1) load_aux(fm, std::integral_constant<int, 0>{});
      else if constexpr (int(fm) + 1 < FM)
        load_aux(std::integral_constant<int, int(fm) + 1>{}, std::integral_constant<int, BUF ^ 1>{});
      const int rowbase = it.row0 + wm * WM + fm * 32;   // grouped row of lane 0 of the fragment row
      float dgacc = 0.f;
      static_for<FNR>([&](auto fn) SMOE_INL {
        uint2 ax0[4], ax1[4];
        if constexpr (AUX0) {
          if (aux0_on) aux_vals(rx0[BUF][fn], ax0);
        }
        if constexpr (AUX1) aux_vals(rx1[BUF][fn], ax1);
        // every lane computes all of its chunks (rows and columns outside
        // the tile's valid range compute on in-range data that is never
        // stored); only the gate-gradient sums leave out columns past N
        static_for<4>([&](auto q) SMOE_INL {
          const bool cok = col(fn, q) < p.N;
          {
            float v[4] = {acc[fm][fn][4 * int(q)], acc[fm][fn][4 * int(q) + 1], acc[fm][fn][4 * int(q) + 2],
                          acc[fm][fn][4 * int(q) + 3]};
            if constexpr (EPI == EPI_STORE) {
              if (p.dgpart) {
                float xv[4];
                unpack(ax0[q], xv);
                const float dot = xv[0] * v[0] + xv[1] * v[1] + xv[2] * v[2] + xv[3] * v[3];
                dgacc += cok ? dot : 0.f;
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
              float dot = 0.f;
              static_for<4>([&](auto i) SMOE_INL {
                dot += a[i] * v[i];
                dh[i] = g[fm] * v[i] * gelu_grad_f(h[i]);
                ag[i] = g[fm] * a[i];
              });
              dgacc += cok ? dot : 0.f;
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
              float dot = 0.f;
              static_for<4>([&](auto i) SMOE_INL {
                dot += a[i] * v[i];
                const float dA = g[fm] * v[i];
                d1[i] = dA * h3[i] * (sg[i] * (1.0f + h1[i] * (1.0f - sg[i])));
                d3[i] = dA * si[i];
                ag[i] = g[fm] * a[i];
              });
              dgacc += cok ? dot : 0.f;
              put(0, fn, q, d1);
              put(1, fn, q, d3);
              put(2, fn, q, ag);
            }
          }
        });
      });
      if (p.dgpart) {
        // lane l < 32 adds lane l + 32's partial sum of the same row
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dgacc), __float_as_uint(dgacc), false, false);
        dgacc += __uint_as_float(sw[1]);
        if (lane < 32 && rok[fm]) p.dgpart[int64_t(T.nt * WGN + wn) * p.M + gr[fm]] = dgacc;
      }
      // staged rows -> global (grouped rows, or scattered for EPI_STORE)
      const int cb = T.n0 + (DUAL ? wn * (WN / 2) : wn * WN);
      const auto grouped = dense_rows(rowbase, it.row1, p.ldc);
      if constexpr (EPI == EPI_STORE) {
        if (c0) {
          if (p.c_scat || p.c_add_fan > 0) {
            int hr = p.c_scat ? sp[fm] : gr[fm];
            if (p.c_add_fan > 0) hr /= p.c_add_fan;
            const auto rows = held_rows(rok[fm] ? hr : -1, p.ldc);
            if (p.c_add_fan > 0) flush(0, c0, rows, cb, kAdd);
            else flush(0, c0, rows, cb, kStore);
          } else {
            flush(0, c0, grouped, cb, kStore);
          }
        }
      } else if constexpr (EPI == EPI_GELU_FWD) {
        flush(0, c0, grouped, cb, kStore);
        flush(1, c1, grouped, cb, kStore);
      } else if constexpr (EPI == EPI_SWIGLU_FWD) {
        flush(0, c0, grouped, cb, kStore);
        flush(1, c1, grouped, cb, kStore);
        flush(2, c2, grouped, cb, kStore);
      } else if constexpr (EPI == EPI_GELU_BWD) {
        flush(0, c0, grouped, cb, kStore);
        flush(1, c2, grouped, cb, kStore);
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        flush(0, c0, grouped, cb, kStore);
        flush(1, c1, grouped, cb, kStore);
        flush(2, c2, grouped, cb, kStore);
      }
    });
  }
}


// ---------------------------------------------------------------------------
// instance launch (each group of instances lives in its own source file, so
// that the groups compile in parallel)
// ---------------------------------------------------------------------------
template <int BM, int BN, int MODE, int EPI, int BLAY, bool DUAL, class OutT>
inline void go_bf16(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if constexpr (BM == 256 && BN == 256 && MODE == SEG_M) {
    if (pl.nw == 4) {
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 4, MODE, EPI, BLAY, DUAL, OutT>), dim3(unsigned(pl.grid)),
                         dim3(256), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 8, MODE, EPI, BLAY, DUAL, OutT>), dim3(unsigned(pl.grid)),
                     dim3(kThreads), 0, st, a);
}

template <int MODE, int EPI, int BLAY, bool DUAL, class OutT>
inline bool dispatch_tiles(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
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

// one function per group of kernel instances (gemm_*.hip)
bool dispatch_bf16_store_k(const GemmArgs& a, const GemmPlan& pl, int out_f32, hipStream_t st);
bool dispatch_bf16_store_mn(const GemmArgs& a, const GemmPlan& pl, int out_f32, hipStream_t st);
bool dispatch_bf16_act_fwd(const GemmArgs& a, const GemmPlan& pl, hipStream_t st);
bool dispatch_bf16_act_bwd(const GemmArgs& a, const GemmPlan& pl, hipStream_t st);
bool dispatch_bf16_dw(const GemmArgs& a, const GemmPlan& pl, hipStream_t st);

}  // namespace smoe
