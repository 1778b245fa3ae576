// Device helpers shared by the gfx950 kernels: bf16 bit conversions, wave64
// scans and the data-dependent tile maps that turn per-expert row counts
// into grouped-GEMM tiles without a device-to-host copy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#define SMOE_DEV __device__ __forceinline__
// for lambdas in kernels: keep every helper inlined so register arrays they
// index stay in registers
#define SMOE_INL __attribute__((always_inline))

namespace smoe {

constexpr int kWave = 64;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1, so
// register arrays indexed by i stay in registers whatever the body size.
template <class F, int... I>
SMOE_DEV void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
SMOE_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---- bf16 <-> fp32 --------------------------------------------------------
// fp32 -> bf16 is gfx950's v_cvt_pk_bf16_f32 (round to nearest even, NaN
// quieted), two values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
SMOE_DEV float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
// {lo, hi} -> one dword holding bf16(lo) | bf16(hi) << 16
SMOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
SMOE_DEV uint16_t f2bf(float f) { return uint16_t(pack_bf16x2(f, 0.f)); }
// round to bf16 and back (the value a bf16 store would hold)
SMOE_DEV float bfround(float f) { return bf2f(f2bf(f)); }

// element load/store of the two storage types
template <class T> SMOE_DEV float ld(const T* p);
template <> SMOE_DEV float ld<float>(const float* p) { return *p; }
template <> SMOE_DEV float ld<uint16_t>(const uint16_t* p) { return bf2f(*p); }
template <class T> SMOE_DEV void st(T* p, float v);
template <> SMOE_DEV void st<float>(float* p, float v) { *p = v; }
template <> SMOE_DEV void st<uint16_t>(uint16_t* p, float v) { *p = f2bf(v); }
// value as stored by type T (rounding for bf16, identity for fp32)
template <class T> SMOE_DEV float stored(float v);
template <> SMOE_DEV float stored<float>(float v) { return v; }
template <> SMOE_DEV float stored<uint16_t>(float v) { return bfround(v); }

// four consecutive elements
template <class T> SMOE_DEV void st4(T* p, const float v[4]);
template <> SMOE_DEV void st4<float>(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> SMOE_DEV void st4<uint16_t>(uint16_t* p, const float v[4]) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = w;
}
// four values <-> two dwords of bf16
SMOE_DEV uint2 pack4_bf16(const float v[4]) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  return w;
}
SMOE_DEV void unpack4_bf16(uint2 w, float v[4]) {
  v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
}
template <class T> SMOE_DEV void ld4(const T* p, float v[4]);
template <> SMOE_DEV void ld4<float>(const float* p, float v[4]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
template <> SMOE_DEV void ld4<uint16_t>(const uint16_t* p, float v[4]) {
  uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
}

// ---- activations (fp32) ---------------------------------------------------
// Standard normal CDF Phi(z) = (1 + erf(z / sqrt 2)) / 2 and e = exp(-z^2/2)
// (the density's exponential, shared with GELU's derivative).  erf comes
// from Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// for x >= 0, 1 - erf(x) = (a1 t + ... + a5 t^5) exp(-x^2), t = 1/(1 + p x),
// absolute error at most 1.5e-7.  With x = |z|/sqrt 2, exp(-x^2) is e, and
// the lower tail Phi(-|z|) = (1 - erf(x)) / 2 is formed directly (no
// cancellation against 1).
SMOE_DEV void normal_cdf(float z, float& phi, float& e) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * x);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  e = __expf(-0.5f * z * z);
  const float tail = 0.5f * poly * e;   // Phi(-|z|)
  phi = z >= 0.0f ? 1.0f - tail : tail;
}
// GELU with the exact (erf) form, z Phi(z), and its derivative
// Phi(z) + z phi(z), phi(z) = e / sqrt(2 pi)
SMOE_DEV float gelu_f(float z) {
  float phi, e;
  normal_cdf(z, phi, e);
  return z * phi;
}
SMOE_DEV float gelu_grad_f(float z) {
  float phi, e;
  normal_cdf(z, phi, e);
  return phi + z * 0.39894228040143268f * e;
}
// 1 / (1 + e^-z) with the hardware reciprocal (about 1 ulp) instead of an
// IEEE division; e^-z = +inf gives 0, e^-z = 0 gives 1
SMOE_DEV float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
SMOE_DEV float silu_f(float z) { return z * sigmoid_f(z); }
SMOE_DEV float silu_grad_f(float z) {
  float s = sigmoid_f(z);
  return s * (1.0f + z * (1.0f - s));
}

// ---- wave64 helpers ------------------------------------------------------
SMOE_DEV int lane_id() { return __lane_id(); }
SMOE_DEV int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}

// ---- tile maps ------------------------------------------------------------
// Rows of expert e are [offsets[e], offsets[e+1]).  Expert e owns
// ceil(count_e / unit) consecutive work items (m-tiles, or row chunks for
// the weight gradient).  find_item() maps a global item index to its expert
// and row range; every lane of the calling wave gets the same answer.
// Returns false if `item` is past the last item.
struct Item {
  int e;
  int row0;    // first grouped row of the item
  int row1;    // one past the last row of the item
  int first;   // 1 if this is the expert's first item
  int nitems;  // items of this expert
};

// Item `item` from the lanes' per-expert values (expert c + lane: rows
// [lo, hi), n items, excl items before it in the chunk of 64 experts that
// starts at item index base); false if no lane holds it.
SMOE_DEV bool item_of_lanes(int c, int E, int unit, int item, int base, int lo, int hi, int n, int excl, Item& it) {
  const int e = c + lane_id();
  const bool hit = (e < E) && item >= base + excl && item < base + excl + n;
  const unsigned long long m = __ballot(hit);
  if (!m) return false;
  const int src = __ffsll((long long)m) - 1;
  const int ex = __shfl(excl, src, kWave);
  const int lo_s = __shfl(lo, src, kWave);
  const int hi_s = __shfl(hi, src, kWave);
  const int n_s = __shfl(n, src, kWave);
  const int local = item - base - ex;
  // the same on every lane: make that visible to the compiler, so that
  // values derived from the item (buffer descriptors, loop bounds) live in
  // scalar registers
  it.e = __builtin_amdgcn_readfirstlane(c + src);
  it.row0 = __builtin_amdgcn_readfirstlane(lo_s + local * unit);
  it.row1 = __builtin_amdgcn_readfirstlane(min(hi_s, lo_s + local * unit + unit));
  it.first = __builtin_amdgcn_readfirstlane(local == 0);
  it.nitems = __builtin_amdgcn_readfirstlane(n_s);
  return true;
}

SMOE_DEV bool find_item(const int* __restrict__ offsets, int E, int unit, int item, Item& it) {
  const int l = lane_id();
  int base = 0;
  for (int c = 0; c < E; c += kWave) {
    const int e = c + l;
    int lo = 0, hi = 0;
    if (e < E) { lo = offsets[e]; hi = offsets[e + 1]; }
    const int cnt = hi > lo ? hi - lo : 0;
    const int n = (cnt + unit - 1) / unit;
    const int incl = wave_incl_scan(n);
    if (item_of_lanes(c, E, unit, item, base, lo, hi, n, incl - n, it)) return true;
    base += __shfl(incl, kWave - 1, kWave);
  }
  return false;
}

// Up to 64 experts in one pass (one per lane): the offsets are read and
// scanned once for both the item count and the item lookup.
struct ItemScan {
  int lo, hi, n, excl;
  int total;   // items of all experts (wave-uniform)
};
SMOE_DEV ItemScan scan_items(const int* __restrict__ offsets, int E, int unit) {
  const int e = lane_id();
  ItemScan s;
  s.lo = s.hi = 0;
  if (e < E) { s.lo = offsets[e]; s.hi = offsets[e + 1]; }
  const int cnt = s.hi > s.lo ? s.hi - s.lo : 0;
  s.n = (cnt + unit - 1) / unit;
  const int incl = wave_incl_scan(s.n);
  s.excl = incl - s.n;
  s.total = __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));
  return s;
}
SMOE_DEV bool pick_item(const ItemScan& s, int E, int unit, int item, Item& it) {
  return item_of_lanes(0, E, unit, item, 0, s.lo, s.hi, s.n, s.excl, it);
}

// Items of all experts together: the sum over e of ceil(count_e / unit)
// (wave-uniform).
SMOE_DEV int total_items(const int* __restrict__ offsets, int E, int unit) {
  const int l = lane_id();
  int s = 0;
  for (int c = 0; c < E; c += kWave) {
    const int e = c + l;
    if (e < E) {
      const int cnt = offsets[e + 1] - offsets[e];
      s += cnt > 0 ? (cnt + unit - 1) / unit : 0;
    }
  }
  return __builtin_amdgcn_readfirstlane(__shfl(wave_incl_scan(s), kWave - 1, kWave));
}

}  // namespace smoe
