// Routing-index kernels: expert choices [T,k] -> per-expert histogram,
// exclusive prefix sum (offsets) and a stable counting-sort scatter giving
// sorted_scattered_idxs / sorted_expert_idxs (the reordering that
// ParallelLinear fuses with the expert transforms: ScatterMoE project page,
// "How It Works").
//
// Three launches, no host synchronisation:
//  1. route_hist    : one workgroup per chunk of kChunk assignments builds a
//                     chunk histogram in LDS -> blk[e * nb + b].
//  2. route_scan    : one workgroup scans blk in expert-major order, so
//                     blk[e*nb+b] becomes the first output row of chunk b's
//                     expert-e elements; writes offsets and counts.
//  3. route_scatter : each chunk ranks its elements among equal experts with
//                     wave64 ballots (match by bit planes of the expert id),
//                     in ascending p, and writes them at their final rows.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace smoe {

constexpr int kRouteThreads = 256;
constexpr int kRounds = 16;
constexpr int kChunk = kRouteThreads * kRounds;  // 4096 assignments per chunk

__global__ __launch_bounds__(kRouteThreads) void route_hist(const int* __restrict__ eidx, int M, int E,
                                                            int nb, int* __restrict__ blk) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = 0; i < kRounds; ++i) {
    const int p = base + i * kRouteThreads + threadIdx.x;
    if (p < M) {
      const int e = eidx[p];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) blk[(size_t)e * nb + blockIdx.x] = hist[e];
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void route_scan(int* __restrict__ blk, int n, int E, int nb,
                                                           int* __restrict__ offsets, int* __restrict__ counts) {
  __shared__ int wsum[kScanThreads / kWave];
  __shared__ int total_s;
  const int tid = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += blk[i];
  // block exclusive scan of the per-thread sums
  const int incl = wave_incl_scan(s);
  const int w = tid / kWave;
  if (lane_id() == kWave - 1) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    int v = lane_id() < kScanThreads / kWave ? wsum[lane_id()] : 0;
    int vi = wave_incl_scan(v);
    if (lane_id() < kScanThreads / kWave) wsum[lane_id()] = vi - v;
    if (lane_id() == kScanThreads / kWave - 1) total_s = vi;
  }
  __syncthreads();
  int run = wsum[w] + incl - s;
  for (int i = lo; i < hi; ++i) {
    const int c = blk[i];
    blk[i] = run;
    run += c;
  }
  __syncthreads();
  // offsets[e] = first row of expert e = scanned value of (e, chunk 0)
  for (int e = tid; e <= E; e += kScanThreads) {
    const int o = (e < E) ? (nb > 0 ? blk[(size_t)e * nb] : 0) : total_s;
    offsets[e] = o;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kScanThreads) {
    const int nxt = (e + 1 < E) ? (nb > 0 ? blk[(size_t)(e + 1) * nb] : 0) : total_s;
    counts[e] = nxt - offsets[e];
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter(const int* __restrict__ eidx, int M, int E, int nb,
                                                               const int* __restrict__ blk, int* __restrict__ s_exp,
                                                               int* __restrict__ s_sct) {
  constexpr int kWaves = kRouteThreads / kWave;
  __shared__ int run[kMaxExperts + 1];
  __shared__ int wcnt[kWaves][kMaxExperts + 1];
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  for (int e = tid; e < E; e += kRouteThreads) run[e] = blk[(size_t)e * nb + blockIdx.x];
  for (int i = tid; i < kWaves * (kMaxExperts + 1); i += kRouteThreads) (&wcnt[0][0])[i] = 0;
  // bits needed to tell apart keys 0..E (key E marks "no element")
  const int nbits = 32 - __clz(E);
  const unsigned long long lt = (l == 0) ? 0ull : (~0ull >> (kWave - l));
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = 0; i < kRounds; ++i) {
    const int p = base + i * kRouteThreads + tid;
    int key = E;
    if (p < M) {
      const int e = eidx[p];
      if (e >= 0 && e < E) key = e;
    }
    unsigned long long same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const unsigned long long m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lt);
    const bool leader = rank == 0;
    if (leader && key < E) wcnt[w][key] = __popcll(same);
    __syncthreads();
    if (key < E) {
      int pos = run[key] + rank;
      for (int v = 0; v < w; ++v) pos += wcnt[v][key];
      s_sct[pos] = p;
      s_exp[pos] = key;
    }
    __syncthreads();
    // every position of this round is written: advance the running rows by
    // this round's counts and clear them for the next round
    if (leader && key < E) {
      atomicAdd(&run[key], wcnt[w][key]);
      wcnt[w][key] = 0;
    }
    __syncthreads();
  }
}

// Scratch of the allocation-free routing entry point (smoe_route_noalloc):
// the chunk histograms live in this device-resident array instead of a
// caller workspace.  Each device the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (in host code it is a stand-in, not a device address): it asks
// for the device address once per device and uses that.
constexpr size_t kRouteScratchInts = size_t(1) << 20;   // 4 MiB
static __device__ __align__(256) int scratch[kRouteScratchInts];

hipError_t route_static_scratch(int** ptr, size_t* ints) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<int*>(p);
  }
  *ptr = addr[dev];
  *ints = kRouteScratchInts;
  return hipSuccess;
}

size_t route_static_scratch_ints() { return kRouteScratchInts; }

size_t route_ws_bytes(int64_t M, int E) {
  const int64_t nb = (M + kChunk - 1) / kChunk;
  return size_t(std::max<int64_t>(nb * E, 1)) * sizeof(int);
}

hipError_t launch_route(const int* eidx, int M, int E, int* s_exp, int* s_sct, int* counts, int* offsets, void* ws,
                        hipStream_t st) {
  const int nb = (M + kChunk - 1) / kChunk;
  int* blk = static_cast<int*>(ws);
  if (nb > 0) hipLaunchKernelGGL(route_hist, dim3(nb), dim3(kRouteThreads), 0, st, eidx, M, E, nb, blk);
  hipLaunchKernelGGL(route_scan, dim3(1), dim3(kScanThreads), 0, st, blk, nb * E, E, nb, offsets, counts);
  if (nb > 0)
    hipLaunchKernelGGL(route_scatter, dim3(nb), dim3(kRouteThreads), 0, st, eidx, M, E, nb, blk, s_exp, s_sct);
  return hipGetLastError();
}

}  // namespace smoe
