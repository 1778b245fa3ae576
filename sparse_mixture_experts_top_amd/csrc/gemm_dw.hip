// Instances of the bf16 grouped-product kernel (gemm_kernel.h) for
// the weight gradients (groupXtY, weights mode), plain or with per-row gate scales.
#include "gemm_kernel.h"

namespace smoe {

bool dispatch_bf16_dw(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if (a.kscale) return dispatch_tiles<SEG_K, EPI_PARTIAL_GATED, LAY_MN, false, float>(a, pl, st);
  return dispatch_tiles<SEG_K, EPI_PARTIAL, LAY_MN, false, float>(a, pl, st);
}

}  // namespace smoe
