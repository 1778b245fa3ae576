// Instances of the bf16 grouped-product kernel (gemm_kernel.h) for
// the MLP's dA product with the activation backward, the gate-gradient partials and g a.
#include "gemm_kernel.h"

namespace smoe {

bool dispatch_bf16_act_bwd(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if (pl.epi == EPI_SWIGLU_BWD) return dispatch_tiles<SEG_M, EPI_SWIGLU_BWD, LAY_K, false, uint16_t>(a, pl, st);
  return dispatch_tiles<SEG_M, EPI_GELU_BWD, LAY_K, false, uint16_t>(a, pl, st);
}

}  // namespace smoe
