// Instances of the bf16 grouped-product kernel (gemm_kernel.h) for
// the MLP's first layer with its activation (GELU; SwiGLU with W1 and W3 sharing the A tile).
#include "gemm_kernel.h"

namespace smoe {

bool dispatch_bf16_act_fwd(const GemmArgs& a, const GemmPlan& pl, hipStream_t st) {
  if (pl.epi == EPI_SWIGLU_FWD) return dispatch_tiles<SEG_M, EPI_SWIGLU_FWD, LAY_MN, true, uint16_t>(a, pl, st);
  return dispatch_tiles<SEG_M, EPI_GELU_FWD, LAY_MN, false, uint16_t>(a, pl, st);
}

}  // namespace smoe
