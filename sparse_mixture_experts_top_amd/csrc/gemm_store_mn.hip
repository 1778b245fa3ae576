// Instances of the bf16 grouped-product kernel (gemm_kernel.h) for
// the forward products with a plain store (ParallelLinear, the W2 product of the MLP): EPI_STORE with B read as W[e].
#include "gemm_kernel.h"

namespace smoe {

bool dispatch_bf16_store_mn(const GemmArgs& a, const GemmPlan& pl, int out_f32, hipStream_t st) {
  return out_f32 ? dispatch_tiles<SEG_M, EPI_STORE, LAY_MN, false, float>(a, pl, st)
                 : dispatch_tiles<SEG_M, EPI_STORE, LAY_MN, false, uint16_t>(a, pl, st);
}

}  // namespace smoe
