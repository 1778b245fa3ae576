// Instances of the bf16 grouped-product kernel (gemm_kernel.h) for
// the W^T products (dX of the MLP, dx of ParallelLinear): EPI_STORE with B read as W[e]^T.
#include "gemm_kernel.h"

namespace smoe {

bool dispatch_bf16_store_k(const GemmArgs& a, const GemmPlan& pl, int out_f32, hipStream_t st) {
  return out_f32 ? dispatch_tiles<SEG_M, EPI_STORE, LAY_K, false, float>(a, pl, st)
                 : dispatch_tiles<SEG_M, EPI_STORE, LAY_K, false, uint16_t>(a, pl, st);
}

}  // namespace smoe
