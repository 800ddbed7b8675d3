// fa_fwd_d80.hip - the forward kernels of key head dim 80 (value head dims
// 80), in a translation unit of their own so that they build in
// parallel with the others.
#include "fa_fwd_kernel.h"

namespace fa_fwd_detail {

hipError_t dispatch_d80(const FwdArgs& a, int dv, bool causal, bool window, int mask,
                        int n_short, hipStream_t stream) {
  switch (dv) {
    case 80: return dispatch_d<80, 80>(a, causal, window, mask, n_short, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa_fwd_detail
