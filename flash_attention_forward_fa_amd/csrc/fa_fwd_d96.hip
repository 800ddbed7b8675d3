// fa_fwd_d96.hip - the forward kernels of key head dim 96 (value head dims
// 96, 64), in a translation unit of their own so that they build in
// parallel with the others.
#include "fa_fwd_kernel.h"

namespace fa_fwd_detail {

hipError_t dispatch_d96(const FwdArgs& a, int dv, bool causal, bool window, int mask,
                        int n_short, hipStream_t stream) {
  switch (dv) {
    case 96: return dispatch_d<96, 96>(a, causal, window, mask, n_short, stream);
    case 64: return dispatch_d<96, 64>(a, causal, window, mask, n_short, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa_fwd_detail
