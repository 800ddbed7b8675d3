// fa_fwd_d192.hip - the forward kernels of key head dim 192 (value head dims
// 192, 128), in a translation unit of their own so that they build in
// parallel with the others.
#include "fa_fwd_kernel.h"

namespace fa_fwd_detail {

hipError_t dispatch_d192(const FwdArgs& a, int dv, bool causal, bool window, int mask,
                         int n_short, hipStream_t stream) {
  switch (dv) {
    case 192: return dispatch_d<192, 192>(a, causal, window, mask, n_short, stream);
    case 128: return dispatch_d<192, 128>(a, causal, window, mask, n_short, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa_fwd_detail
