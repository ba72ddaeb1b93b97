// Launches of the SSD forward for 128-token chunks (kernels in ssd_fwd_impl.h).
#include "ssd_fwd_impl.h"

namespace ssd_fwd_impl {

ssd_status launch_q128(const Params &prm, const Plan &pl, hipStream_t s, const ssd_desc *d) {
  return dispatch_n<128>(prm, pl, s, d);
}

}  // namespace ssd_fwd_impl
