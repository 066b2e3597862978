// launch_stubs.cpp -- host-only stand-ins for the kernel launchers, so that the host API can be
// linked and run under AddressSanitizer / UndefinedBehaviorSanitizer without compiling the
// kernels.  Every stand-in reports "no device": a call that passes validation stops at device
// set-up and launches nothing.
#include "sfag_launch.h"

namespace sfag {

hipError_t launch_fwd(const FwdArgs&, int64_t, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_q(const BwdArgs&, int64_t, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_pair_chunk(const PairArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t set_q_attributes() { return hipErrorNoDevice; }
hipError_t launch_sort_rows(const DenseArgs&, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_item_list(const DenseArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_dense(const DenseArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_reduce(const DenseArgs&, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t set_dense_attributes() { return hipErrorNoDevice; }
hipError_t set_fwd_attributes() { return hipErrorNoDevice; }
hipError_t launch_indexer(const IxArgs&, int64_t, hipStream_t) { return hipErrorNoDevice; }

}  // namespace sfag
