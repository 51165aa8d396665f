// Launch entry points for the host-only sanitizer build of the C ABI: the
// validation layer (api.cpp) and the split planning are compiled with
// AddressSanitizer and UndefinedBehaviorSanitizer and linked against these
// stand-ins, which report that no device is present.  The CPU tests that
// run against this build never reach a launch with valid arguments.
#include "kvq_launch.h"

namespace kvq {

hipError_t launch_quantize_rows(const QuantArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quantize_dense(const QuantArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quantize_grouped(const QuantArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void **) { return hipErrorNoDevice; }

}  // namespace kvq
