// Dense-rotation write path (MFMA).  Not yet implemented.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

hipError_t launch_quantize_dense(const QuantArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvq
