// Scratch memory of kvq_decode_attention_noalloc, the decode entry point
// that allocates nothing: one fixed device array, `scratch`, which every GPU
// the library runs on holds until the process ends.  The decode carves its
// prepared queries and split partials out of it instead of a caller-owned
// workspace.  Its device address is looked up once per GPU, with that GPU
// current, on the entry point's first call there; host code uses only that
// address, never the array's name (on the host the name is a stand-in, not
// a device address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq.h"
#include "kvq_launch.h"

namespace kvq {

static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];     // device address of `scratch` per GPU, once looked up
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kvq
