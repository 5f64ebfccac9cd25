// Device scratch of the decode entry point that allocates nothing
// (spark_attn_decode_noalloc): a static device array, which every GPU the library runs on
// holds from the library's load until the process ends.  On the host, `scratch` names a
// host-side stand-in, not device memory: its device address is looked up once per device,
// with that device current, and only that address is handed to kernels.
#include "spark_launch.hpp"

#include <mutex>

namespace spark {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};   // device address of `scratch`, per device id

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace spark
