// The library's own device workspace, for the layout + dispatch call that
// allocates nothing (ep_layout_dispatch_noalloc): a file-scope device array
// that every GPU the library runs on holds from the first use until the
// process ends.
//
// In host code the array's name only stands in for it; its device address
// comes from hipGetSymbolAddress, once per device (with that device
// current), and is kept per device.  Every call on a device shares that
// device's array and leaves its contents to the next call: calls that
// overlap on one device race, and a handle made by one call is valid only
// until the next call on the same device.
#include <mutex>

#include "static_ws.hpp"

namespace ep {

namespace {

constexpr size_t kStaticWsBytes = 4u << 20;    // 4 MiB: 1M ints of slots, rows and chunk counts
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticWsBytes];

std::mutex g_mu;
void *g_addr[kMaxDevices];

}  // namespace

size_t static_workspace_bytes() { return kStaticWsBytes; }

hipError_t static_workspace(void **addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  return hipSuccess;
}

}  // namespace ep
