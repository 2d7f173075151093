// A library-owned device buffer for the execution entry point that allocates
// nothing (mpaMLAStaticScratch): a file-scope device array, one copy per GPU,
// held until the process ends.  Host code never passes the array's name to a
// kernel or a copy (on the host it is only a stand-in for the symbol): it uses
// the device address that hipGetSymbolAddress returns, looked up once per
// device with that device current.

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "kernels.h"

namespace mpa {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_mu;
std::vector<void*> g_addr;  // device address of `scratch`, per device id
}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_addr.size() <= dev) g_addr.resize(dev + 1, nullptr);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

}  // namespace mpa
