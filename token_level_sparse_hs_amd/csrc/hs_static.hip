// Library-owned scratch for the entry point that allocates nothing
// (hs_decode_step_noalloc): a file-scope device array, one copy per GPU the
// library runs on, held until the process ends.
//
// Host code never uses the array's name as a device address (in host code it
// is only a host-side stand-in): the address is looked up once per device,
// with that device current, by hipGetSymbolAddress, and that pointer is what
// the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "hs_kernels.hpp"

namespace {

static __device__ __align__(256) uint8_t scratch[hs::kStaticScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device: the array's device address (null: not looked up yet)

}  // namespace

namespace hs {

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace hs
