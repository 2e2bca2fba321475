// Scratch of the allocation-free step (zero_adam_step_static): the norm
// partials a step's launches write and its fold and finalize kernels read --
// what a caller's workspace holds in zero_adam_step -- in a device array of
// this module instead. Each GPU holds its own copy from module load to
// process end; its address is looked up once per device, with that device
// current, and kept. The contents need no clearing: every partial a launch
// reads was written earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "zero_dp_internal.h"

namespace zdp {

static __device__ __align__(256) unsigned char scratch[kWorkspaceBytes];

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static std::unordered_map<int, void*> known;  // device -> its copy's address
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = known.find(dev);
  if (it == known.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = known.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace zdp
