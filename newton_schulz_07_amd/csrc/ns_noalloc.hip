// ns_noalloc.hip - the fixed device scratch of ns_orthogonalize_noalloc.
//
// A caller that cannot allocate device memory (work under HIP graph capture
// before any warm-up, serving loops, harnesses that forbid hipMalloc) uses
// this array as the call's workspace instead of the library's cached one.
// Each GPU the library runs on holds its own copy of NS_NOALLOC_SCRATCH_BYTES
// from the moment the code object is loaded until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever handed to kernels or copies.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "../../include/ns_hip.h"
#include "ns_kernels.h"

static __device__ __align__(256) char scratch[NS_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::map<int, char*> g_scratch_addr;  // device -> device address of its copy

}  // namespace

namespace ns {

hipError_t noalloc_scratch(int dev, char** ptr) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_addr.find(dev);
  if (it == g_scratch_addr.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    it = g_scratch_addr.emplace(dev, static_cast<char*>(p)).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace ns
