// Scratch memory of the forward entry point that allocates nothing
// (llama_layer_forward_noalloc): callers that cannot allocate -- code under
// HIP graph capture, tight serving loops, harnesses that forbid it -- pass
// only inputs and outputs, and the forward's intermediate tensors (the
// workspace llama_layer_forward takes from its caller) live in this
// file-scope device array instead.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, from module load until the process ends.  Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in
// for the symbol): it looks up each device's address once, with that device
// current, and uses that address.  Every call on a device shares that
// device's copy, so calls that overlap on one GPU race; nothing in it needs
// to start at zero (every forward writes each workspace byte it reads).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace llk {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
bool g_done[kMaxDevices] = {};
void* g_ptr[kMaxDevices] = {};
hipError_t g_err[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_done[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != device) (void)hipSetDevice(cur);
    g_ptr[device] = e == hipSuccess ? p : nullptr;
    g_err[device] = e;
    g_done[device] = true;
  }
  return g_err[device];
}

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_done[device] ? g_ptr[device] : nullptr;
}

}  // namespace llk
