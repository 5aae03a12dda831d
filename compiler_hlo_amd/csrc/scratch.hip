// scratch.hip -- the launch entry point that allocates nothing.
//
// For callers that cannot allocate device memory around a launch (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc),
// hf_fusion_launch_noalloc runs a fusion with the library's own scratch
// memory in place of the caller's workspace: a file-scope device array of
// HF_SCRATCH_BYTES, one copy per GPU, held until the process ends.
//
// Its device address is taken once per device with hipGetSymbolAddress, at
// set-up: hf_fusion_create calls hf_scratch_prepare while it loads a fusion
// with that device current.  After that only the kept address is used (the
// array's name in host code is a host-side stand-in, not a device address).
//
// The only plans that use a workspace are column reduces split into
// segments: their first kernel writes every segment partial before the fold
// kernel reads it, so nothing in the scratch needs clearing between calls.
// Every call on one GPU shares that GPU's array: calls that overlap in time on
// one GPU (other streams or threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "hlofusion.h"
#include "scratch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[HF_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;                         // serialises set-up
std::atomic<void *> g_ptr[kMaxDevices];  // device address of `scratch` on each device (NULL: not prepared)

}  // namespace

namespace hf {

hf_status scratch_prepare(int device, std::string *err) {
  if (device < 0 || device >= kMaxDevices) {
    *err = "device number out of range for the scratch table";
    return HF_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[device].load(std::memory_order_acquire)) return HF_OK;
  // with `device` current (the caller's contract): this device's copy
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
    return HF_ERR_HIP;
  }
  g_ptr[device].store(p, std::memory_order_release);
  return HF_OK;
}

void *scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  return g_ptr[device].load(std::memory_order_acquire);
}

}  // namespace hf

extern "C" hf_status hf_fusion_launch_noalloc(hf_fusion *f, const void *const *params, int32_t n_params,
                                              void *result, void *stream) {
  return hf::launch_in_scratch(f, params, n_params, result, stream);
}
