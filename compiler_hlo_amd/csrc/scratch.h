// scratch.h -- the library's own per-device scratch memory (scratch.hip) and
// the launch that uses it in place of a caller's workspace.
#pragma once

#include <string>

#include "hlofusion.h"

namespace hf {

// Takes the device address of this device's scratch array (once per device;
// `device` must be current).  Called by hf_fusion_create when it loads a
// fusion on a device.
hf_status scratch_prepare(int device, std::string *err);
// The address kept by scratch_prepare (NULL if the device was not prepared).
void *scratch_address(int device);
// hf_fusion_launch with the device's scratch array as the workspace.
hf_status launch_in_scratch(hf_fusion *f, const void *const *params, int32_t n_params, void *result, void *stream);

}  // namespace hf
