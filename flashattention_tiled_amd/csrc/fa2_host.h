// Host-side helpers shared by the entry points of the library (defined in
// fa2_runtime.hip, not exported from the shared object). The byte-range
// checks on strided tensors are in fa2_plan.h.
#pragma once

#include <cstddef>

namespace fa2_host {

// FA2_OK when the current HIP device is a gfx950, with its compute-unit count
// in *n_cu; FA2_ERR_NO_DEVICE otherwise. Both facts are cached per device.
__attribute__((visibility("hidden"))) int check_device(int* n_cu);

}  // namespace fa2_host
