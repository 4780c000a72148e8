// Host-side helpers shared by the entry points of the library (defined in
// fa2_runtime.hip, not exported from the shared object).
#pragma once

#include <cstddef>

namespace fa2_host {

// Whether byte ranges [a, a + na) and [b, b + nb) overlap.
__attribute__((visibility("hidden"))) bool overlaps(const void* a, size_t na, const void* b,
                                                    size_t nb);

// FA2_OK when the current HIP device is a gfx950, with its compute-unit count
// in *n_cu; FA2_ERR_NO_DEVICE otherwise. Both facts are cached per device.
__attribute__((visibility("hidden"))) int check_device(int* n_cu);

}  // namespace fa2_host
