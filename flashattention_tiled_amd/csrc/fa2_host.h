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

// Whether the rows (b, h, s) of a (B, H, S, D) tensor with these element
// strides (head dim contiguous) are pairwise disjoint.
__attribute__((visibility("hidden"))) bool rows_disjoint(int B, int H, int S, int D, long long sb,
                                                         long long sh, long long ss);

// Bytes from a strided (B, H, S, D) tensor's base pointer to the end of its
// last element.
__attribute__((visibility("hidden"))) size_t extent_bytes(int B, int H, int S, int D, long long sb,
                                                          long long sh, long long ss,
                                                          int elem_bytes);

}  // namespace fa2_host
