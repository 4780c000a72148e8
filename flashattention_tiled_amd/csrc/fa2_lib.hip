// The library is compiled as one translation unit from its parts: the
// host-side runtime pieces, the prefill kernel with fa2_fwd, the split-KV
// decoding kernels with fa2_fwd_splitkv, and the FP8 prefill kernel with
// fa2_fwd_fp8.
#include "fa2_runtime.hip"
#include "fa2_fwd.hip"
#include "fa2_splitkv.hip"
#include "fa2_fwd_fp8.hip"
