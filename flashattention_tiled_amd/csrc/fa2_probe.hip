// Matrix-core ceiling probe for MI355X (gfx950): fp16 or bf16 32x32x16
// products on random operands and nothing else, with the clock each wave ran
// at. The attention kernels are bounded by the same matrix cores; this gives
// the rate they sustain on data like attention's, next to the nominal peak.
#include "fa2_probe.h"

#include <cstdint>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool BF16>
__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Four independent accumulators per wave (one dependent chain already keeps
// the matrix core of a SIMD busy; four leave slack), A operands rotated over
// four registers and B over two, so consecutive products see different
// inputs as they do in attention.
template <bool BF16>
__global__ __launch_bounds__(256, 2) void mfma_ceiling_kernel(const f16x8* __restrict__ ops,
                                                              int iters, float* __restrict__ sink,
                                                              unsigned long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  f16x8 a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = ops[i * 64 + lane];
#pragma unroll
  for (int i = 0; i < 2; ++i) b[i] = ops[(4 + i) * 64 + lane];
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = mfma<BF16>(a[(u + j) & 3], b[(u + j) & 1], acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
  if (lane == 0) {
    clocks[2 * (size_t)wave] = t1 - t0;
    clocks[2 * (size_t)wave + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" double fa2_probe_mfma_flops(int n_wg, int iters) {
  return (double)n_wg * 4.0 * (double)iters * 16.0 * (32.0 * 32.0 * 16.0 * 2.0);
}

extern "C" int fa2_probe_mfma_ceiling(const void* operands, int n_wg, int iters, float* sink,
                                      unsigned long long* clocks, int dtype, hipStream_t stream) {
  if (!operands || !sink || !clocks) return 1;
  if (n_wg < 1 || iters < 1) return 2;
  if (dtype != 0 && dtype != 1) return 4;
  if (dtype == 1)
    mfma_ceiling_kernel<true><<<dim3((unsigned)n_wg), dim3(256), 0, stream>>>(
        (const f16x8*)operands, iters, sink, clocks);
  else
    mfma_ceiling_kernel<false><<<dim3((unsigned)n_wg), dim3(256), 0, stream>>>(
        (const f16x8*)operands, iters, sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}
