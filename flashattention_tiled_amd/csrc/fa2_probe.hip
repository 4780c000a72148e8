// Matrix-core probes for MI355X (gfx950), measurement aids beside the
// attention library:
//  - the ceiling probe: fp16 or bf16 32x32x16 products on random operands
//    and nothing else, with the clock each wave ran at. The attention kernels
//    are bounded by the same matrix cores; this gives the rate they sustain on
//    data like attention's, next to the nominal peak;
//  - the FP8 product probe: single e4m3 32x32x64 products on given operands,
//    from which a test measures how far the instruction's sum is from the
//    exact one (the FP8 attention path's tolerance rests on that bound);
//  - the FP8 conversion probe: fp32 -> e4m3 codes by the instruction that
//    rounds P in the FP8 attention kernel, to check its rounding.
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

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One FP8 product per wave: C_out = A B + C_in for one 32 x 64 (A, e4m3)
// by 64 x 32 (B, e4m3) block on v_mfma_f32_32x32x64_f8f6f4, the operand
// layout of the instruction: lane l holds row (A) / column (B) l % 32 and
// k = 32 (l / 32) .. + 31, one byte each; C register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
__global__ __launch_bounds__(64) void mfma_fp8_probe_kernel(const unsigned char* __restrict__ a,
                                                             const unsigned char* __restrict__ b,
                                                             const float* __restrict__ c_in,
                                                             float* __restrict__ c_out) {
  const int lane = threadIdx.x, l32 = lane & 31, hi = lane >> 5;
  const size_t blk = blockIdx.x;
  const i32x8 av = *(const i32x8*)(a + blk * 2048 + l32 * 64 + 32 * hi);
  const i32x8 bv = *(const i32x8*)(b + blk * 2048 + l32 * 64 + 32 * hi);
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = c_in[blk * 1024 + (8 * (r / 4) + 4 * hi + r % 4) * 32 + l32];
  // operand formats 0, 0: both e4m3; no block scales
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) c_out[blk * 1024 + (8 * (r / 4) + 4 * hi + r % 4) * 32 + l32] = c[r];
}

// e4m3 codes of fp32 values by the conversion the FP8 attention kernel
// rounds P with (v_cvt_pk_fp8_f32, two values per instruction, into the low
// or the high half of a word): four values per thread.
__global__ __launch_bounds__(256) void cvt_fp8_probe_kernel(const float* __restrict__ in,
                                                            unsigned* __restrict__ out, int n4) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 x = *(const float4*)(in + 4 * (size_t)i);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x.x, x.y, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x.z, x.w, w, true);
  out[i] = (unsigned)w;
}

}  // namespace

extern "C" int fa2_probe_cvt_fp8(const float* in, void* out, int n, hipStream_t stream) {
  if (!in || !out) return 1;
  if (n < 4 || n % 4) return 2;
  if (((uintptr_t)in | (uintptr_t)out) & 15u) return 16;
  const int n4 = n / 4;
  cvt_fp8_probe_kernel<<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream>>>(
      in, (unsigned*)out, n4);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

extern "C" int fa2_probe_mfma_fp8(const void* a, const void* b, const float* c_in, float* c_out,
                                  int n_blocks, hipStream_t stream) {
  if (!a || !b || !c_in || !c_out) return 1;
  if (n_blocks < 1) return 2;
  if (((uintptr_t)a | (uintptr_t)b) & 31u || ((uintptr_t)c_in | (uintptr_t)c_out) & 3u) return 16;
  mfma_fp8_probe_kernel<<<dim3((unsigned)n_blocks), dim3(64), 0, stream>>>(
      (const unsigned char*)a, (const unsigned char*)b, c_in, c_out);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

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
