// Measurement aids beside the attention library (libfa2probe.so, a library of
// its own; not part of the attention path):
//  - the ceiling probe, a kernel that does nothing but fp16 or bf16
//    matrix-core products on random operands, timed by the caller, to give
//    the rate the matrix cores of the GPU actually sustain on data like
//    attention's. The nominal dense fp16/bf16 peak of MI355X (256 CUs x
//    2.4 GHz x 4096 FLOP/clk/CU) assumes the top clock; under matrix-core
//    load on random data the part lowers its clock to stay within its power
//    limit, and this kernel reports both the rate and the clock it ran at;
//  - the FP8 product probe, single e4m3 matrix-core products on operands the
//    caller chooses, to measure the instruction's rounding of its sum;
//  - the FP8 conversion probe, fp32 -> e4m3 by the instruction the FP8
//    attention kernel rounds P with.
#pragma once

#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

// Number of 8 x 16-bit operand vectors the kernel reads (6 per lane of a wave:
// 4 A and 2 B operands, rotated so that consecutive products see different
// inputs).
#define FA2_PROBE_OPERAND_VECTORS 384

// FLOPs one launch performs: n_wg workgroups of 4 waves, each wave `iters`
// rounds of 16 products of a 32x32x16 matrix-core op (32 x 32 x 16 x 2 FLOPs).
double fa2_probe_mfma_flops(int n_wg, int iters);

// Enqueue one launch on `stream` (asynchronous, never synchronises).
//   operands  device, FA2_PROBE_OPERAND_VECTORS x 8 values of `dtype`
//             (16-byte aligned), read only; random N(0, 1) values model
//             attention's
//   n_wg      workgroups (256 threads each; two fit on a compute unit)
//   iters     rounds per wave, >= 1
//   sink      device, n_wg x 256 floats: each thread writes one sum of its
//             results there, so that the products are not optimised away
//   clocks    device, n_wg x 4 x 2 unsigned 64-bit values: per wave, the
//             shader-clock ticks (s_memtime) and the constant 100 MHz
//             reference ticks (s_memrealtime) its loop took
//   dtype     0: fp16 operands (v_mfma_f32_32x32x16_f16), 1: bf16
//             (v_mfma_f32_32x32x16_bf16), the codes of fa2.h's fa2_dtype
// Returns 0, or 1 for a null pointer, 2 for n_wg < 1 or iters < 1, 4 for
// another dtype, 8 when the launch fails. The caller owns every buffer.
int fa2_probe_mfma_ceiling(const void* operands, int n_wg, int iters, float* sink,
                           unsigned long long* clocks, int dtype, hipStream_t stream);

// Enqueue n_blocks independent FP8 matrix-core products on `stream`, one
// v_mfma_f32_32x32x64_f8f6f4 (both operands OCP e4m3, no block scales)
// per block:
//   C_out[n][i][j] = C_in[n][i][j] + sum_k A[n][i][k] * B[n][j][k]
//   a, b    device, n_blocks x 32 x 64 e4m3 codes each, row-major (A by row
//           i, B by column j, 64 k values per row), 32-byte aligned
//   c_in    device, n_blocks x 32 x 32 floats, row-major
//   c_out   device, the same shape (may not overlap c_in)
// Returns 0, or 1 for a null pointer, 2 for n_blocks < 1, 16 for
// misaligned buffers, 8 when the launch fails. Used to bound how far the
// instruction's internal sum can be from the exact one, which the FP8
// attention path's tolerance depends on.
int fa2_probe_mfma_fp8(const void* a, const void* b, const float* c_in, float* c_out,
                       int n_blocks, hipStream_t stream);

// Enqueue the conversion of n fp32 values to OCP e4m3 codes on `stream`,
// by v_cvt_pk_fp8_f32 (the instruction that rounds P in the FP8 attention
// kernel), code i of value i:
//   in    device, n floats, 16-byte aligned
//   out   device, n bytes, 16-byte aligned
//   n     a multiple of 4, >= 4
// Returns 0, or 1 for a null pointer, 2 for a bad n, 16 for misaligned
// buffers, 8 when the launch fails.
int fa2_probe_cvt_fp8(const float* in, void* out, int n, hipStream_t stream);

#ifdef __cplusplus
}
#endif
