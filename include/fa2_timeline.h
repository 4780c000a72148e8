// Per-workgroup timeline of the prefill kernel: a measurement aid, exported
// only by the timeline build of the library (libfa2_timeline.so, the same
// sources compiled with -DFA2_TIMELINE; flashattention_tiled_amd/timeline.py
// builds and reads it). It is not part of the attention path: the library's
// own build (libfa2.so) compiles the recording out and exports none of this.
//
// In the timeline build, wave 0 of each of the first fa2_timeline_capacity()
// workgroups of every prefill launch (fa2_fwd, fa2_fwd_balanced,
// fa2_fwd_strided) writes 8 64-bit words, slot s of workgroup w at index
// 8 w + s (w: the workgroup's linear index in its launch grid):
//   0  start, 100 MHz real-time clock (s_memrealtime)
//   1  after the prologue's barrier, its first K/V tiles in LDS (on the
//      unpipelined key loop: once its first tiles' loads are issued)
//   2  after the key loop (and the wait for its last loads)
//   3  end, after the stores of O and lse are issued
//   4  HW_ID register in the low 32 bits, XCC_ID register in the high 32
//   5  query tile | (b, h) << 16 | key-loop steps << 32
//   6, 7  unused
// A later launch overwrites the slots of the workgroups it runs.
#pragma once

#ifdef __cplusplus
extern "C" {
#endif

// Workgroups per launch that record (16384).
int fa2_timeline_capacity(void);

// Zero every slot, on `stream` (a hipStream_t; NULL: the default stream).
// Returns FA2_OK or FA2_ERR_LAUNCH.
int fa2_timeline_clear(void *stream);

// Wait for the device, then copy the slots of the first n_wg workgroups
// (8 n_wg words) to host memory the caller owns. Returns FA2_OK,
// FA2_ERR_SHAPE (host NULL or n_wg outside [0, capacity]) or FA2_ERR_LAUNCH.
int fa2_timeline_read(unsigned long long *host, int n_wg);

#ifdef __cplusplus
}
#endif
