// Device building blocks shared by the FlashAttention-2 kernels of this
// library (the prefill kernel in fa2_fwd.hip, the split-KV decoding kernels
// in fa2_splitkv.hip): element types, LDS-direct tile loads with their
// swizzles, the K Q^T score product and the probabilities of one tile.
//
// Matrix-core formulation. The wave computes the transposed products
//   S^T = K_j Q^T   (A = K_j from LDS,   B = Q^T resident in registers)
//   O^T = V_j^T P^T (A = V_j^T from LDS, B = P^T straight from S^T's registers)
// with v_mfma_f32_32x32x16_{f16,bf16}. Output column n of a 32x32 block lives
// in lane n (mod 32), so each lane holds one query row per 32-row block: the
// row max and row sum are in-lane reductions plus one exchange with the lane
// 32 away, and the per-row rescale is a per-lane scalar multiply.
//
// MFMA 32x32x16 lane layouts used below (lane l, l32 = l % 32, hi = l / 32):
//   A (32 x 16): lane l holds row l32, 8 k values of half hi.
//   B (16 x 32): lane l holds column l32, the same 8 k values.
//   C (32 x 32): register r of lane l holds row 8*(r/4) + 4*hi + r%4, column l32.
// Any bijection between (hi, element) and k is valid as long as A and B use
// the same one, which is how P^T is fed from the S^T accumulator registers:
// B element e of P^T step (kb, h) is accumulator register 8h + e, that is
// key 32 kb + 16 h + 8 (e / 4) + 4 hi + e % 4, and the V^T operand gathers
// the same keys.
//
// LDS staging. Tiles arrive by buffer loads that write LDS directly, 16 bytes
// per lane; a 64-lane load fills 1 KiB of consecutive 16-byte slots, so the
// layout is chosen by which global chunk each lane fetches. Key rows are
// row-major with their 16-byte chunks XOR-swizzled per row so that the reads
// below hit distinct banks. Buffer loads past the end of a head return zero,
// which zero-fills the keys beyond S of a ragged last tile.
//   K^T A operand: one 16-byte read of row key, chunk (2 s + hi).
//   V^T A operand: two ds_read_b64_tr_b16, the gfx950 transposing read. In
//   each 16-lane group, output lane i element e comes from source lane
//   4 e + i / 4, element i % 4; sources pointed at 4 key rows x 16 dims return
//   4 consecutive keys of one dim per lane, the layout the A operand needs.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <type_traits>
#include <cstdint>
#include <cstring>

#include "fa2.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Buffer resource word 3 for raw (unswizzled, stride 0) buffers on gfx9.
constexpr int kBufferFlags = 0x00020000;

// Element-type specific pieces: the matrix-core product, the RNE packing of
// two fp32 values into the input dtype, and the sum of a packed pair.
template <int DT> struct Elem;

template <> struct Elem<FA2_F16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
  // acc + lo + hi of a packed pair, in fp32
  static __device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
  }
};

template <> struct Elem<FA2_BF16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 h = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
  static __device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
  }
};

// Chunk swizzles (XOR on the 16-byte chunk index within a key row). gfx950
// LDS has 64 banks (256 bytes per cycle); a ds_read_b128 serves 16 lanes per
// cycle and a ds_read_b64_tr_b16 32 lanes, so:
//   K: 16 lanes read chunk c of 16 consecutive rows -> XOR row & 15 puts
//      them in 16 distinct 16-byte bank groups (D = 64: two rows share a
//      256-byte line, so XOR (row / 2) & 7 instead);
//   V: 32 lanes read chunks 4 db .. 4 db + 3 of 4 consecutive rows -> XOR
//      4 (row & 3) spreads them over all 16 groups (D = 64: XOR
//      4 ((row / 2) & 1), rows r and r + 1 already sit in different halves).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 64 ? (row >> 1) & 7 : row & 15;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 64 ? ((row >> 1) & 1) << 2 : (row & 3) << 2;
}

// 16-byte chunk swizzles of FP8 tiles (rows of D bytes, D / 16 chunks).
// K is read 16 bytes per lane, 16 lanes (rows 0-15 or 16-31 of a key block)
// per cycle: XOR by the row bits above those that already separate rows in
// the 64 banks. V is read by ds_read_b64_tr_b8, 32 lanes per cycle over 8
// rows x 2 chunks; an even XOR keeps a chunk pair together and gives each
// of the 4 rows of one parity (D = 64: of the 2 rows of one residue mod 4;
// D = 256: each of the 8 rows) its own pair.
template <int D>
__device__ __forceinline__ int swz_k8(int row) {
  return D == 64 ? (row >> 2) & 3 : D == 128 ? (row >> 1) & 7 : row & 15;
}
template <int D>
__device__ __forceinline__ int swz_v8(int row) {
  return D == 64    ? ((row >> 3) & 1) << 1
         : D == 128 ? (((row >> 1) & 1) | ((row >> 2) & 2)) << 1
                    : ((row & 3) | ((row >> 1) & 4)) << 1;
}

// Per-lane byte offsets of the 16-byte chunks this wave's share of an FP8
// tile load fetches from key rows `row_bytes` apart: LDS slot
// p = (wave * LPW + i) * 64 + lane of the tile receives chunk
// (p % (D/16)) ^ swz(row) of key row p / (D/16).
template <int D, int LPW, bool IS_V>
__device__ __forceinline__ void tile_load_offsets8(int wave, int lane, uint32_t row_bytes,
                                                   uint32_t (&off)[LPW]) {
  constexpr int CPR = D / 16;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int p = (wave * LPW + i) * 64 + lane;
    const int r = p / CPR, cp = p % CPR;
    const int c = cp ^ (IS_V ? swz_v8<D>(r) : swz_k8<D>(r));
    off[i] = (uint32_t)r * row_bytes + (uint32_t)(c * 16);
  }
}

// s_waitcnt with vmcnt(N) and lgkmcnt(0) (gfx9 encoding; expcnt not waited;
// N = 63 leaves the vector memory counter alone).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// x made wave-uniform (scalar register); x must already be equal in all lanes.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// s_barrier alone: it does not wait for this wave's memory operations, so
// LDS writes another wave reads after it need a wait_vm_lgkm0 first.
__device__ __forceinline__ void workgroup_barrier() {
  __asm__ volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Write one 32-column block of a row of O, x * inv rounded to the dtype,
// from the accumulator layout of O~^T: lane (l32, hi) holds columns
// 8 g + 4 hi + 0..3 of its row in x[4 g .. 4 g + 3], g = 0..3. One swap of
// the upper half's even-g and the lower half's odd-g words gives lane hi the
// 8 consecutive columns 16 gp + 8 hi + 0..7 of each pair gp of g: two
// 16-byte stores per lane, each writing 32 contiguous bytes of every row.
// `dst` points at the block's first column of this lane's row (16-byte
// aligned). X is f32x16 or float[16].
template <int DT, class X>
__device__ __forceinline__ void store_o_block(uint16_t* dst, const X& x, float inv, int hi) {
#pragma unroll
  for (int gp = 0; gp < 2; ++gp) {
    const int r = 8 * gp;
    const uint32_t e0 = Elem<DT>::pack2(x[r] * inv, x[r + 1] * inv);
    const uint32_t e1 = Elem<DT>::pack2(x[r + 2] * inv, x[r + 3] * inv);
    const uint32_t d0 = Elem<DT>::pack2(x[r + 4] * inv, x[r + 5] * inv);
    const uint32_t d1 = Elem<DT>::pack2(x[r + 6] * inv, x[r + 7] * inv);
    const auto y0 = __builtin_amdgcn_permlane32_swap(e0, d0, false, false);
    const auto y1 = __builtin_amdgcn_permlane32_swap(e1, d1, false, false);
    *(u32x4*)(dst + 16 * gp + 8 * hi) = u32x4{y0[0], y1[0], y0[1], y1[1]};
  }
}

// Per-lane byte offsets, within one tile, of the 16-byte chunks this wave
// loads: LDS slot p = block * 64 + lane of the tile receives chunk
// (p % CPR) ^ swz(row) of key row p / CPR.
template <int D, int LPW, bool IS_V>
__device__ __forceinline__ void tile_load_offsets(int wave, int lane, uint32_t (&off)[LPW]) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int p = (wave * LPW + i) * 64 + lane;
    const int r = p / CPR, cp = p % CPR;
    const int c = cp ^ (IS_V ? swz_v<D>(r) : swz_k<D>(r));
    off[i] = (uint32_t)((r * D + c * 8) * 2);
  }
}

// The same offsets for key rows `row_bytes` apart in memory (a strided K or
// V; row_bytes >= 2 D). Only the source offsets change: the LDS layout is
// that of tile_load_offsets.
template <int D, int LPW, bool IS_V>
__device__ __forceinline__ void tile_load_offsets_strided(int wave, int lane, uint32_t row_bytes,
                                                          uint32_t (&off)[LPW]) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int p = (wave * LPW + i) * 64 + lane;
    const int r = p / CPR, cp = p % CPR;
    const int c = cp ^ (IS_V ? swz_v<D>(r) : swz_k<D>(r));
    off[i] = (uint32_t)r * row_bytes + (uint32_t)(c * 16);
  }
}

// Buffer descriptor for the K or V rows from row0 on of a head whose rows
// are row_bytes apart, based at row row0. Its record count covers the rows
// left before `rows` (the end of the head, so that loads past it return
// zero; 0 for a tile that is not needed, whose loads then all return zero),
// at most cap_rows of them, where cap_rows * row_bytes < 2^31: the rows one
// tile load reaches through its 32-bit offsets. The base is a 64-bit
// address, so a head may span any size; the count stays in 32-bit
// arithmetic. All values are wave-uniform; readfirstlane keeps them (and so
// the descriptor) in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc_rows(const unsigned char* head_base,
                                                                 int rows, int row0,
                                                                 uint32_t row_bytes, int cap_rows) {
  const int r0 = wave_uniform(row0);
  const int left = wave_uniform(min(max(rows - r0, 0), cap_rows));
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(head_base + (uint64_t)(uint32_t)r0 * row_bytes), 0,
      (int)((uint32_t)left * row_bytes), kBufferFlags);
}

// The largest cap_rows of tile_rsrc_rows for rows row_bytes apart.
__device__ __forceinline__ int rows_within_2g(uint32_t row_bytes) {
  return (int)(0x7fffffffu / row_bytes);
}

// Block i (of this wave's LPW) of a tile load into LDS at `dst`: 64 lanes x
// 16 bytes into the 1 KiB block (wave * LPW + i) of the stage.
template <int LPW>
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rsrc, unsigned char* dst,
                                           int wave, uint32_t off, int i) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (wave * LPW + i) * 1024), 16,
                                           off, 0, 0, 0);
}

// Start loading a whole tile (this wave's LPW blocks) through `rsrc`.
template <int LPW>
__device__ __forceinline__ void load_tile_rsrc(__amdgpu_buffer_rsrc_t rsrc, unsigned char* dst,
                                               int wave, const uint32_t* off) {
#pragma unroll
  for (int i = 0; i < LPW; ++i) load_block<LPW>(rsrc, dst, wave, off[i], i);
}

// S^T = K_t Q^T for one tile whose K sits at byte k_stage of LDS. Chunk
// (2 s + hi) ^ x of a key row (x = swz_k(row)) is byte offset
// (32 s) ^ (16 (hi ^ x)) within it, and row and stage bases have no bits in
// common with it, so the address of k-step s is one per-tile base XOR 32 s.
template <int D, int DT, int RB, int NKB>
__device__ __forceinline__ void tile_scores(const unsigned char* smem, uint32_t k_stage, uint32_t k_lane,
                                            const u32x4 (&qf)[RB][D / 16],
                                            f32x16 (&acc)[RB][NKB]) {
  constexpr int CPR = D / 8, NDS = D / 16;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) acc[rb][kb] = f32x16{};
  const uint32_t k_base = k_stage + k_lane;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      const uint32_t off = (k_base ^ (uint32_t)(32 * s)) + (uint32_t)(kb * 32 * CPR * 16);
      const u32x4 a = *(const u32x4*)(smem + off);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb][kb] = Elem<DT>::mfma(a, qf[rb][s], acc[rb][kb]);
    }
}

// Each row's tile max of t = c_eff * (masked) scores. The max is taken of
// the products, so it holds for a negative c_eff as well (where it is c_eff
// times the smallest score).
template <int RB, int NKB>
__device__ __forceinline__ void tile_max(const f32x16 (&acc)[RB][NKB], const float (&c_eff)[RB],
                                         float (&tmax)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        mx = fmaxf(fmaxf(mx, acc[rb][kb][r] * c_eff[rb]), acc[rb][kb][r + 1] * c_eff[rb]);
    tmax[rb] = xor32_max(mx);
  }
}

// P = 2^(t - m) rounded to the input dtype, packed as the B operand of the
// P V product; tsum and trnd are this lane's shares of the tile's row sums
// of P as computed and as rounded.
template <int DT, int RB, int NKB>
__device__ __forceinline__ void tile_probs(const f32x16 (&acc)[RB][NKB], const float (&c_eff)[RB],
                                           const float (&m_run)[RB], float (&tsum)[RB],
                                           float (&trnd)[RB], u32x4 (&pb)[RB][NKB][2]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    tsum[rb] = 0.f;
    trnd[rb] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = 8 * h + 2 * w;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(acc[rb][kb][r], c_eff[rb], -m_run[rb]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(acc[rb][kb][r + 1], c_eff[rb], -m_run[rb]));
          const uint32_t pk = Elem<DT>::pack2(p0, p1);
          tsum[rb] += p0 + p1;
          trnd[rb] = Elem<DT>::add_pair(pk, trnd[rb]);
          pb[rb][kb][h][w] = pk;
        }
  }
}

}  // namespace
