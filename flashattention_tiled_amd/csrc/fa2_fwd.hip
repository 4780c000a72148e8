// FlashAttention-2 forward pass for MI355X (gfx950 / CDNA4).
//
// One workgroup owns a tile of B_r query rows of one (batch, head); the grid
// is (ceil(S / B_r), H, B), the sequence-parallel grid of FlashAttention-2
// (jared-hpc Lecture 6, "FA2 change 1"). Inside the workgroup every 64-lane
// wavefront owns its query rows outright and runs the whole key loop on them,
// so waves never exchange softmax state (infra.bea.ai FlashAttention V2 guide,
// "Optimization 3: Warp-Level Work Partitioning", split-Q). K and V tiles of
// B_c keys stream through a ring of LDS stages shared by the workgroup's
// waves; the next tiles are in flight while the current one is computed.
//
// Per key tile j a wave computes, for each query row it owns (infra.bea.ai
// guide, "Optimization 2: Delay Rescaling"; the cookbook notebook's Triton
// kernel loop):
//   S   = Q K_j^T                         (matrix cores, fp32 accumulate)
//   t   = c * S,  c = scale * log2(e)     (base-2 logits)
//   P   = 2^(t - m)                       rounded to the input dtype
//   l   = l + rowsum(P)
//   O~  = O~ + P V_j                      (matrix cores, fp32 accumulate)
// and only the epilogue divides by l and writes lse = ln2 * (m + log2 l).
// 2^(x log2 e) = e^x, so these are the pages' exp-based recurrences.
//
// The reference point m is set to the row max of the first key tile and
// moved lazily after that: it is raised (rescaling O~ and l by
// alpha = 2^(m_old - m_new), as the guide's recurrence does) only when one
// lane's share of a tile's row sum of P exceeds kSumLimit = 2^12. Any m
// gives the same O and lse in exact arithmetic -- it cancels between O~ and
// l -- and every P of a tile that passes the test is at most 2^12, inside
// the fp16/bf16 range, so the test replaces the per-tile row max of the
// pages' recurrence on the vector unit. A tile that fails it is redone: its
// row max is taken, m is raised to it, O~ and l are rescaled and its P is
// recomputed. l sums P in fp32 as computed, before P is rounded for the
// P V product, as the pages' l does, and gives lse; O is divided by a second
// sum, of P as rounded, which makes it an exact convex combination of V rows
// whatever the rounding of P (a near one-hot row then reproduces its V row
// up to fp32 accumulation, not up to the rounding of its largest P).
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
constexpr float kSumLimit = 4096.0f;  // lazy-rescale threshold on a lane's tile sum of P
// Phase-1 k-steps between this wave's tile-load blocks (0: all at the start
// of the step). Spacing them out helps D = 128 slightly; D = 64 and D = 256
// run best with all loads up front.
template <int D> struct LoadEvery { static constexpr int kValue = D == 128 ? 2 : 0; };

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

// Tile shape per head dimension.
//   kWaves      waves per workgroup (they share the LDS rings)
//   kRowBlocks  32-row MFMA blocks per wave
//   kBc         keys per tile
//   kWavesPerSimd  waves per SIMD the register budget is sized for
// K and V each have a two-stage LDS ring: iteration j reads K of tile j + 1
// and V of tile j while K of tile j + 2 and V of tile j + 1 load.
template <int D> struct Tile;
template <> struct Tile<64> {
  static constexpr int kWaves = 4, kRowBlocks = 1, kBc = 64, kWavesPerSimd = 2;
};
template <> struct Tile<128> {
  static constexpr int kWaves = 4, kRowBlocks = 1, kBc = 64, kWavesPerSimd = 2;
};
template <> struct Tile<256> {
  static constexpr int kWaves = 4, kRowBlocks = 1, kBc = 32, kWavesPerSimd = 1;
};

template <int D> struct Shape {
  static constexpr int kWaves = Tile<D>::kWaves;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRB = Tile<D>::kRowBlocks;
  static constexpr int kRowsPerWave = 32 * kRB;
  static constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
  static constexpr int kBc = Tile<D>::kBc;
  static constexpr int kChunksPerRow = D / 8;        // 16-byte chunks per key row
  static constexpr int kTileBytes = kBc * D * 2;     // one K or one V tile
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;  // per K (or V) tile
  static constexpr int kLdsBytes = 4 * kTileBytes;   // K ring (2) + V ring (2)
  static_assert(kTileBytes % (1024 * kWaves) == 0, "tile must split into 1 KiB wave loads");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
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

// s_waitcnt with vmcnt(N) and lgkmcnt(0) (gfx9 encoding; expcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// x made wave-uniform (scalar register); x must already be equal in all lanes.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

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

// Buffer descriptor for tile t of a head (K or V), rebased on the tile. Its
// record count ends at `limit` bytes from the head start (the end of the
// head, so that loads past S return zero; 0 for a tile that is not needed,
// whose loads then all return zero).
template <int TB>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const unsigned char* head_base,
                                                            uint32_t limit, int t) {
  // both values are wave-uniform; readfirstlane keeps them (and so the buffer
  // descriptor) in scalar registers
  const uint32_t start = (uint32_t)t * TB;
  const uint32_t left = (uint32_t)wave_uniform((int)(limit - (start < limit ? start : limit)));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(head_base + start), 0, (int)left, kBufferFlags);
}

// Block i (of this wave's LPW) of a tile load into LDS at `dst`: 64 lanes x
// 16 bytes into the 1 KiB block (wave * LPW + i) of the stage.
template <int LPW>
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rsrc, unsigned char* dst,
                                           int wave, uint32_t off, int i) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (wave * LPW + i) * 1024), 16,
                                           off, 0, 0, 0);
}

// Start loading a whole tile (this wave's LPW blocks).
template <int LPW, int TB>
__device__ __forceinline__ void load_tile(const unsigned char* head_base, uint32_t head_bytes,
                                          int t, unsigned char* dst, int wave,
                                          const uint32_t* off) {
  const __amdgpu_buffer_rsrc_t rsrc = tile_rsrc<TB>(head_base, head_bytes, t);
#pragma unroll
  for (int i = 0; i < LPW; ++i) load_block<LPW>(rsrc, dst, wave, off[i], i);
}

// The loads one pipeline step issues: this wave's LPW blocks of the next K
// tile, then its LPW blocks of the next V tile, issued one at a time between
// the step's matrix ops (or all at its start) so that the waves of a compute
// unit do not all queue their loads at once.
template <int LPW>
struct StepLoads {
  __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;
  unsigned char* k_dst;
  unsigned char* v_dst;
  const uint32_t* k_off;
  const uint32_t* v_off;
  int wave;
  __device__ __forceinline__ void issue(int n) const {
    if (n < LPW)
      load_block<LPW>(k_rsrc, k_dst, wave, k_off[n], n);
    else
      load_block<LPW>(v_rsrc, v_dst, wave, v_off[n - LPW], n - LPW);
  }
};

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

// Mask one tile's scores. Register r of key block kb holds key
// key0 + 32 kb + 8 (r / 4) + 4 hi + r % 4; it is kept iff that key is < S
// and (causal) <= row. Masked tiles are scaled here and masked in the scaled
// domain, so a zero scale never meets a -inf score; their c_eff is then 1,
// else c.
template <int RB, int NKB, bool CAUSAL>
__device__ __forceinline__ void tile_mask(f32x16 (&acc)[RB][NKB], int key0, int row0, int S,
                                          float c, int l32, int hi, float (&c_eff)[RB]) {
  constexpr int Bc = 32 * NKB;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    c_eff[rb] = c;
    const int row = row0 + 32 * rb + l32;
    if ((key0 + Bc > S) || (CAUSAL && key0 + Bc - 1 > row0 + 32 * rb)) {
      const int base_key = key0 + 4 * hi;
      const int lim = CAUSAL ? min(S - base_key, row - base_key + 1) : S - base_key;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = 32 * kb + 8 * (r / 4) + (r % 4);
          acc[rb][kb][r] = rel < lim ? acc[rb][kb][r] * c : -INFINITY;
        }
      c_eff[rb] = 1.f;
    }
  }
}

// Whether any row block of the wave needs masking for the tile at key0.
template <int RB, int NKB, bool CAUSAL>
__device__ __forceinline__ bool tile_needs_mask(int key0, int row0, int S) {
  constexpr int Bc = 32 * NKB;
  return (key0 + Bc > S) || (CAUSAL && key0 + Bc - 1 > row0);
}

// Each row's tile max of t = c_eff * (masked) scores.
template <int RB, int NKB>
__device__ __forceinline__ void tile_max(const f32x16 (&acc)[RB][NKB], const float (&c_eff)[RB],
                                         float (&tmax)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, acc[rb][kb][r]), acc[rb][kb][r + 1]);
    tmax[rb] = xor32_max(mx) * c_eff[rb];
  }
}

// Raise each row's reference max to at least its tile max tmax, rescaling
// O~ and both sums by alpha = 2^(m_old - m_new).
template <int RB, int NDB>
__device__ __forceinline__ void raise_max(const float (&tmax)[RB], float (&m_run)[RB],
                                          float (&l_run)[RB], float (&l_rnd)[RB],
                                          f32x16 (&acc_o)[RB][NDB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float m_new = fmaxf(m_run[rb], tmax[rb]);
    const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
    l_run[rb] *= alpha;
    l_rnd[rb] *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[rb][db] *= alpha;
    m_run[rb] = m_new;
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

// The main block of one pipeline step, written in the order it should
// issue (two waves per SIMD fill each other's gaps; the source order gives
// the scheduler the interleave):
//   phase 1, one step per 16-wide k-step of the scores of tile j + 1: the RB
//     matrix ops of that k-step (its K operand read PFK steps ahead) beside
//     the next PPS probability pairs of tile j on the vector unit;
//   the lazy-rescale test on tile j's sums of P (and, rarely, the redo);
//   phase 2, one step per (key block, half, head-dim block) of the P V
//     product of tile j: its RB matrix ops, V^T operands read PFV steps
//     ahead.
// Probability pairs come in the order the P V steps consume them.
template <int D, int DT, int RB, int NKB, int LPW, int LEVERY>
__device__ __forceinline__ void pipeline_block(
    const StepLoads<LPW>& ld, const unsigned char* smem, uint32_t k_stage, uint32_t v_stage,
    uint32_t k_lane, uint32_t vt_x,
    const u32x4 (&qf)[RB][D / 16], const f32x16 (&cur)[RB][NKB], const float (&ce_cur)[RB],
    float (&m_run)[RB], float (&l_run)[RB], float (&l_rnd)[RB], f32x16 (&nxt)[RB][NKB],
    f32x16 (&acc_o)[RB][D / 32]) {
  using E = Elem<DT>;
  constexpr int CPR = D / 8, NDS = D / 16, NDB = D / 32;
  constexpr int NS1 = NKB * NDS;                   // phase-1 steps
  constexpr int NPAIR = RB * NKB * 8;              // probability pairs per lane
  constexpr int PPS = (NPAIR + NS1 - 1) / NS1;     // pairs per phase-1 step
  constexpr int NS2 = NKB * 2 * NDB;               // phase-2 steps
  constexpr int PFK = 3, PFV = 2;                  // operand read-ahead (steps)
  static_assert(LEVERY == 0 || (NS1 + LEVERY - 1) / LEVERY >= 2 * LPW,
                "the load spacing must leave a k-step for every load block");

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) nxt[rb][kb] = f32x16{};
  float tsum[RB], trnd[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    tsum[rb] = 0.f;
    trnd[rb] = 0.f;
  }

  // phase 1
  const uint32_t k_base = k_stage + k_lane;
  auto k_read = [&](int st) {
    const int kb = st / NDS, s = st % NDS;
    const uint32_t off = (k_base ^ (uint32_t)(32 * s)) + (uint32_t)(kb * 32 * CPR * 16);
    return *(const u32x4*)(smem + off);
  };
  u32x4 kq[PFK];
#pragma unroll
  for (int i = 0; i < PFK; ++i)
    if (i < NS1) kq[i] = k_read(i);
  u32x4 pb[RB][NKB][2];
#pragma unroll
  for (int st = 0; st < NS1; ++st) {
    const int kb = st / NDS, s = st % NDS;
    if (LEVERY == 0) {
      if (st == 0)
#pragma unroll
        for (int n = 0; n < 2 * LPW; ++n) ld.issue(n);
    } else if (st % LEVERY == 0 && st / LEVERY < 2 * LPW) {
      ld.issue(st / LEVERY);
      // keep each load in its own k-step: vector, scalar and LDS instructions
      // may be scheduled across this point, matrix ops and memory loads not
      __builtin_amdgcn_sched_barrier(0x786);
    }
    const u32x4 a = kq[st % PFK];
    if (st + PFK < NS1) kq[st % PFK] = k_read(st + PFK);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) nxt[rb][kb] = E::mfma(a, qf[rb][s], nxt[rb][kb]);
#pragma unroll
    for (int pp = 0; pp < PPS; ++pp) {
      const int p = st * PPS + pp;  // pair p = ((kb * 2 + h) * RB + rb) * 4 + w
      if (p < NPAIR) {
        const int w = p % 4, rb = (p / 4) % RB, h = (p / (4 * RB)) % 2, pkb = p / (8 * RB);
        const int r = 8 * h + 2 * w;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[rb][pkb][r], ce_cur[rb], -m_run[rb]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(cur[rb][pkb][r + 1], ce_cur[rb], -m_run[rb]));
        const uint32_t pk = E::pack2(p0, p1);
        tsum[rb] += p0 + p1;
        trnd[rb] = E::add_pair(pk, trnd[rb]);
        pb[rb][pkb][h][w] = pk;
      }
    }
  }

  // phase 2 operand reads, then the lazy-rescale test: every P of this lane
  // is at most its tsum, so tsum <= kSumLimit in all lanes bounds all of P.
  // Otherwise (rarely) raise m to the tile's row max and redo the tile's P.
  const unsigned char* v_lds = smem + v_stage;
  auto v_read = [&](int st) {
    const int kb = st / (2 * NDB), h = (st / NDB) % 2, db = st % NDB;
    const unsigned char* vp = v_lds + (32 * kb + 16 * h) * CPR * 16 + (vt_x ^ (uint32_t)(64 * db));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
    const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * CPR * 16));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
    return u32x4{lo2[0], lo2[1], up2[0], up2[1]};
  };
  u32x4 vq[PFV];
#pragma unroll
  for (int i = 0; i < PFV; ++i)
    if (i < NS2) vq[i] = v_read(i);
  bool big = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) big |= !(tsum[rb] <= kSumLimit);
  if (__builtin_amdgcn_ballot_w64(big) != 0) {
    float tm[RB], m_old[RB], ts2[RB], tr2[RB];
    u32x4 pb2[RB][NKB][2];
    tile_max<RB, NKB>(cur, ce_cur, tm);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m_old[rb] = m_run[rb];
    raise_max<RB, NDB>(tm, m_run, l_run, l_rnd, acc_o);
    tile_probs<DT, RB, NKB>(cur, ce_cur, m_run, ts2, tr2, pb2);
    // rows whose m did not move keep the P already computed (the same
    // values); selecting rather than overwriting keeps the phase-1 packing
    // of P where it is instead of letting it sink past this test
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool moved = m_run[rb] != m_old[rb];
      tsum[rb] = moved ? ts2[rb] : tsum[rb];
      trnd[rb] = moved ? tr2[rb] : trnd[rb];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int w = 0; w < 4; ++w) pb[rb][kb][h][w] = moved ? pb2[rb][kb][h][w] : pb[rb][kb][h][w];
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += tsum[rb];
    l_rnd[rb] += trnd[rb];
  }

  // phase 2
#pragma unroll
  for (int st = 0; st < NS2; ++st) {
    const int kb = st / (2 * NDB), h = (st / NDB) % 2, db = st % NDB;
    const u32x4 a = vq[st % PFV];
    if (st + PFV < NS2) vq[st % PFV] = v_read(st + PFV);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc_o[rb][db] = E::mfma(a, pb[rb][kb][h], acc_o[rb][db]);
  }
}

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(Shape<D>::kThreads, Tile<D>::kWavesPerSimd) void fa2_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int S, float c /* scale * log2(e) */, int pair_split) {
  using SH = Shape<D>;
  using E = Elem<DT>;
  constexpr int RB = SH::kRB, Bc = SH::kBc, Br = SH::kBr;
  constexpr int CPR = SH::kChunksPerRow, TB = SH::kTileBytes, LPW = SH::kLoadsPerWave;
  constexpr int NKB = Bc / 32;  // 32-key blocks per tile
  constexpr int NDS = D / 16;   // k-steps of 16 over the head dim (S^T product)
  constexpr int NDB = D / 32;   // 32-wide head-dim blocks of O^T

  // K ring (stages 0, 1) then V ring (stages 0, 1), TB bytes each.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SH::kLdsBytes];
  constexpr uint32_t kK0 = 0, kK1 = TB, kV0 = 2 * TB, kV1 = 3 * TB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroup -> (query tile, batch*head). Tiles are taken in descending
  // query-tile order across all heads, so under causal masking the longest
  // tiles start first; the workgroups of one (b, h) are H*B apart in launch
  // order, which keeps them on one XCD when H*B is a multiple of 8. When the
  // whole causal grid is resident at once (pair_split > 0, set by the host),
  // the workgroups from pair_split on take the query tiles in ascending
  // order instead, so that the second workgroup a compute unit receives is
  // a light tile beside its heavy first one.
  const int n_qt = gridDim.x;
  const int n_bh = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int bh = lin % n_bh;
  const int qt = (pair_split > 0 && lin >= pair_split) ? (lin - pair_split) / n_bh
                                                       : n_qt - 1 - lin / n_bh;
  const int q0 = qt * Br;
  const size_t head = (size_t)bh * (size_t)S * D;
  const int wave_row0 = q0 + wave * SH::kRowsPerWave;

  // Q^T operands: lane holds Q[row][16 s + 8 hi .. +7] of each of its rows.
  u32x4 qf[RB][NDS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wave_row0 + 32 * rb + l32;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      qf[rb][s] = u32x4{0, 0, 0, 0};
      if (row < S) qf[rb][s] = *(const u32x4*)(q + head + (size_t)row * D + 16 * s + 8 * hi);
    }
  }

  // K and V of this head, loaded through bounds-checked buffers.
  const uint32_t head_bytes = (uint32_t)S * D * 2;
  const unsigned char* k_head = (const unsigned char*)(k + head);
  const unsigned char* v_head = (const unsigned char*)(v + head);
  uint32_t k_off[LPW], v_off[LPW];
  tile_load_offsets<D, LPW, false>(wave, lane, k_off);
  tile_load_offsets<D, LPW, true>(wave, lane, v_off);

  // LDS read offsets that do not depend on the tile.
  // K^T operand: row 32 kb + l32, chunk (2 s + hi) ^ swz_k(l32).
  const uint32_t k_lane = (uint32_t)(l32 * CPR * 16 + 16 * (hi ^ swz_k<D>(l32)));
  // V^T operand: row 32 kb + 16 h + 4 hi + (lane % 16) / 4 (+8 for e >= 4),
  // dims 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4) .. +3, i.e. chunk
  // 4 db + vt_chunk, byte 8 (lane % 2) within it. The swizzle is 4 w for a
  // per-row w, and (4 db + c) ^ 4 w = 4 (db ^ w) + c, so head-dim block db
  // is at vt_x ^ (64 db) with vt_x = the db = 0 offset plus 64 w (the bits
  // of 64 db are clear in every other term).
  const int vt_row = 4 * hi + (lane & 15) / 4;
  const int vt_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const uint32_t vt_x = (uint32_t)((vt_row * CPR + vt_chunk) * 16 + 8 * (lane & 1) +
                                   64 * (swz_v<D>(vt_row) >> 2));

  f32x16 acc_o[RB][NDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[rb][db] = f32x16{};
  // Per row: the reference max m of t (base-2) and this lane's shares of the
  // row sums of P as computed (for lse) and as rounded (normalises O).
  float m_run[RB], l_run[RB], l_rnd[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = 0.f;
    l_run[rb] = 0.f;
    l_rnd[rb] = 0.f;
  }

  const int kv_end = CAUSAL ? min(q0 + Br, S) : S;
  const int n_tiles = (kv_end + Bc - 1) / Bc;  // tiles the workgroup loads
  // tiles this wave computes (under causal masking the later tiles of the
  // workgroup lie wholly above this wave's rows)
  const int n_act =
      CAUSAL ? min(n_tiles, (wave_row0 + SH::kRowsPerWave + Bc - 1) / Bc) : n_tiles;

  // Software pipeline. Iteration j computes the scores of tile j + 1 on the
  // matrix cores while the vector unit turns tile j's scores into P, then the
  // P V product of tile j.
  // At its top every load issued in iteration j - 1 (K of tile j + 1, V of
  // tile j) has landed, and after the barrier every wave is done with
  // iteration j - 1, so K of tile j + 2 goes into tile j's K stage and V of
  // tile j + 1 into tile j - 1's V stage.
  load_tile<LPW, TB>(k_head, head_bytes, 0, smem + kK0, wave, k_off);
  load_tile<LPW, TB>(v_head, head_bytes, 0, smem + kV0, wave, v_off);
  if (n_tiles > 1) load_tile<LPW, TB>(k_head, head_bytes, 1, smem + kK1, wave, k_off);

  f32x16 s_a[RB][NKB], s_b[RB][NKB];
  float ce_a[RB], ce_b[RB];
  wait_vm_lgkm0<0>();
  workgroup_barrier();
  if (n_act > 0) {
    // m starts at the row max of tile 0, which holds an unmasked key for
    // every row (key 0), so m is finite from here on
    tile_scores<D, DT, RB, NKB>(smem, kK0, k_lane, qf, s_a);
    tile_mask<RB, NKB, CAUSAL>(s_a, 0, wave_row0, S, c, l32, hi, ce_a);
    tile_max<RB, NKB>(s_a, ce_a, m_run);
  }

  // One pipeline step for tile j with parity PAR = j % 2 (known at compile
  // time after unrolling by two); `cur` holds tile j's scores, `nxt` receives
  // tile j + 1's.
  auto step = [&](auto par, int j, f32x16 (&cur)[RB][NKB], float (&ce_cur)[RB],
                  f32x16 (&nxt)[RB][NKB], float (&ce_nxt)[RB]) {
    constexpr int PAR = decltype(par)::value;
    constexpr uint32_t k_next = PAR ? kK0 : kK1;  // K of tile j + 1
    constexpr uint32_t k_free = PAR ? kK1 : kK0;  // K of tile j (done)
    constexpr uint32_t v_cur = PAR ? kV1 : kV0;   // V of tile j
    constexpr uint32_t v_free = PAR ? kV0 : kV1;  // V of tile j - 1 (done)
    wait_vm_lgkm0<0>();
    workgroup_barrier();
    // K of tile j + 2 and V of tile j + 1; a tile past the workgroup's last
    // gets a zero-length buffer, so its loads only write zeros to a free stage
    const StepLoads<LPW> ld{
        tile_rsrc<TB>(k_head, j + 2 < n_tiles ? head_bytes : 0u, j + 2),
        tile_rsrc<TB>(v_head, j + 1 < n_tiles ? head_bytes : 0u, j + 1),
        smem + k_free, smem + v_free, k_off, v_off, wave};
    if (j < n_act) {
      // scores of tile j + 1 || probabilities of tile j, then P V of tile j
      // (past the wave's last tile the scores come from a stale stage and are
      // never used)
      pipeline_block<D, DT, RB, NKB, LPW, LoadEvery<D>::kValue>(
          ld, smem, k_next, v_cur, k_lane, vt_x, qf, cur, ce_cur, m_run, l_run, l_rnd, nxt, acc_o);
      if (j + 1 < n_act) {
        if (tile_needs_mask<RB, NKB, CAUSAL>((j + 1) * Bc, wave_row0, S)) {
          tile_mask<RB, NKB, CAUSAL>(nxt, (j + 1) * Bc, wave_row0, S, c, l32, hi, ce_nxt);
        } else {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) ce_nxt[rb] = c;
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < 2 * LPW; ++n) ld.issue(n);
    }
  };
  for (int j = 0; j < n_tiles; j += 2) {
    step(std::integral_constant<int, 0>{}, j, s_a, ce_a, s_b, ce_b);
    if (j + 1 < n_tiles) step(std::integral_constant<int, 1>{}, j + 1, s_b, ce_b, s_a, ce_a);
  }
  // the last steps' loads (zeros into free stages) must land before the
  // workgroup's LDS is released
  wait_vm_lgkm0<0>();

  // Epilogue: O = O~ / sum(rounded P), rounded once to the input dtype, and
  // lse = ln2 (m + log2 l) from the unrounded sum.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wave_row0 + 32 * rb + l32;
    const float l_tot = xor32_sum(l_run[rb]);
    const float l_o = xor32_sum(l_rnd[rb]);
    if (row < S) {
      const float inv = 1.0f / l_o;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 out = {E::pack2(acc_o[rb][db][4 * g] * inv, acc_o[rb][db][4 * g + 1] * inv),
                             E::pack2(acc_o[rb][db][4 * g + 2] * inv, acc_o[rb][db][4 * g + 3] * inv)};
          *(u32x2*)(o + head + (size_t)row * D + 32 * db + 8 * g + 4 * hi) = out;
        }
      if (hi == 0) lse[(size_t)bh * S + row] = (m_run[rb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

template <int D, int DT, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int S, float scale, int n_cu, hipStream_t stream) {
  using SH = Shape<D>;
  const int n_qt = (S + SH::kBr - 1) / SH::kBr;
  const dim3 grid((unsigned)n_qt, (unsigned)H, (unsigned)B);
  const dim3 block(SH::kThreads);
  // workgroups resident per compute unit: the register budget allows
  // kWavesPerSimd waves per SIMD, i.e. that many 4-wave workgroups
  const long long slots = (long long)n_cu * Tile<D>::kWavesPerSimd * 4 / SH::kWaves;
  const long long n_wg = (long long)n_qt * H * B;
  const int pair_split =
      (CAUSAL && n_qt > 1 && n_wg <= slots) ? (int)(((n_qt + 1) / 2) * (long long)H * B) : 0;
  fa2_fwd_kernel<D, DT, CAUSAL><<<grid, block, 0, stream>>>(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, S,
      scale * kLog2e, pair_split);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_causal(int causal, const void* q, const void* k, const void* v, void* o,
                         float* lse, int B, int H, int S, float scale, int n_cu,
                         hipStream_t stream) {
  return causal ? launch<D, DT, true>(q, k, v, o, lse, B, H, S, scale, n_cu, stream)
                : launch<D, DT, false>(q, k, v, o, lse, B, H, S, scale, n_cu, stream);
}

template <int D>
hipError_t launch_dtype(int dtype, int causal, const void* q, const void* k, const void* v,
                        void* o, float* lse, int B, int H, int S, float scale, int n_cu,
                        hipStream_t stream) {
  return dtype == FA2_F16
             ? launch_causal<D, FA2_F16>(causal, q, k, v, o, lse, B, H, S, scale, n_cu, stream)
             : launch_causal<D, FA2_BF16>(causal, q, k, v, o, lse, B, H, S, scale, n_cu, stream);
}

// ---------------------------------------------------------------------------
// Split-KV attention: Sq query rows against Sk key rows per head, the
// decoding (KV-cache) form that the infra.bea.ai guide says a FlashDecoding
// variant of FlashAttention-2 serves ("When V2 Is Used vs Not"). The queries
// are the last Sq positions of the sequence, so causal masking keeps key j
// for query i iff j <= i + (Sk - Sq).
//
// Few queries give few query tiles, so the key range of each (b, h) is cut
// into chunks that run in parallel; each produces partial softmax state for
// its keys and a second kernel merges them. That is the split-then-combine
// structure of jared-hpc Lecture 6 ("FA2 change 2": parts of the KV range
// computed apart and their (m, l) combined at the end), moved from warps to
// workgroups. The merge is the guide's rescaling algebra applied across
// chunks: with M = max_g m_g and w_g = 2^(m_g - M),
//   O = sum_g w_g O~_g / sum_g w_g l_g,   lse = ln2 (M + log2 sum_g w_g l_g).
//
// The partial kernel runs one wave per workgroup: a 32-row query block (rows
// past Sq are zero and never stored) against one key chunk, streamed through
// a two-stage LDS ring of 32-key tiles by the wave's own LDS-direct loads.
// Decoding reads every K/V byte once per 32 queries, so it is bound by
// memory bandwidth, not by the matrix cores; the kernel keeps the exact
// running row max per tile (no lazy reference point), which also covers rows
// that have no key in a chunk (their partial is m = -inf, l = 0).
//
// Workspace (caller-owned device memory, fp32):
//   part_o  [B*H][n_split][Sq][D]   unnormalised O~ of each chunk
//   part_ml [B*H][n_split][Sq][3]   m (base 2), l (P as computed), l (P as rounded)
// part_ml starts at the part_o size rounded up to 256 bytes.
template <int D> struct SplitTile {
  static constexpr int kBc = 32;
  static constexpr int kTileBytes = kBc * D * 2;
  static constexpr int kLoadsPerWave = kTileBytes / 1024;  // one wave loads the whole tile
  static constexpr int kLdsBytes = 4 * kTileBytes;         // K and V, two stages each
};

size_t splitkv_part_o_bytes(int B, int H, int Sq, int D, int n_split) {
  const size_t b = (size_t)B * H * n_split * Sq * D * sizeof(float);
  return (b + 255) / 256 * 256;
}
size_t splitkv_workspace_bytes(int B, int H, int Sq, int D, int n_split) {
  return splitkv_part_o_bytes(B, H, Sq, D, n_split) + (size_t)B * H * n_split * Sq * 3 * sizeof(float);
}

// Scale every score of the tile and mask keys at or past `lim` (this lane's
// row keeps keys < lim), in the scaled domain.
template <int NKB>
__device__ __forceinline__ void tile_mask_lim(f32x16 (&acc)[1][NKB], int key0, int lim, float c,
                                              int hi) {
  const int rel_lim = lim - (key0 + 4 * hi);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rel = 32 * kb + 8 * (r / 4) + (r % 4);
      acc[0][kb][r] = rel < rel_lim ? acc[0][kb][r] * c : -INFINITY;
    }
}

// O~ += P V for one tile (V at v_stage), V^T operands read two steps ahead.
template <int D, int DT, int RB, int NKB>
__device__ __forceinline__ void tile_pv(const unsigned char* smem, uint32_t v_stage, uint32_t vt_x,
                                        const u32x4 (&pb)[RB][NKB][2],
                                        f32x16 (&acc_o)[RB][D / 32]) {
  using E = Elem<DT>;
  constexpr int CPR = D / 8, NDB = D / 32;
  constexpr int NS2 = NKB * 2 * NDB;
  constexpr int PFV = 2;
  const unsigned char* v_lds = smem + v_stage;
  auto v_read = [&](int st) {
    const int kb = st / (2 * NDB), h = (st / NDB) % 2, db = st % NDB;
    const unsigned char* vp = v_lds + (32 * kb + 16 * h) * CPR * 16 + (vt_x ^ (uint32_t)(64 * db));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
    const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * CPR * 16));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
    return u32x4{lo2[0], lo2[1], up2[0], up2[1]};
  };
  u32x4 vq[PFV];
#pragma unroll
  for (int i = 0; i < PFV; ++i)
    if (i < NS2) vq[i] = v_read(i);
#pragma unroll
  for (int st = 0; st < NS2; ++st) {
    const int kb = st / (2 * NDB), h = (st / NDB) % 2, db = st % NDB;
    const u32x4 a = vq[st % PFV];
    if (st + PFV < NS2) vq[st % PFV] = v_read(st + PFV);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc_o[rb][db] = E::mfma(a, pb[rb][kb][h], acc_o[rb][db]);
  }
}

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(64) void fa2_splitkv_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ part_o, float* __restrict__ part_ml,
    int Sq, int Sk, int n_split, int chunk_keys, float c /* scale * log2(e) */) {
  using ST = SplitTile<D>;
  constexpr int RB = 1, Bc = ST::kBc, NKB = Bc / 32;
  constexpr int CPR = D / 8, TB = ST::kTileBytes, LPW = ST::kLoadsPerWave;
  constexpr int NDS = D / 16, NDB = D / 32;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[ST::kLdsBytes];
  constexpr uint32_t kK0 = 0, kK1 = TB, kV0 = 2 * TB, kV1 = 3 * TB;
  static_assert((TB & (TB - 1)) == 0, "stage ^ TB toggles between the two stages of a ring");

  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x % n_split;
  const int qblk = blockIdx.x / n_split;
  const int bh = blockIdx.y + gridDim.y * blockIdx.z;
  const int q0 = qblk * 32;
  const int row = q0 + l32;
  const int off = Sk - Sq;  // position of query 0 in the sequence

  // this chunk's keys, cut short where no row of the block can see them
  const int k_begin = split * chunk_keys;
  int k_end = min(k_begin + chunk_keys, Sk);
  if (CAUSAL) k_end = min(k_end, min(q0 + 31, Sq - 1) + off + 1);
  // keys this lane's row keeps, within the chunk
  const int row_lim = CAUSAL ? min(k_end, row + off + 1) : k_end;

  u32x4 qf[RB][NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    qf[0][s] = u32x4{0, 0, 0, 0};
    if (row < Sq) qf[0][s] = *(const u32x4*)(q + ((size_t)bh * Sq + row) * D + 16 * s + 8 * hi);
  }

  const uint32_t head_bytes = (uint32_t)Sk * D * 2;
  const unsigned char* k_head = (const unsigned char*)(k + (size_t)bh * Sk * D);
  const unsigned char* v_head = (const unsigned char*)(v + (size_t)bh * Sk * D);
  uint32_t k_off[LPW], v_off[LPW];
  tile_load_offsets<D, LPW, false>(0, lane, k_off);
  tile_load_offsets<D, LPW, true>(0, lane, v_off);
  const uint32_t k_lane = (uint32_t)(l32 * CPR * 16 + 16 * (hi ^ swz_k<D>(l32)));
  const int vt_row = 4 * hi + (lane & 15) / 4;
  const int vt_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const uint32_t vt_x = (uint32_t)((vt_row * CPR + vt_chunk) * 16 + 8 * (lane & 1) +
                                   64 * (swz_v<D>(vt_row) >> 2));

  f32x16 acc_o[RB][NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[0][db] = f32x16{};
  float m_run[RB] = {-INFINITY}, l_run[RB] = {0.f}, l_rnd[RB] = {0.f};
  const float one[RB] = {1.f};

  const int t_first = k_begin / Bc;
  const int n_t = k_end > k_begin ? (k_end - k_begin + Bc - 1) / Bc : 0;
  if (n_t > 0) {
    load_tile<LPW, TB>(k_head, head_bytes, t_first, smem + kK0, 0, k_off);
    load_tile<LPW, TB>(v_head, head_bytes, t_first, smem + kV0, 0, v_off);
  }
  for (int t = 0; t < n_t; ++t) {
    const uint32_t ks = (t & 1) ? kK1 : kK0, vs = (t & 1) ? kV1 : kV0;
    // tile t has landed, and every LDS read of tile t - 1 is done, so its
    // stages can take tile t + 1
    wait_vm_lgkm0<0>();
    if (t + 1 < n_t) {
      load_tile<LPW, TB>(k_head, head_bytes, t_first + t + 1, smem + (ks ^ TB), 0, k_off);
      load_tile<LPW, TB>(v_head, head_bytes, t_first + t + 1, smem + (vs ^ TB), 0, v_off);
    }
    f32x16 sc[RB][NKB];
    tile_scores<D, DT, RB, NKB>(smem, ks, k_lane, qf, sc);
    tile_mask_lim<NKB>(sc, (t_first + t) * Bc, row_lim, c, hi);
    float tm[RB];
    tile_max<RB, NKB>(sc, one, tm);
    // exact running max; a row with no key so far keeps m = -inf and uses 0
    // as its exponent reference
    const float m_new = fmaxf(m_run[0], tm[0]);
    const float m_ref[RB] = {m_new == -INFINITY ? 0.f : m_new};
    const float alpha = m_run[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - m_ref[0]);
    l_run[0] *= alpha;
    l_rnd[0] *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[0][db] *= alpha;
    m_run[0] = m_new;
    float tsum[RB], trnd[RB];
    u32x4 pb[RB][NKB][2];
    tile_probs<DT, RB, NKB>(sc, one, m_ref, tsum, trnd, pb);
    l_run[0] += tsum[0];
    l_rnd[0] += trnd[0];
    tile_pv<D, DT, RB, NKB>(smem, vs, vt_x, pb, acc_o);
  }

  // partial state of rows < Sq
  const float lr = xor32_sum(l_run[0]), lo = xor32_sum(l_rnd[0]);
  if (row < Sq) {
    const size_t prow = ((size_t)bh * n_split + split) * Sq + row;
    float* po = part_o + prow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 val = {acc_o[0][db][4 * g], acc_o[0][db][4 * g + 1], acc_o[0][db][4 * g + 2],
                            acc_o[0][db][4 * g + 3]};
        *(float4*)(po + 32 * db + 8 * g + 4 * hi) = val;
      }
    if (hi == 0) {
      part_ml[prow * 3 + 0] = m_run[0];
      part_ml[prow * 3 + 1] = lr;
      part_ml[prow * 3 + 2] = lo;
    }
  }
}

// Merge the chunks of each query row: one wave per row, D / 64 columns per
// lane.
template <int D, int DT>
__global__ __launch_bounds__(256) void fa2_splitkv_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, uint16_t* __restrict__ o,
    float* __restrict__ lse, int n_rows, int Sq, int n_split) {
  using E = Elem<DT>;
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;  // whole waves leave together
  const int bh = r / Sq, i = r % Sq;
  const size_t first = (size_t)bh * n_split * Sq + i;  // partial row of chunk 0
  float mx = -INFINITY;
  for (int g = 0; g < n_split; ++g) {
    const float* ml = part_ml + (first + (size_t)g * Sq) * 3;
    if (ml[2] > 0.f) mx = fmaxf(mx, ml[0]);
  }
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  float den = 0.f, lsum = 0.f;
  for (int g = 0; g < n_split; ++g) {
    const size_t prow = first + (size_t)g * Sq;
    const float* ml = part_ml + prow * 3;
    const float w = ml[2] > 0.f ? __builtin_amdgcn_exp2f(ml[0] - mx) : 0.f;
    lsum += w * ml[1];
    den += w * ml[2];
    const float* po = part_o + prow * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] += w * po[lane * PER + e];
  }
  const float inv = 1.0f / den;
  uint16_t* orow = o + (size_t)r * D;
#pragma unroll
  for (int e = 0; e < PER; e += 2) {
    const uint32_t pk = E::pack2(num[e] * inv, (e + 1 < PER ? num[e + 1] : 0.f) * inv);
    if (PER >= 2) {
      *(uint32_t*)(orow + lane * PER + e) = pk;
    } else {
      orow[lane] = (uint16_t)(pk & 0xffffu);
    }
  }
  if (lane == 0) lse[r] = (mx + __builtin_amdgcn_logf(lsum)) * kLn2;
}

// Key chunks per (b, h) for a launch: enough workgroups for about two on
// every compute unit (decoding is bandwidth bound; each one-wave workgroup
// keeps a K and a V tile in flight), each chunk at least 4 tiles long.
int splitkv_default_splits(int B, int H, int Sq, int Sk, int n_cu) {
  const long long n_qblk = (Sq + 31) / 32;
  const long long n_tiles = (Sk + SplitTile<64>::kBc - 1) / SplitTile<64>::kBc;
  // measured on decode shapes: more, shorter chunks lose bandwidth
  const long long target = 2LL * n_cu;
  long long want = (target + (long long)B * H * n_qblk - 1) / ((long long)B * H * n_qblk);
  const long long cap = n_tiles / 4 > 0 ? n_tiles / 4 : 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  if (want > 1024) want = 1024;
  return (int)want;
}

template <int D, int DT, bool CAUSAL>
hipError_t launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int H, int Sq, int Sk, float scale, int n_split, void* ws,
                          hipStream_t stream) {
  using ST = SplitTile<D>;
  // chunks of whole tiles; trailing splits that would be empty are dropped
  const int n_tiles = (Sk + ST::kBc - 1) / ST::kBc;
  const int chunk_tiles = (n_tiles + n_split - 1) / n_split;
  const int n_eff = (n_tiles + chunk_tiles - 1) / chunk_tiles;
  const int n_qblk = (Sq + 31) / 32;
  float* part_o = (float*)ws;
  float* part_ml = (float*)((char*)ws + splitkv_part_o_bytes(B, H, Sq, D, n_eff));
  const dim3 grid((unsigned)(n_eff * n_qblk), (unsigned)H, (unsigned)B);
  fa2_splitkv_partial_kernel<D, DT, CAUSAL><<<grid, dim3(64), 0, stream>>>(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, part_o, part_ml, Sq, Sk, n_eff,
      chunk_tiles * ST::kBc, scale * kLog2e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_rows = B * H * Sq;
  fa2_splitkv_combine_kernel<D, DT><<<dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream>>>(
      part_o, part_ml, (uint16_t*)o, lse, n_rows, Sq, n_eff);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_splitkv_causal(int causal, const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int H, int Sq, int Sk, float scale,
                                 int n_split, void* ws, hipStream_t stream) {
  return causal ? launch_splitkv<D, DT, true>(q, k, v, o, lse, B, H, Sq, Sk, scale, n_split, ws, stream)
                : launch_splitkv<D, DT, false>(q, k, v, o, lse, B, H, Sq, Sk, scale, n_split, ws, stream);
}

template <int D>
hipError_t launch_splitkv_dtype(int dtype, int causal, const void* q, const void* k, const void* v,
                                void* o, float* lse, int B, int H, int Sq, int Sk, float scale,
                                int n_split, void* ws, hipStream_t stream) {
  return dtype == FA2_F16 ? launch_splitkv_causal<D, FA2_F16>(causal, q, k, v, o, lse, B, H, Sq, Sk,
                                                               scale, n_split, ws, stream)
                          : launch_splitkv_causal<D, FA2_BF16>(causal, q, k, v, o, lse, B, H, Sq,
                                                                Sk, scale, n_split, ws, stream);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Per-device verdict on whether the device is gfx950 (0 unknown, 1 yes,
// 2 no) and its compute-unit count, both cached on first use.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];
std::atomic<int> g_device_cus[kMaxDevices];

int check_device(int* n_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FA2_ERR_NO_DEVICE;
  }
  int verdict = g_device_ok[dev].load(std::memory_order_acquire);
  if (verdict == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FA2_ERR_NO_DEVICE;
    }
    verdict = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                            std::memory_order_relaxed);
    g_device_ok[dev].store(verdict, std::memory_order_release);
  }
  *n_cu = g_device_cus[dev].load(std::memory_order_relaxed);
  return verdict == 1 ? FA2_OK : FA2_ERR_NO_DEVICE;
}

}  // namespace

extern "C" int fa2_supported(int D, int dtype) {
  return (D == 64 || D == 128 || D == 256) && (dtype == FA2_F16 || dtype == FA2_BF16);
}

extern "C" int fa2_rows_per_workgroup(int D) {
  switch (D) {
    case 64: return Shape<64>::kBr;
    case 128: return Shape<128>::kBr;
    case 256: return Shape<256>::kBr;
    default: return 0;
  }
}

extern "C" const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL: return "a tensor pointer is NULL";
    case FA2_ERR_SHAPE:
      return "B, H and S must be >= 1, B and H <= 65535, one head (S*D elements) under 2 GiB, "
             "and the grid within 2^31 workgroups";
    case FA2_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA2_ERR_DTYPE: return "dtype must be FA2_F16 or FA2_BF16";
    case FA2_ERR_ALIGN: return "q, k, v and o must be 16-byte aligned and lse 4-byte aligned";
    case FA2_ERR_SCALE: return "scale must be finite and >= 0";
    case FA2_ERR_NO_DEVICE: return "no current HIP device, or it is not a gfx950 (MI355X)";
    case FA2_ERR_LAUNCH: return "the HIP runtime reported an error at kernel launch";
    case FA2_ERR_ALIAS: return "o or lse overlaps q, k, v or each other (or the workspace overlaps any of them)";
    case FA2_ERR_WORKSPACE:
      return "the workspace is NULL, not 16-byte aligned, or smaller than fa2_splitkv_workspace_bytes";
    default: return "unknown fa2 status";
  }
}

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int S, int D, int causal, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (B < 1 || H < 1 || S < 1 || B > 65535 || H > 65535) return FA2_ERR_SHAPE;
  if (dtype != FA2_F16 && dtype != FA2_BF16) return FA2_ERR_DTYPE;
  if (!(D == 64 || D == 128 || D == 256)) return FA2_ERR_HEADDIM;
  // One head, plus one tile of keys past its end, is addressed with 32-bit
  // byte offsets (buffer loads): keep it under 2 GiB.
  if (((long long)S + 256) * D * 2 > (long long)INT32_MAX) return FA2_ERR_SHAPE;
  const unsigned long long elems =
      (unsigned long long)B * (unsigned long long)H * (unsigned long long)S * (unsigned long long)D;
  // the kernel linearises its block index in a 32-bit int
  const int rows = fa2_rows_per_workgroup(D);
  const unsigned long long blocks = (((unsigned long long)S + rows - 1) / rows) *
                                    (unsigned long long)H * (unsigned long long)B;
  if (blocks > (unsigned long long)INT32_MAX) return FA2_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA2_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA2_ERR_ALIGN;
  if (!std::isfinite(scale) || scale < 0.f) return FA2_ERR_SCALE;
  const size_t tensor_bytes = (size_t)elems * 2;
  const size_t lse_bytes = (size_t)B * H * S * sizeof(float);
  if (overlaps(o, tensor_bytes, q, tensor_bytes) || overlaps(o, tensor_bytes, k, tensor_bytes) ||
      overlaps(o, tensor_bytes, v, tensor_bytes) || overlaps(lse, lse_bytes, q, tensor_bytes) ||
      overlaps(lse, lse_bytes, k, tensor_bytes) || overlaps(lse, lse_bytes, v, tensor_bytes) ||
      overlaps(lse, lse_bytes, o, tensor_bytes))
    return FA2_ERR_ALIAS;
  int n_cu = 0;
  const int dev = check_device(&n_cu);
  if (dev != FA2_OK) return dev;

  (void)hipGetLastError();  // start from a clean error state
  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  switch (D) {
    case 64: err = launch_dtype<64>(dtype, causal, q, k, v, o, lse, B, H, S, scale, n_cu, st); break;
    case 128:
      err = launch_dtype<128>(dtype, causal, q, k, v, o, lse, B, H, S, scale, n_cu, st);
      break;
    default:
      err = launch_dtype<256>(dtype, causal, q, k, v, o, lse, B, H, S, scale, n_cu, st);
      break;
  }
  return err == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

extern "C" int fa2_splitkv_splits(int B, int H, int Sq, int Sk) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return 1;
  int n_cu = 0;
  if (check_device(&n_cu) != FA2_OK) n_cu = 256;
  return splitkv_default_splits(B, H, Sq, Sk, n_cu);
}

extern "C" size_t fa2_splitkv_workspace_bytes(int B, int H, int Sq, int Sk, int D, int n_split) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || n_split < 0) return 0;
  if (!(D == 64 || D == 128 || D == 256)) return 0;
  if (n_split == 0) n_split = fa2_splitkv_splits(B, H, Sq, Sk);
  return splitkv_workspace_bytes(B, H, Sq, D, n_split);
}

extern "C" int fa2_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Sq, int Sk, int D, int causal, float scale,
                               int dtype, int n_split, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || B > 65535 || H > 65535 || n_split < 0)
    return FA2_ERR_SHAPE;
  if (causal && Sq > Sk) return FA2_ERR_SHAPE;  // the first queries would have no key
  if (dtype != FA2_F16 && dtype != FA2_BF16) return FA2_ERR_DTYPE;
  if (!(D == 64 || D == 128 || D == 256)) return FA2_ERR_HEADDIM;
  // one head of K or V, plus a tile past its end, within 32-bit byte offsets;
  // query rows of the whole call indexed in 32 bits
  if (((long long)Sk + 256) * D * 2 > (long long)INT32_MAX) return FA2_ERR_SHAPE;
  if ((long long)B * H * Sq > (long long)INT32_MAX / 4) return FA2_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA2_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA2_ERR_ALIGN;
  if (!std::isfinite(scale) || scale < 0.f) return FA2_ERR_SCALE;
  // the default split count needs the device's size; an explicit one lets
  // every argument be checked before the device is looked up
  int n_cu = 0;
  bool device_checked = false;
  if (n_split == 0) {
    const int dev = check_device(&n_cu);
    if (dev != FA2_OK) return dev;
    device_checked = true;
    n_split = splitkv_default_splits(B, H, Sq, Sk, n_cu);
  }
  if (n_split > 65536) return FA2_ERR_SHAPE;
  const size_t need = splitkv_workspace_bytes(B, H, Sq, D, n_split);
  if (!workspace || ((uintptr_t)workspace & 15u) || workspace_bytes < need) return FA2_ERR_WORKSPACE;
  const size_t q_bytes = (size_t)B * H * Sq * D * 2, kv_bytes = (size_t)B * H * Sk * D * 2;
  const size_t lse_bytes = (size_t)B * H * Sq * sizeof(float);
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, kv_bytes) ||
      overlaps(o, q_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, q_bytes) ||
      overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
      overlaps(lse, lse_bytes, o, q_bytes) || overlaps(workspace, need, q, q_bytes) ||
      overlaps(workspace, need, k, kv_bytes) || overlaps(workspace, need, v, kv_bytes) ||
      overlaps(workspace, need, o, q_bytes) || overlaps(workspace, need, lse, lse_bytes))
    return FA2_ERR_ALIAS;
  if (!device_checked) {
    const int dev = check_device(&n_cu);
    if (dev != FA2_OK) return dev;
  }

  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  switch (D) {
    case 64:
      err = launch_splitkv_dtype<64>(dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale, n_split,
                                     workspace, st);
      break;
    case 128:
      err = launch_splitkv_dtype<128>(dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale, n_split,
                                      workspace, st);
      break;
    default:
      err = launch_splitkv_dtype<256>(dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale, n_split,
                                      workspace, st);
      break;
  }
  return err == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}
