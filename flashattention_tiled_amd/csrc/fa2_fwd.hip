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
// The matrix-core formulation, lane layouts and LDS staging shared with
// the split-KV kernels are described in fa2_tile.h.

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "fa2_plan.h"
#include "fa2_tile.h"
#include "fa2_host.h"
#include "fa2_combine.h"

using fa2_host::check_device;
using fa2_host::extent_bytes;
using fa2_host::overlaps;
using fa2_host::elements_fit_int64;
using fa2_host::rows_disjoint;

namespace {

// Per-workgroup timeline, a measurement aid compiled in only with
// -DFA2_TIMELINE (into a library of its own, see timeline.py): wave 0 of
// each of the first kTimelineWgs workgroups of a launch records the 100 MHz
// real-time clock at its start, after its prologue's barrier (at its first
// key tile on the unpipelined path), after its key loop and at its end; its
// compute unit's hardware ids (HW_ID, and XCC_ID above bit 32); and its
// query tile, (b, h) and key-loop steps. Vector stores of thread 0.
#ifdef FA2_TIMELINE
constexpr int kTimelineWgs = 16384, kTimelineSlots = 8;
__device__ unsigned long long fa2_tl[kTimelineWgs * kTimelineSlots];
#define FA2_TL(lin, slot, value)                                                  \
  do {                                                                            \
    if ((lin) < kTimelineWgs && threadIdx.x == 0)                                 \
      fa2_tl[(size_t)(lin) * kTimelineSlots + (slot)] = (unsigned long long)(value); \
  } while (0)
#define FA2_TL_NOW() __builtin_amdgcn_s_memrealtime()
#else
#define FA2_TL(lin, slot, value) \
  do {                           \
  } while (0)
#endif

constexpr float kSumLimit = 4096.0f;  // lazy-rescale threshold on a lane's tile sum of P
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

// One step of the unpipelined loop on tile j (kPipelined = 0): its scores
// on the matrix cores, with this wave's share of the loads of tile
// j + NST - 1 issued between them; the mask; on the wave's first tile the
// reference max; P and the lazy-rescale test (and, rarely, the redo); then
// the P V product. One score buffer instead of two; the SIMD's other waves
// fill the gaps this leaves on the matrix cores and the vector unit.
template <int D, int DT, int RB, int NKB, int LPW, int LEVERY, bool CAUSAL>
__device__ __forceinline__ void serial_block(
    const StepLoads<LPW>& ld, const unsigned char* smem, uint32_t k_stage, uint32_t v_stage,
    uint32_t k_lane, uint32_t vt_x, const u32x4 (&qf)[RB][D / 16], int key0, int row0, int S,
    float c, int l32, int hi, bool first, float (&m_run)[RB], float (&l_run)[RB],
    float (&l_rnd)[RB], f32x16 (&acc_o)[RB][D / 32]) {
  using E = Elem<DT>;
  constexpr int CPR = D / 8, NDS = D / 16, NDB = D / 32;
  constexpr int NS1 = NKB * NDS;       // score k-steps
  constexpr int NS2 = NKB * 2 * NDB;   // P V steps
  constexpr int PFK = 2, PFV = 2;      // operand read-ahead (steps)
  static_assert(LEVERY == 0 || (NS1 + LEVERY - 1) / LEVERY >= 2 * LPW,
                "the load spacing must leave a k-step for every load block");

  f32x16 sc[RB][NKB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sc[rb][kb] = f32x16{};
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
#pragma unroll
  for (int st = 0; st < NS1; ++st) {
    const int kb = st / NDS, s = st % NDS;
    if (LEVERY == 0) {
      if (st == 0)
#pragma unroll
        for (int n = 0; n < 2 * LPW; ++n) ld.issue(n);
    } else if (st % LEVERY == 0 && st / LEVERY < 2 * LPW) {
      ld.issue(st / LEVERY);
      __builtin_amdgcn_sched_barrier(0x786);
    }
    const u32x4 a = kq[st % PFK];
    if (st + PFK < NS1) kq[st % PFK] = k_read(st + PFK);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sc[rb][kb] = E::mfma(a, qf[rb][s], sc[rb][kb]);
  }

  float ce[RB];
  if (tile_needs_mask<RB, NKB, CAUSAL>(key0, row0, S)) {
    tile_mask<RB, NKB, CAUSAL>(sc, key0, row0, S, c, l32, hi, ce);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ce[rb] = c;
  }
  // the first tile holds an unmasked key for every row (its first key is at
  // most the tile's first row), so m is finite from here on
  if (first) tile_max<RB, NKB>(sc, ce, m_run);
  const unsigned char* v_lds = smem + v_stage;
  auto v_read = [&](int st) {
    const int kb = st / (2 * NDB), h = (st / NDB) % 2, db = st % NDB;
    const unsigned char* vp = v_lds + (32 * kb + 16 * h) * CPR * 16 + (vt_x ^ (uint32_t)(64 * db));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
    const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * CPR * 16));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
    return u32x4{lo2[0], lo2[1], up2[0], up2[1]};
  };
  float tsum[RB], trnd[RB];
  u32x4 pb[RB][NKB][2];
  tile_probs<DT, RB, NKB>(sc, ce, m_run, tsum, trnd, pb);
  bool big = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) big |= !(tsum[rb] <= kSumLimit);
  if (__builtin_amdgcn_ballot_w64(big) != 0) {
    // rows whose m does not move recompute the same P
    float tm[RB];
    tile_max<RB, NKB>(sc, ce, tm);
    raise_max<RB, NDB>(tm, m_run, l_run, l_rnd, acc_o);
    tile_probs<DT, RB, NKB>(sc, ce, m_run, tsum, trnd, pb);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += tsum[rb];
    l_rnd[rb] += trnd[rb];
  }

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

// Element strides of the batch, head and sequence dims of Q, K, V and O (the
// head dim is contiguous). Read only by the STRIDED kernels; the others use
// the contiguous (B, H, S, D) layout.
struct Strides {
  long long qb, qh, qs, kb, kh, ks, vb, vh, vs, ob, oh, os;
};

template <int D, int DT, bool CAUSAL, bool STRIDED, int ALT>
__global__ __launch_bounds__((Shape<D, ALT>::kThreads), (Tile<D, ALT>::kWavesPerSimd)) void fa2_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int S, float c /* scale * log2(e) */, int pair_split, Strides st, KeySplit ks, int tk_from,
    unsigned int* __restrict__ tk) {
  using SH = Shape<D, ALT>;
  constexpr int RB = SH::kRB, Bc = SH::kBc, Br = SH::kBr;
  constexpr int CPR = SH::kChunksPerRow, TB = SH::kTileBytes, LPW = SH::kLoadsPerWave;
  constexpr int NKB = Bc / 32;  // 32-key blocks per tile
  constexpr int NDS = D / 16;   // k-steps of 16 over the head dim (S^T product)
  constexpr int NDB = D / 32;   // 32-wide head-dim blocks of O^T

  constexpr int NST = SH::kStages;
  constexpr int KG = SH::kKeyGroups, GW = SH::kGroupWaves;
  static_assert(KG == 1 || RB == 1, "key groups take one row block per wave");

  // Per key group: a K ring (stages 0 .. NST - 1) then a V ring (stages
  // 0 .. NST - 1), TB bytes each.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SH::kLdsBytes];
  constexpr uint32_t kK0 = 0, kK1 = TB, kV0 = NST * TB, kV1 = (NST + 1) * TB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  // the wave's key group and its place in the group, which fixes its rows
  // and its share of the group's tile loads
  const int grp = KG > 1 ? wave_uniform(wave / GW) : 0;
  const int gw = KG > 1 ? wave_uniform(wave % GW) : wave;
  unsigned char* const ring = smem + grp * SH::kRingBytes;

  // Workgroup -> (query tile, batch*head). Tiles are taken in descending
  // query-tile order across all heads, so under causal masking the longest
  // tiles start first; the workgroups of one (b, h) are H*B apart in launch
  // order, which keeps them on one XCD when H*B is a multiple of 8. When the
  // whole causal grid is resident at once (pair_split > 0, set by the host),
  // the workgroups from pair_split on take the query tiles in ascending
  // order instead, so that the second workgroup a compute unit receives is
  // a light tile beside its heavy first one.
  // Under a key split the grid's x dimension runs over work items instead,
  // each one key chunk (of ct tiles from tile t0) of one query tile.
  // With tk (multi-round grids), the workgroups from tk_from on take their
  // place in that order from the counter instead of from blockIdx: in the
  // order they start, so that the XCDs that run faster take more of the
  // short tiles at the end. The last of them wraps the counter back to 0.
  const int n_bh = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  int lin_t = lin;
  if (lin >= tk_from) {
    const int n_wg = (int)(gridDim.x * gridDim.y * gridDim.z);
    unsigned int* const got = (unsigned int*)smem;  // before the prologue's loads
    if (threadIdx.x == 0) *got = atomicInc(tk, (unsigned int)(n_wg - tk_from - 1));
    wait_vm_lgkm0<63>();
    workgroup_barrier();
    lin_t = tk_from + wave_uniform((int)*got);
    wait_vm_lgkm0<63>();
    workgroup_barrier();
  }
  const int bh = lin_t % n_bh;
  FA2_TL(lin, 0, FA2_TL_NOW());
  FA2_TL(lin, 4, (unsigned long long)(unsigned)__builtin_amdgcn_s_getreg(0xf804) |
                     ((unsigned long long)(unsigned)__builtin_amdgcn_s_getreg(0xf814) << 32));
  int qt, chunk = 0;
  if (ks.ct > 0) {
    split_item(lin / n_bh, ks, CAUSAL, qt, chunk);
  } else {
    const int n_qt = gridDim.x;
    qt = (pair_split > 0 && lin >= pair_split) ? (lin - pair_split) / n_bh
                                                : n_qt - 1 - lin_t / n_bh;
  }
  const int t0 = chunk * ks.ct;  // first key tile
  // chunks of this query tile (more than one: the rows leave partials)
  const int n_chunks = ks.ct == 0 ? 1 : CAUSAL ? qt / ks.m + 1 : ks.n_split;
  const int q0 = qt * Br;
  const int wave_row0 = q0 + gw * SH::kRowsPerWave;

  // This (b, h)'s Q, K, V and O, as element offsets from the base pointers,
  // their row strides in elements, and K's and V's row strides in bytes.
  size_t q_at, k_at, v_at, o_at, q_rs, o_rs;
  uint32_t k_rb, v_rb;
  if constexpr (STRIDED) {
    const int b = bh / (int)gridDim.y, h = bh - b * (int)gridDim.y;
    q_at = (size_t)(b * st.qb + h * st.qh);
    k_at = (size_t)(b * st.kb + h * st.kh);
    v_at = (size_t)(b * st.vb + h * st.vh);
    o_at = (size_t)(b * st.ob + h * st.oh);
    q_rs = (size_t)st.qs;
    o_rs = (size_t)st.os;
    k_rb = (uint32_t)st.ks * 2u;
    v_rb = (uint32_t)st.vs * 2u;
  } else {
    const size_t head = (size_t)bh * (size_t)S * D;
    q_at = k_at = v_at = o_at = head;
    q_rs = o_rs = D;
    k_rb = v_rb = 2u * D;
  }

  // Q^T operands: lane holds Q[row][16 s + 8 hi .. +7] of each of its rows,
  // loaded here or through LDS in the prologue (SH::kQStaged,
  // SH::kQThroughRing), in whole 1 KiB blocks and, with key groups, once for
  // both groups.
  constexpr bool QS = SH::kQStaged, QS4 = SH::kQThroughRing;
  u32x4 qf[RB][NDS];
  if constexpr (!QS && !QS4) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = wave_row0 + 32 * rb + l32;
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        qf[rb][s] = u32x4{0, 0, 0, 0};
        if (row < S) qf[rb][s] = *(const u32x4*)(q + q_at + (size_t)row * q_rs + 16 * s + 8 * hi);
      }
    }
  }

  // K and V of this head, loaded through bounds-checked buffers that end
  // with row S - 1 (loads of rows >= S return zero).
  const int k_cap = rows_within_2g(k_rb), v_cap = rows_within_2g(v_rb);
  const unsigned char* k_head = (const unsigned char*)(k + k_at);
  const unsigned char* v_head = (const unsigned char*)(v + v_at);
  uint32_t k_off[LPW], v_off[LPW];
  if constexpr (STRIDED) {
    tile_load_offsets_strided<D, LPW, false>(gw, lane, k_rb, k_off);
    tile_load_offsets_strided<D, LPW, true>(gw, lane, v_rb, v_off);
  } else {
    tile_load_offsets<D, LPW, false>(gw, lane, k_off);
    tile_load_offsets<D, LPW, true>(gw, lane, v_off);
  }
  // buffer for key tile t of K or V (limit 0: a tile that is not needed,
  // whose loads return zero)
  auto k_tile = [&](int rows, int t) { return tile_rsrc_rows(k_head, rows, t * Bc, k_rb, k_cap); };
  auto v_tile = [&](int rows, int t) { return tile_rsrc_rows(v_head, rows, t * Bc, v_rb, v_cap); };
  // Q through LDS: a key tile's worth of Q rows from row r (rows >= S read
  // as zero), loaded in K's LDS layout with offsets for Q's row stride
  const uint32_t q_rb = (uint32_t)q_rs * 2u;
  [[maybe_unused]] uint32_t q_off[LPW];
  if constexpr (QS || QS4) {
    if constexpr (STRIDED)
      tile_load_offsets_strided<D, LPW, false>(gw, lane, q_rb, q_off);
    else
#pragma unroll
      for (int i = 0; i < LPW; ++i) q_off[i] = k_off[i];
  }
  [[maybe_unused]] auto q_rows = [&](int r) {
    return tile_rsrc_rows((const unsigned char*)(q + q_at), S, r, q_rb, rows_within_2g(q_rb));
  };

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
  const int t_all = (kv_end + Bc - 1) / Bc;
  const int t_stop = ks.ct > 0 ? min(t_all, t0 + ks.ct) : t_all;
  // The key tiles of this wave's group, g_t0 .. g_stop - 1. With two key
  // groups, group 0 takes the first h tiles and group 1 the rest (under
  // causal masking, the diagonal ones). h is at most the number of tiles
  // that end at or before the query tile's first row, so that the first
  // tile of either group holds a key for every row; for the first query
  // tile that is none, and group 1 takes them all. Both groups run n_steps
  // pipeline steps (the shorter one's last step only loads zeros) so that
  // they meet at every barrier.
  int g_t0 = t0, g_stop = t_stop, n_steps = t_stop - t0, h_split = 0;
  if constexpr (KG > 1) {
    const int n = t_stop - t0;
    h_split = CAUSAL ? max(0, min(n / 2, q0 / Bc - t0)) : n / 2;
    g_t0 = grp ? t0 + h_split : t0;
    g_stop = grp ? t_stop : t0 + h_split;
    n_steps = max(h_split, n - h_split);
  }
  const int n_tiles = g_stop - g_t0;  // tiles the group loads, from g_t0
  // tiles this wave computes (under causal masking the later tiles of the
  // workgroup lie wholly above this wave's rows); at least one when the
  // group has any, as g_t0 B_c is at most the tile's first row
  const int n_act =
      CAUSAL ? min(g_stop, (wave_row0 + SH::kRowsPerWave + Bc - 1) / Bc) - g_t0 : n_tiles;

  // Software pipeline. Iteration j computes the scores of tile j + 1 on the
  // matrix cores while the vector unit turns tile j's scores into P, then the
  // P V product of tile j.
  // At its top every load issued in iteration j - NST + 1 (K of tile j + 1,
  // V of tile j) has landed -- this wave's later loads, 2 LPW per iteration,
  // may still be in flight -- and after the barrier every wave is done with
  // iteration j - 1, so K of tile j + NST goes into tile j's K stage and V of
  // tile j + NST - 1 into tile j - 1's V stage. Tile t sits in stage t % NST
  // of each ring.
  if constexpr (!SH::kPipelined) {
    // Unpipelined: iteration j computes tile j from stage j % NST, after
    // every load of iteration j - NST + 1 (tile j) has landed and every wave
    // is done with iteration j - 1, whose stage then takes tile j + NST - 1.
    if constexpr (QS4) {
      // Q's rows 32 i .. 32 i + 31 in K's layout in stage region i (K0, K1,
      // V0, V1), whole 1 KiB blocks; wave w reads region w, then the rings
      // take their first tiles
#pragma unroll
      for (int i = 0; i < 4; ++i) load_tile_rsrc<LPW>(q_rows(q0 + Bc * i), ring + i * TB, gw, q_off);
      wait_vm_lgkm0<0>();
      workgroup_barrier();
      const uint32_t q_base = (uint32_t)(gw * TB) + k_lane;
#pragma unroll
      for (int s = 0; s < NDS; ++s) qf[0][s] = *(const u32x4*)(smem + (q_base ^ (uint32_t)(32 * s)));
      wait_vm_lgkm0<0>();
      workgroup_barrier();
    }
#pragma unroll
    for (int i = 0; i + 1 < NST; ++i) {
      load_tile_rsrc<LPW>(k_tile(i < n_tiles ? S : 0, g_t0 + i), ring + kK0 + i * TB, gw, k_off);
      load_tile_rsrc<LPW>(v_tile(i < n_tiles ? S : 0, g_t0 + i), ring + kV0 + i * TB, gw, v_off);
    }
    FA2_TL(lin, 1, FA2_TL_NOW());
    auto step_s = [&](auto sj_c, int j) {
      constexpr int SJ = decltype(sj_c)::value, SF = (SJ + NST - 1) % NST;
      wait_vm_lgkm0<(NST - 2) * 2 * LPW>();
      workgroup_barrier();
      const int tn = j + NST - 1;
      const StepLoads<LPW> ld{k_tile(tn < n_tiles ? S : 0, g_t0 + tn),
                              v_tile(tn < n_tiles ? S : 0, g_t0 + tn),
                              ring + kK0 + SF * TB, ring + kV0 + SF * TB, k_off, v_off, gw};
      if (j < n_act) {
        serial_block<D, DT, RB, NKB, LPW, Tile<D, ALT>::kLoadEvery, CAUSAL>(
            ld, ring, kK0 + SJ * TB, kV0 + SJ * TB, k_lane, vt_x, qf, (g_t0 + j) * Bc, wave_row0,
            S, c, l32, hi, j == 0, m_run, l_run, l_rnd, acc_o);
      } else {
#pragma unroll
        for (int n = 0; n < 2 * LPW; ++n) ld.issue(n);
      }
    };
    auto step_su = [&](auto u, int j0) {
      constexpr int UU = decltype(u)::value;
      if constexpr (UU < NST)
        if (UU == 0 || j0 + UU < n_steps) step_s(std::integral_constant<int, UU>{}, j0 + UU);
    };
    for (int j = 0; j < n_steps; j += NST) {
      step_su(std::integral_constant<int, 0>{}, j);
      step_su(std::integral_constant<int, 1>{}, j);
      step_su(std::integral_constant<int, 2>{}, j);
      step_su(std::integral_constant<int, 3>{}, j);
    }
    static_assert(NST <= 4, "unroll");
  } else {
    // Q's loads stay ahead of the tile loads, so that the wait below for the
    // first K tile covers them while V of tile 0 and K of tile 1 still land
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QS) {
      // Q rows Bc h .. Bc h + Bc - 1 of the tile (half h) in K's LDS layout:
      // with key groups group g loads half g into the second stage of its V
      // ring, else every wave loads its share of both halves, half 1 into
      // the region after the ring. The first step refills that V stage only
      // after every wave has read Q (its top barrier).
      if constexpr (KG > 1) {
        load_tile_rsrc<LPW>(q_rows(q0 + Bc * grp), ring + kV1, gw, q_off);
      } else {
        load_tile_rsrc<LPW>(q_rows(q0), smem + kV1, gw, q_off);
        load_tile_rsrc<LPW>(q_rows(q0 + Bc), smem + SH::kRingBytes, gw, q_off);
      }
    }
    load_tile_rsrc<LPW>(k_tile(n_tiles > 0 ? S : 0, g_t0), ring + kK0, gw, k_off);
    if constexpr (NST == 2) {
      load_tile_rsrc<LPW>(v_tile(n_tiles > 0 ? S : 0, g_t0), ring + kV0, gw, v_off);
      if (n_tiles > 1) load_tile_rsrc<LPW>(k_tile(S, g_t0 + 1), ring + kK1, gw, k_off);
    } else {
      // the loads iterations 1 - NST .. -1 would have issued, K then V of each
      // (a tile past the workgroup's last gets a zero-length buffer)
#pragma unroll
      for (int i = 1; i < NST; ++i) {
        load_tile_rsrc<LPW>(k_tile(i < n_tiles ? S : 0, g_t0 + i), ring + kK0 + i * TB, gw,
                            k_off);
        load_tile_rsrc<LPW>(v_tile(i - 1 < n_tiles ? S : 0, g_t0 + i - 1),
                            ring + kV0 + (i - 1) * TB, gw, v_off);
      }
    }

    f32x16 s_a[RB][NKB], s_b[RB][NKB];
    float ce_a[RB], ce_b[RB];
    // Q and K of the first tile before its scores; the rest of the
    // prologue's loads are waited for at the top of the first step
    if constexpr (NST == 2) {
      if (n_tiles > 1)
        wait_vm_lgkm0<2 * LPW>();
      else
        wait_vm_lgkm0<LPW>();
    } else {
      wait_vm_lgkm0<2 * (NST - 1) * LPW>();
    }
    workgroup_barrier();
    if constexpr (QS) {
      // this wave's rows: rows 32 (gw % 2) .. + 31 of half gw / 2
      const uint32_t q_half_at = KG > 1 ? (uint32_t)((gw / 2) * SH::kRingBytes) + kV1
                                        : (gw / 2 == 0 ? kV1 : (uint32_t)SH::kRingBytes);
      const uint32_t q_base = q_half_at + k_lane + (uint32_t)((gw % 2) * 32 * CPR * 16);
#pragma unroll
      for (int s = 0; s < NDS; ++s) qf[0][s] = *(const u32x4*)(smem + (q_base ^ (uint32_t)(32 * s)));
    }
    FA2_TL(lin, 1, FA2_TL_NOW());
    if (n_act > 0) {
      // m starts at the row max of tile g_t0, which holds an unmasked key
      // for every row (key g_t0 B_c <= q0), so m is finite from here on
      tile_scores<D, DT, RB, NKB>(ring, kK0, k_lane, qf, s_a);
      tile_mask<RB, NKB, CAUSAL>(s_a, g_t0 * Bc, wave_row0, S, c, l32, hi, ce_a);
      tile_max<RB, NKB>(s_a, ce_a, m_run);
    }

    // One pipeline step for tile j with parity PAR = j % 2 and ring stage
    // SJ = j % NST (both known at compile time: the loop is unrolled by a
    // multiple of 2 and of NST); `cur` holds tile j's scores, `nxt` receives
    // tile j + 1's.
    auto step = [&](auto par, auto sj_c, int j, f32x16 (&cur)[RB][NKB], float (&ce_cur)[RB],
                    f32x16 (&nxt)[RB][NKB], float (&ce_nxt)[RB]) {
      constexpr int PAR = decltype(par)::value, SJ = decltype(sj_c)::value;
      uint32_t k_next, k_free, v_cur, v_free;  // K of tile j + 1, of tile j (done);
                                               // V of tile j, of tile j - 1 (done)
      if constexpr (NST == 2) {
        k_next = PAR ? kK0 : kK1;
        k_free = PAR ? kK1 : kK0;
        v_cur = PAR ? kV1 : kV0;
        v_free = PAR ? kV0 : kV1;
      } else {
        constexpr int sn = (SJ + 1) % NST, sp = (SJ + NST - 1) % NST;
        k_next = kK0 + (uint32_t)(sn * TB);
        k_free = kK0 + (uint32_t)(SJ * TB);
        v_cur = kV0 + (uint32_t)(SJ * TB);
        v_free = kV0 + (uint32_t)(sp * TB);
      }
      wait_vm_lgkm0<(NST - 2) * 2 * LPW>();
      workgroup_barrier();
      // K of tile j + NST and V of tile j + NST - 1; a tile past the
      // workgroup's last gets a zero-length buffer, so its loads only write
      // zeros to a free stage
      const StepLoads<LPW> ld{
          k_tile(j + NST < n_tiles ? S : 0, g_t0 + j + NST),
          v_tile(j + NST - 1 < n_tiles ? S : 0, g_t0 + j + NST - 1),
          ring + k_free, ring + v_free, k_off, v_off, gw};
      if (j < n_act) {
        // scores of tile j + 1 || probabilities of tile j, then P V of tile j
        // (past the wave's last tile the scores come from a stale stage and are
        // never used)
        pipeline_block<D, DT, RB, NKB, LPW, Tile<D, ALT>::kLoadEvery>(
            ld, ring, k_next, v_cur, k_lane, vt_x, qf, cur, ce_cur, m_run, l_run, l_rnd, nxt,
            acc_o);
        if (j + 1 < n_act) {
          if (tile_needs_mask<RB, NKB, CAUSAL>((g_t0 + j + 1) * Bc, wave_row0, S)) {
            tile_mask<RB, NKB, CAUSAL>(nxt, (g_t0 + j + 1) * Bc, wave_row0, S, c, l32, hi,
                                       ce_nxt);
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
    // unrolled by U steps, a multiple of 2 (score buffers) and of NST (stages)
    constexpr int U = NST % 2 == 0 ? NST : 2 * NST;
    auto step_u = [&](auto u, int j0) {
      constexpr int UU = decltype(u)::value;
      if constexpr (UU < U) {
        if (UU == 0 || j0 + UU < n_steps) {
          if constexpr (UU % 2 == 0)
            step(std::integral_constant<int, 0>{}, std::integral_constant<int, UU % NST>{}, j0 + UU,
                 s_a, ce_a, s_b, ce_b);
          else
            step(std::integral_constant<int, 1>{}, std::integral_constant<int, UU % NST>{}, j0 + UU,
                 s_b, ce_b, s_a, ce_a);
        }
      }
    };
    for (int j = 0; j < n_steps; j += U) {
      step_u(std::integral_constant<int, 0>{}, j);
      step_u(std::integral_constant<int, 1>{}, j);
      step_u(std::integral_constant<int, 2>{}, j);
      step_u(std::integral_constant<int, 3>{}, j);
      step_u(std::integral_constant<int, 4>{}, j);
      step_u(std::integral_constant<int, 5>{}, j);
    }
    static_assert(U <= 6, "unroll");
  }
  // the last steps' loads (zeros into free stages) must land before the
  // workgroup's LDS is released (or reused for the merge)
  wait_vm_lgkm0<0>();
  FA2_TL(lin, 2, FA2_TL_NOW());
  FA2_TL(lin, 5, (unsigned long long)(unsigned)qt | ((unsigned long long)(unsigned)bh << 16) |
                     ((unsigned long long)(unsigned)n_steps << 32));

  if constexpr (KG > 1) {
    // Merge the key groups' partial results for each row, as the pages'
    // split of a row's keys into parts merges them: both are rescaled to the
    // larger reference max, O~ and both sums added. Each group finishes half
    // of every row's columns, group 0 the first NDB / 2 column blocks and
    // group 1 the rest: it hands the other half of its O~, with its m, l and
    // l', to the other group through the LDS the rings leave free (lane l of
    // wave w of either group holds the same elements) and takes that group's
    // half in turn. Group 0 has no tiles (weight 0 for its unset state) when
    // h_split is 0. A key split never takes this tile: one chunk.
    constexpr int NH = NDB / 2, HF = SH::kMergeFloats;
    static_assert(NDB % 2 == 0 && HF == NH * 16 + 3 && 2 * GW * HF * 64 * 4 <= SH::kLdsBytes,
                  "merge area");
    workgroup_barrier();
    float* const give = (float*)smem + (size_t)(grp * GW + gw) * HF * 64 + lane;
    const float* const take = (const float*)smem + (size_t)((1 - grp) * GW + gw) * HF * 64 + lane;
    auto hand = [&](auto first) {
      constexpr int F = decltype(first)::value;
#pragma unroll
      for (int i = 0; i < NH; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) give[(i * 16 + r) * 64] = acc_o[0][F + i][r];
    };
    if (grp == 0)
      hand(std::integral_constant<int, NH>{});
    else
      hand(std::integral_constant<int, 0>{});
    give[(NH * 16) * 64] = m_run[0];
    give[(NH * 16 + 1) * 64] = l_run[0];
    give[(NH * 16 + 2) * 64] = l_rnd[0];
    // the barrier is plain s_barrier: this wave's LDS writes must have
    // completed before the other group reads them
    wait_vm_lgkm0<63>();
    workgroup_barrier();
    const float m_t = take[(NH * 16) * 64];
    const float l_t = take[(NH * 16 + 1) * 64], lr_t = take[(NH * 16 + 2) * 64];
    const bool g0 = grp == 0;
    const float m0 = g0 ? m_run[0] : m_t, m1 = g0 ? m_t : m_run[0];
    const float m_new = h_split > 0 ? fmaxf(m0, m1) : m1;
    const float a0 = h_split > 0 ? __builtin_amdgcn_exp2f(m0 - m_new) : 0.f;
    const float a1 = __builtin_amdgcn_exp2f(m1 - m_new);
    const float l_tot = xor32_sum(g0 ? l_run[0] * a0 + l_t * a1 : l_t * a0 + l_run[0] * a1);
    const float l_o = xor32_sum(g0 ? l_rnd[0] * a0 + lr_t * a1 : lr_t * a0 + l_rnd[0] * a1);
    const int row = wave_row0 + l32;
    if (row < S) {
      const float inv = 1.0f / l_o;
      // this group's half: blocks F .. F + NH - 1, the other group's
      // values from LDS; x0 * a0 + x1 * a1 with x0 group 0's value
      auto finish = [&](auto first) {
        constexpr int F = decltype(first)::value;
#pragma unroll
        for (int i = 0; i < NH; ++i) {
          float x[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float own = acc_o[0][F + i][r], other = take[(i * 16 + r) * 64];
            x[r] = F == 0 ? own * a0 + other * a1 : other * a0 + own * a1;
          }
          store_o_block<DT>(o + o_at + (size_t)row * o_rs + 32 * (F + i), x, inv, hi);
        }
      };
      if (g0)
        finish(std::integral_constant<int, 0>{});
      else
        finish(std::integral_constant<int, NH>{});
      if (g0 && hi == 0) lse[(size_t)bh * S + row] = (m_new + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    FA2_TL(lin, 3, FA2_TL_NOW());
    return;
  }

  // Epilogue: O = O~ / sum(rounded P), rounded once to the input dtype, and
  // lse = ln2 (m + log2 l) from the unrounded sum; or, for one chunk of a
  // split tile, the chunk's partial O~, m, l and l' for the merge.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wave_row0 + 32 * rb + l32;
    const float l_tot = xor32_sum(l_run[rb]);
    const float l_o = xor32_sum(l_rnd[rb]);
    if (row < S && n_chunks > 1) {
      const size_t prow =
          ((size_t)bh * ks.n_split + chunk) * (size_t)(S - ks.row0) + (size_t)(row - ks.row0);
      float* po = ks.part_o + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(float4*)(po + 32 * db + 8 * g + 4 * hi) =
              float4{acc_o[rb][db][4 * g], acc_o[rb][db][4 * g + 1], acc_o[rb][db][4 * g + 2],
                     acc_o[rb][db][4 * g + 3]};
      if (hi == 0) {
        ks.part_ml[prow * 3 + 0] = m_run[rb];
        ks.part_ml[prow * 3 + 1] = l_tot;
        ks.part_ml[prow * 3 + 2] = l_o;
      }
    } else if (row < S) {
      const float inv = 1.0f / l_o;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        store_o_block<DT>(o + o_at + (size_t)row * o_rs + 32 * db, acc_o[rb][db], inv, hi);
      if (hi == 0) lse[(size_t)bh * S + row] = (m_run[rb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
  FA2_TL(lin, 3, FA2_TL_NOW());
}

// Launch the kernel over (B, H, S); `st` gives the strides of a strided call
// (nullptr: contiguous tensors), `ks` a key split (ct = 0: none), whose
// merge follows on the same stream.
template <int D, int DT, bool CAUSAL, int ALT>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int S, float scale, const Strides* st, const KeySplit& ks, int n_cu,
                  unsigned int* tk, hipStream_t stream) {
  using SH = Shape<D, ALT>;
  constexpr bool ALT_KG = SH::kKeyGroups > 1;
  const int n_qt = (S + SH::kBr - 1) / SH::kBr;
  // work items per (b, h): query tiles, or their key chunks under a split
  const int n_x = (int)split_items_per_head(ks, n_qt, CAUSAL);
  const dim3 grid((unsigned)n_x, (unsigned)H, (unsigned)B);
  const dim3 block(SH::kThreads);
  // workgroups resident per compute unit: the register budget allows
  // kWavesPerSimd waves per SIMD, i.e. that many 4-wave workgroups
  const long long slots = (long long)n_cu * Tile<D, ALT>::kWavesPerSimd * 4 / SH::kWaves;
  const long long n_wg = (long long)n_qt * H * B;
  const int pair_split = (CAUSAL && ks.ct == 0 && n_qt > 1 && n_wg <= slots)
                             ? (int)(((n_qt + 1) / 2) * (long long)H * B)
                             : 0;
  // the last quarter of a multi-round grid takes tickets (none under a key
  // split, whose items are not in longest-first order, nor on the key-group
  // tile: one workgroup per unit exposes the ticket's latency, and the
  // in-order dispatch already gives each freed unit the longest tile left on
  // its XCD)
  const int tk_from =
      (tk && !ALT_KG && ks.ct == 0 && n_wg > slots) ? (int)(n_wg - n_wg / 4) : INT32_MAX;
  const Strides cs{(long long)H * S * D, (long long)S * D, D, (long long)H * S * D,
                   (long long)S * D,     D,                 (long long)H * S * D, (long long)S * D,
                   D,                    (long long)H * S * D, (long long)S * D, D};
  if (st)
    fa2_fwd_kernel<D, DT, CAUSAL, true, ALT><<<grid, block, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, S,
        scale * kLog2e, pair_split, *st, ks, tk_from, tk);
  else
    fa2_fwd_kernel<D, DT, CAUSAL, false, ALT><<<grid, block, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, S,
        scale * kLog2e, pair_split, cs, ks, tk_from, tk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || ks.ct == 0) return err;
  const Strides& os = st ? *st : cs;
  return launch_combine<D, DT>(ks.part_o, ks.part_ml, o, lse, B * H, H, S, ks.row0,
                               CAUSAL ? ks.row0 : 0, ks.n_split, os.ob, os.oh, os.os, stream);
}

template <int D, int ALT>
hipError_t launch_dtype(int dtype, int causal, const void* q, const void* k, const void* v,
                        void* o, float* lse, int B, int H, int S, float scale, const Strides* st,
                        const KeySplit& ks, int n_cu, unsigned int* tk, hipStream_t stream) {
  if (dtype == FA2_F16)
    return causal ? launch<D, FA2_F16, true, ALT>(q, k, v, o, lse, B, H, S, scale, st, ks, n_cu,
                                                   tk, stream)
                  : launch<D, FA2_F16, false, ALT>(q, k, v, o, lse, B, H, S, scale, st, ks, n_cu,
                                                    tk, stream);
  return causal ? launch<D, FA2_BF16, true, ALT>(q, k, v, o, lse, B, H, S, scale, st, ks, n_cu,
                                                  tk, stream)
                : launch<D, FA2_BF16, false, ALT>(q, k, v, o, lse, B, H, S, scale, st, ks, n_cu,
                                                   tk, stream);
}

hipError_t launch_any(int D, int dtype, int causal, const void* q, const void* k, const void* v,
                      void* o, float* lse, int B, int H, int S, float scale, const Strides* st,
                      const KeySplit& ks, int n_cu, unsigned int* tk, hipStream_t stream) {
  switch (D) {
    case 64:
      return S >= FA2_D64_LONG_S
                 ? launch_dtype<64, 1>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st, ks,
                                       n_cu, tk, stream)
             : d64_kg(B, H, S, causal != 0, ks.ct > 0, n_cu)
                 ? launch_dtype<64, 2>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st, ks,
                                       n_cu, tk, stream)
                 : launch_dtype<64, 0>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st, ks,
                                       n_cu, tk, stream);
    case 128:
      return d128_alt(B, H, S, causal != 0, ks.ct > 0, n_cu)
                 ? launch_dtype<128, 1>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st, ks,
                                           n_cu, tk, stream)
                 : launch_dtype<128, 0>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st,
                                            ks, n_cu, tk, stream);
    default:
      return launch_dtype<256, 0>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st, ks,
                                      n_cu, tk, stream);
  }
}

}  // namespace

static_assert(Shape<64, 1>::kBr == Shape<64>::kBr && Shape<64, 2>::kBr == Shape<64>::kBr &&
                  (FA2_D128_ALT == 0 || Shape<128, 1>::kBr == Shape<128>::kBr),
              "both tiles of a head dim (where both are used) take the query rows per "
              "workgroup fa2_rows_per_workgroup reports");

// Counters for the tickets of the prefill kernel's last workgroups: one per
// (device, stream) that has launched a multi-round grid, in this array (its
// copy on each GPU, zero when the library is loaded; every complete launch
// leaves its counter at zero). Calls on one stream run one after another and
// calls on two streams (hipStreamPerThread counts as one per host thread)
// never share a counter. A call being captured into a
// graph takes none (its launch keeps the fixed order): a graph may be
// replayed beside eager calls on another stream. In host code `tickets`
// names a host-side stand-in; ticket_counter() looks up each device's
// address once.
constexpr int kTicketSlots = 1024;
static __device__ __align__(256) unsigned int tickets[kTicketSlots];

namespace {

constexpr int kMaxTicketDevices = 64;
std::mutex g_ticket_mu;
unsigned int* g_ticket_base[kMaxTicketDevices] = {};
int g_ticket_used[kMaxTicketDevices] = {};
std::map<std::pair<int, uintptr_t>, int> g_ticket_slot;

// The counter for `stream` on the current device, or nullptr (no tickets:
// the stream is capturing, its state cannot be read, or every slot is taken).
unsigned int* ticket_counter(hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (cap != hipStreamCaptureStatusNone) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxTicketDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_ticket_mu);
  if (!g_ticket_base[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(tickets)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ticket_base[dev] = (unsigned int*)p;
  }
  // hipStreamPerThread names a different stream in each host thread: key it
  // by a number each thread draws once (never reused, unlike a thread's id)
  static std::atomic<uintptr_t> next_thread{1};
  static thread_local const uintptr_t this_thread = next_thread.fetch_add(1);
  const uintptr_t id = stream == hipStreamPerThread ? ~this_thread : (uintptr_t)stream;
  const auto key = std::make_pair(dev, id);
  auto it = g_ticket_slot.find(key);
  if (it == g_ticket_slot.end()) {
    if (g_ticket_used[dev] >= kTicketSlots) return nullptr;
    it = g_ticket_slot.emplace(key, g_ticket_used[dev]++).first;
  }
  return g_ticket_base[dev] + it->second;
}

}  // namespace

extern "C" int fa2_rows_per_workgroup(int D) {
  switch (D) {
    case 64: return Shape<64>::kBr;
    case 128: return Shape<128>::kBr;
    case 256: return Shape<256>::kBr;
    default: return 0;
  }
}

namespace {

// Checks shared by the prefill entry points, in their documented order,
// then the launch. strides: nullptr for contiguous tensors, else 12 element
// strides. balanced: split the keys of long query tiles when the grid is
// small (fa2_fwd_balanced), with `workspace` for the partials.
int prefill_call(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int S, int D, const long long* strides, int causal, float scale, int dtype,
                 bool balanced, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  // S leaves room for the tile indices past its end in 32-bit key counts
  if (B < 1 || H < 1 || S < 1 || B > 65535 || H > 65535 || S > INT32_MAX - 1024)
    return FA2_ERR_SHAPE;
  if (dtype != FA2_F16 && dtype != FA2_BF16) return FA2_ERR_DTYPE;
  if (!(D == 64 || D == 128 || D == 256)) return FA2_ERR_HEADDIM;
  // every stride in [0, 2^40], a multiple of 8 elements (16-byte rows), and
  // each sequence stride at least D
  Strides st{(long long)H * S * D, (long long)S * D, D, (long long)H * S * D,
             (long long)S * D,     D,                 (long long)H * S * D, (long long)S * D,
             D,                    (long long)H * S * D, (long long)S * D, D};
  if (strides) {
    for (int i = 0; i < 12; ++i) {
      const long long x = strides[i];
      if (x < 0 || x > (1LL << 40) || (x & 7)) return FA2_ERR_STRIDE;
      if (i % 3 == 2 && x < D) return FA2_ERR_STRIDE;
    }
    st = Strides{strides[0], strides[1], strides[2],  strides[3], strides[4],  strides[5],
                 strides[6], strides[7], strides[8],  strides[9], strides[10], strides[11]};
  }
  // the elements of every tensor within int64, and the 256 rows of Q, K or
  // V one tile load spans within 31-bit offsets from the tile's start
  // (buffer loads; a head itself may span any size)
  if (!elements_fit_int64(B, H, S, D) || 256LL * st.qs * 2 > (long long)INT32_MAX ||
      256LL * st.ks * 2 > (long long)INT32_MAX || 256LL * st.vs * 2 > (long long)INT32_MAX)
    return FA2_ERR_SHAPE;
  // the kernel linearises its block index in a 32-bit int (a key split
  // only runs on grids of a few thousand workgroups)
  const int rows = fa2_rows_per_workgroup(D);
  const unsigned long long blocks = (((unsigned long long)S + rows - 1) / rows) *
                                    (unsigned long long)H * (unsigned long long)B;
  if (blocks > (unsigned long long)INT32_MAX) return FA2_ERR_SHAPE;
  // the output's rows must not share memory
  if (strides && !rows_disjoint(B, H, S, D, st.ob, st.oh, st.os)) return FA2_ERR_STRIDE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA2_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA2_ERR_ALIGN;
  if (!std::isfinite(scale)) return FA2_ERR_SCALE;
  // overlap of the outputs with anything, by the byte ranges the tensors span
  const size_t qe = extent_bytes(B, H, S, D, st.qb, st.qh, st.qs, 2);
  const size_t ke = extent_bytes(B, H, S, D, st.kb, st.kh, st.ks, 2);
  const size_t ve = extent_bytes(B, H, S, D, st.vb, st.vh, st.vs, 2);
  const size_t oe = extent_bytes(B, H, S, D, st.ob, st.oh, st.os, 2);
  const size_t lse_bytes = (size_t)B * H * S * sizeof(float);
  if (overlaps(o, oe, q, qe) || overlaps(o, oe, k, ke) || overlaps(o, oe, v, ve) ||
      overlaps(lse, lse_bytes, q, qe) || overlaps(lse, lse_bytes, k, ke) ||
      overlaps(lse, lse_bytes, v, ve) || overlaps(lse, lse_bytes, o, oe))
    return FA2_ERR_ALIAS;
  int n_cu = 0;
  const int dev = check_device(&n_cu);
  if (dev != FA2_OK) return dev;

  KeySplit ks{};
  if (balanced) {
    ks = plan_split(D, B, H, S, causal != 0, n_cu);
    const size_t need = split_workspace_bytes(ks, B, H, S, D);
    if (need > 0) {
      if (!workspace || ((uintptr_t)workspace & 15u) || workspace_bytes < need)
        return FA2_ERR_WORKSPACE;
      if (overlaps(workspace, need, q, qe) || overlaps(workspace, need, k, ke) ||
          overlaps(workspace, need, v, ve) || overlaps(workspace, need, o, oe) ||
          overlaps(workspace, need, lse, lse_bytes))
        return FA2_ERR_ALIAS;
      ks.part_o = (float*)workspace;
      ks.part_ml =
          (float*)((char*)workspace + chunk_part_o_bytes(B, H, S - ks.row0, D, ks.n_split));
    }
  }

  (void)hipGetLastError();  // start from a clean error state
  const hipError_t err =
      launch_any(D, dtype, causal, q, k, v, o, lse, B, H, S, scale, strides ? &st : nullptr, ks,
                 n_cu, ticket_counter((hipStream_t)stream), (hipStream_t)stream);
  return err == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

}  // namespace

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int S, int D, int causal, float scale, int dtype, void* stream) {
  return prefill_call(q, k, v, o, lse, B, H, S, D, nullptr, causal, scale, dtype, false, nullptr,
                      0, stream);
}

extern "C" int fa2_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int S, int D, const long long* strides, int causal,
                               float scale, int dtype, void* stream) {
  if (!strides) return FA2_ERR_NULL;
  return prefill_call(q, k, v, o, lse, B, H, S, D, strides, causal, scale, dtype, false, nullptr,
                      0, stream);
}

extern "C" size_t fa2_fwd_balanced_workspace_bytes(int B, int H, int S, int D, int causal) {
  if (B < 1 || H < 1 || S < 1 || !(D == 64 || D == 128 || D == 256)) return 0;
  int n_cu = 0;
  if (check_device(&n_cu) != FA2_OK) return 0;
  return split_workspace_bytes(plan_split(D, B, H, S, causal != 0, n_cu), B, H, S, D);
}

extern "C" int fa2_fwd_balanced(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int S, int D, const long long* strides, int causal,
                                float scale, int dtype, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return prefill_call(q, k, v, o, lse, B, H, S, D, strides, causal, scale, dtype, true, workspace,
                      workspace_bytes, stream);
}

#ifdef FA2_TIMELINE
// The timeline build's own entry points (include/fa2_timeline.h).
namespace {
__global__ void fa2_timeline_clear_kernel() {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (size_t)kTimelineWgs * kTimelineSlots) fa2_tl[i] = 0ull;
}
}  // namespace

extern "C" int fa2_timeline_capacity(void) { return kTimelineWgs; }

extern "C" int fa2_timeline_clear(void* stream) {
  fa2_timeline_clear_kernel<<<kTimelineWgs * kTimelineSlots / 256, 256, 0, (hipStream_t)stream>>>();
  return hipGetLastError() == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

extern "C" int fa2_timeline_read(unsigned long long* host, int n_wg) {
  if (!host || n_wg < 0 || n_wg > kTimelineWgs) return FA2_ERR_SHAPE;
  if (hipDeviceSynchronize() != hipSuccess) return FA2_ERR_LAUNCH;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(fa2_tl),
                             (size_t)n_wg * kTimelineSlots * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess
             ? FA2_OK
             : FA2_ERR_LAUNCH;
}
#endif
