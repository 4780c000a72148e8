// FlashAttention-2 split-KV decoding for MI355X (gfx950 / CDNA4).
//
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
// workgroups; fa2_combine.h holds the merge.
//
// The partial kernel runs one wave per workgroup: a 32-row query block (rows
// past Sq are zero and never stored) against one key chunk, streamed through
// a two-stage LDS ring of 32-key tiles by the wave's own LDS-direct loads.
// Decoding reads every K/V byte once per 32 queries, so it is bound by
// memory bandwidth, not by the matrix cores; the kernel keeps the exact
// running row max per tile (no lazy reference point), which also covers rows
// that have no key in a chunk (their partial is m = -inf, l = 0).
//
// Workspace (caller-owned device memory, fp32): the chunk partials of
// fa2_combine.h for all Sq rows (row0 = 0); part_ml starts at the part_o
// size rounded up to 256 bytes.

#include <mutex>

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

// ---- FP8 (e4m3) K and V ------------------------------------------------
// Codes (OCP FP8 e4m3: sign, 4 exponent bits of bias 7, 3 mantissa bits)
// become matrix-core operands through gfx950's packed conversion, two codes
// (bytes 0-1, or 2-3, of a word) per instruction, exactly: every e4m3 value
// is representable in fp16 and in bf16.
template <int DT>
__device__ __forceinline__ u32x2 e4m3x4_op(uint32_t x) {
  if constexpr (DT == FA2_F16) {
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  } else {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  }
}
// Eight codes (two words, in byte order) as one operand of element type DT.
template <int DT>
__device__ __forceinline__ u32x4 e4m3x8_op(uint32_t x0, uint32_t x1) {
  const u32x2 a = e4m3x4_op<DT>(x0), b = e4m3x4_op<DT>(x1);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// S^T = K_t Q^T for an FP8 K tile at byte k_stage: each 16-byte read of row
// 32 kb + l32 (chunk 2 u + hi) gives the K operands of k-steps 2 u and
// 2 u + 1, so k-step 2 u + v covers dims 32 u + 16 hi + 8 v .. + 7, the
// order in which Q^T was loaded.
template <int D, int DT, int NKB>
__device__ __forceinline__ void tile_scores_kv8(const unsigned char* smem, uint32_t k_stage,
                                                int l32, int hi, const u32x4 (&qf)[1][D / 16],
                                                f32x16 (&acc)[1][NKB]) {
  using E = Elem<DT>;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) acc[0][kb] = f32x16{};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int row = 32 * kb + l32;
    const unsigned char* rp = smem + k_stage + row * D;
    const int sw = swz_k8<D>(row);
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const u32x4 raw = *(const u32x4*)(rp + (((2 * u + hi) ^ sw) * 16));
      acc[0][kb] = E::mfma(e4m3x8_op<DT>(raw[0], raw[1]), qf[0][2 * u], acc[0][kb]);
      acc[0][kb] = E::mfma(e4m3x8_op<DT>(raw[2], raw[3]), qf[0][2 * u + 1], acc[0][kb]);
    }
  }
}

// O~ += P V for an FP8 V tile at byte v_stage. One ds_read_b64_tr_b8 per
// (key block, half, head-dim block): in each 16-lane group, output lane i
// byte e comes from source lane 2 e + i / 8, byte i % 8, so source lane s
// points at key row R(s / 2) and dims 8 (s % 2) .. + 7 of the group's 16;
// output lane i then holds dim 16 grp + i for the 8 keys R(0..7). R(e) is
// the key of P^T element e in this lane half (32 kb + 16 h + 8 (e / 4) +
// 4 hi + e % 4), so the operands pair up without any exchange.
template <int D, int DT, int NKB>
__device__ __forceinline__ void tile_pv_kv8(const unsigned char* smem, uint32_t v_stage,
                                            uint32_t v8_base, uint32_t v8_x,
                                            const u32x4 (&pb)[1][NKB][2],
                                            f32x16 (&acc_o)[1][D / 32]) {
  using E = Elem<DT>;
  constexpr int NDB = D / 32;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint32_t a = v_stage + (uint32_t)((32 * kb + 16 * h) * D) + v8_base +
                           ((uint32_t)(32 * db) ^ v8_x);
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(smem + a));
        acc_o[0][db] = E::mfma(e4m3x8_op<DT>((uint32_t)raw[0], (uint32_t)raw[1]), pb[0][kb][h],
                               acc_o[0][db]);
      }
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

// Element strides of the batch, head and sequence dims of Q, K, V and O
// (the head dim is contiguous; FP8 K and V count bytes).
struct SkvStrides {
  long long qb, qh, qs, kb, kh, ks, vb, vh, vs, ob, oh, os;
};

SkvStrides contiguous_strides(int H, int Sq, int Sk, int D) {
  const long long q_h = (long long)Sq * D, k_h = (long long)Sk * D;
  return SkvStrides{H * q_h, q_h, D, H * k_h, k_h, D, H * k_h, k_h, D, H * q_h, q_h, D};
}

// c multiplies q . k into base-2 logits; v_mult multiplies O~ before it is
// stored (1 for 16-bit K and V; for FP8, c carries K's descale and v_mult
// is V's).
template <int D, int DT, bool CAUSAL, bool KV8>
__global__ __launch_bounds__(64) void fa2_splitkv_partial_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    float* __restrict__ part_o, float* __restrict__ part_ml, int Sq, int Sk, int n_split,
    int chunk_keys, float c, float v_mult, SkvStrides st) {
  using ST = SplitTile<D, KV8>;
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
  const int b = blockIdx.z, h = blockIdx.y;
  const int q0 = qblk * 32;
  const int row = q0 + l32;
  const int off = Sk - Sq;  // position of query 0 in the sequence

  // this chunk's keys, cut short where no row of the block can see them
  const int k_begin = split * chunk_keys;
  int k_end = min(k_begin + chunk_keys, Sk);
  if (CAUSAL) k_end = min(k_end, min(q0 + 31, Sq - 1) + off + 1);
  // keys this lane's row keeps, within the chunk
  const int row_lim = CAUSAL ? min(k_end, row + off + 1) : k_end;

  // Q^T operands: k-step s covers dims 16 s + 8 hi .. + 7, or, with FP8 K,
  // dims 32 (s / 2) + 16 hi + 8 (s % 2) .. + 7 (the order its reads give)
  u32x4 qf[RB][NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    const int d0 = KV8 ? 32 * (s / 2) + 16 * hi + 8 * (s % 2) : 16 * s + 8 * hi;
    qf[0][s] = u32x4{0, 0, 0, 0};
    if (row < Sq)
      qf[0][s] = *(const u32x4*)(q + (size_t)(b * st.qb + h * st.qh) + (size_t)row * st.qs + d0);
  }

  constexpr int EB = KV8 ? 1 : 2;  // bytes per K or V element
  // K and V rows of this head, `k_rb` / `v_rb` bytes apart; buffers end
  // with key Sk - 1, so loads of keys >= Sk return zero
  const uint32_t k_rb = (uint32_t)st.ks * EB, v_rb = (uint32_t)st.vs * EB;
  const int k_cap = rows_within_2g(k_rb), v_cap = rows_within_2g(v_rb);
  const unsigned char* k_head = (const unsigned char*)k + (size_t)(b * st.kb + h * st.kh) * EB;
  const unsigned char* v_head = (const unsigned char*)v + (size_t)(b * st.vb + h * st.vh) * EB;
  uint32_t k_off[LPW], v_off[LPW];
  if constexpr (KV8) {
    tile_load_offsets8<D, LPW, false>(0, lane, k_rb, k_off);
    tile_load_offsets8<D, LPW, true>(0, lane, v_rb, v_off);
  } else {
    tile_load_offsets_strided<D, LPW, false>(0, lane, k_rb, k_off);
    tile_load_offsets_strided<D, LPW, true>(0, lane, v_rb, v_off);
  }
  auto load_k = [&](int t, uint32_t stage) {
    load_tile_rsrc<LPW>(tile_rsrc_rows(k_head, Sk, t * Bc, k_rb, k_cap),
                        smem + stage, 0, k_off);
  };
  auto load_v = [&](int t, uint32_t stage) {
    load_tile_rsrc<LPW>(tile_rsrc_rows(v_head, Sk, t * Bc, v_rb, v_cap),
                        smem + stage, 0, v_off);
  };
  const uint32_t k_lane = (uint32_t)(l32 * CPR * 16 + 16 * (hi ^ swz_k<D>(l32)));
  const int vt_row = 4 * hi + (lane & 15) / 4;
  const int vt_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const uint32_t vt_x = (uint32_t)((vt_row * CPR + vt_chunk) * 16 + 8 * (lane & 1) +
                                   64 * (swz_v<D>(vt_row) >> 2));
  // FP8 V^T source address of this lane: key row R(e), e = (lane % 16) / 2,
  // dims 16 grp + 8 (lane % 2) of the 32-dim block, grp = (lane / 16) % 2;
  // the head-dim block's chunk pair is XORed with the row's swizzle
  const int e8 = (lane & 15) >> 1, grp8 = (lane >> 4) & 1;
  const int r8 = 8 * (e8 >> 2) + 4 * hi + (e8 & 3);
  const uint32_t v8_base = (uint32_t)(r8 * D + 16 * grp8 + 8 * (lane & 1));
  const uint32_t v8_x = (uint32_t)(16 * swz_v8<D>(r8));

  f32x16 acc_o[RB][NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[0][db] = f32x16{};
  float m_run[RB] = {-INFINITY}, l_run[RB] = {0.f}, l_rnd[RB] = {0.f};
  const float one[RB] = {1.f};

  const int t_first = k_begin / Bc;
  const int n_t = k_end > k_begin ? (k_end - k_begin + Bc - 1) / Bc : 0;
  if (n_t > 0) {
    load_k(t_first, kK0);
    load_v(t_first, kV0);
  }
  for (int t = 0; t < n_t; ++t) {
    const uint32_t ks = (t & 1) ? kK1 : kK0, vs = (t & 1) ? kV1 : kV0;
    // tile t has landed, and every LDS read of tile t - 1 is done, so its
    // stages can take tile t + 1
    wait_vm_lgkm0<0>();
    if (t + 1 < n_t) {
      load_k(t_first + t + 1, ks ^ TB);
      load_v(t_first + t + 1, vs ^ TB);
    }
    f32x16 sc[RB][NKB];
    if constexpr (KV8)
      tile_scores_kv8<D, DT, NKB>(smem, ks, l32, hi, qf, sc);
    else
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
    if constexpr (KV8)
      tile_pv_kv8<D, DT, NKB>(smem, vs, v8_base, v8_x, pb, acc_o);
    else
      tile_pv<D, DT, RB, NKB>(smem, vs, vt_x, pb, acc_o);
  }
  if constexpr (KV8) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[0][db] *= v_mult;
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

// Launch the partial and combine kernels. kv8: K and V are FP8 codes with
// these descales (k_mult, v_mult), else 16-bit values (both 1).
template <int D, int DT, bool CAUSAL, bool KV8>
hipError_t launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int H, int Sq, int Sk, float scale, float k_mult, float v_mult,
                          const SkvStrides& st, int n_split, void* ws, hipStream_t stream) {
  using ST = SplitTile<D, KV8>;
  // chunks of whole tiles; trailing splits that would be empty are dropped
  int chunk_tiles = 0, n_eff = 0;
  splitkv_chunking(Sk, ST::kBc, n_split, chunk_tiles, n_eff);
  const int n_qblk = (Sq + 31) / 32;
  float* part_o = (float*)ws;
  float* part_ml = (float*)((char*)ws + chunk_part_o_bytes(B, H, Sq, D, n_eff));
  const dim3 grid((unsigned)(n_eff * n_qblk), (unsigned)H, (unsigned)B);
  fa2_splitkv_partial_kernel<D, DT, CAUSAL, KV8><<<grid, dim3(64), 0, stream>>>(
      (const uint16_t*)q, k, v, part_o, part_ml, Sq, Sk, n_eff, chunk_tiles * ST::kBc,
      scale * kLog2e * k_mult, v_mult, st);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine<D, DT>(part_o, part_ml, o, lse, B * H, H, Sq, 0, 0, n_eff, st.ob, st.oh,
                               st.os, stream);
}

template <int D, int DT, bool KV8>
hipError_t launch_splitkv_causal(int causal, const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int H, int Sq, int Sk, float scale,
                                 float k_mult, float v_mult, const SkvStrides& st, int n_split,
                                 void* ws, hipStream_t stream) {
  return causal ? launch_splitkv<D, DT, true, KV8>(q, k, v, o, lse, B, H, Sq, Sk, scale, k_mult,
                                                   v_mult, st, n_split, ws, stream)
                : launch_splitkv<D, DT, false, KV8>(q, k, v, o, lse, B, H, Sq, Sk, scale, k_mult,
                                                    v_mult, st, n_split, ws, stream);
}

template <int D, bool KV8>
hipError_t launch_splitkv_dtype(int dtype, int causal, const void* q, const void* k, const void* v,
                                void* o, float* lse, int B, int H, int Sq, int Sk, float scale,
                                float k_mult, float v_mult, const SkvStrides& st, int n_split,
                                void* ws, hipStream_t stream) {
  return dtype == FA2_F16
             ? launch_splitkv_causal<D, FA2_F16, KV8>(causal, q, k, v, o, lse, B, H, Sq, Sk, scale,
                                                      k_mult, v_mult, st, n_split, ws, stream)
             : launch_splitkv_causal<D, FA2_BF16, KV8>(causal, q, k, v, o, lse, B, H, Sq, Sk, scale,
                                                       k_mult, v_mult, st, n_split, ws, stream);
}

template <bool KV8>
hipError_t launch_splitkv_any(int D, int dtype, int causal, const void* q, const void* k,
                              const void* v, void* o, float* lse, int B, int H, int Sq, int Sk,
                              float scale, float k_mult, float v_mult, const SkvStrides& st,
                              int n_split, void* ws, hipStream_t stream) {
  switch (D) {
    case 64:
      return launch_splitkv_dtype<64, KV8>(dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale,
                                           k_mult, v_mult, st, n_split, ws, stream);
    case 128:
      return launch_splitkv_dtype<128, KV8>(dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale,
                                            k_mult, v_mult, st, n_split, ws, stream);
    default:
      return launch_splitkv_dtype<256, KV8>(dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale,
                                            k_mult, v_mult, st, n_split, ws, stream);
  }
}

}  // namespace

// Scratch of fa2_fwd_splitkv_noalloc: the chunk partials of calls that
// bring no workspace. The library's code object holds one copy per GPU it
// is loaded on, for the life of the process. In host code `scratch` names a
// host-side stand-in, never the device memory: scratch_here() looks up the
// current device's address once and every launch takes that pointer.
static __device__ __align__(256) unsigned char scratch[FA2_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices] = {};

// The current device's copy of `scratch` (FA2_OK), found by
// hipGetSymbolAddress on the first call on that device.
int scratch_here(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return FA2_ERR_NO_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return FA2_ERR_LAUNCH;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA2_OK;
}

// Checks shared by the split-KV entry points, in the documented order, and
// the launch. kv_elem_bytes: 2 for 16-bit K and V, 1 for FP8. strides:
// nullptr for contiguous tensors, else 12 element strides. use_scratch: the
// partials go to the library's scratch (no workspace is passed; a call
// that needs more than FA2_SCRATCH_BYTES is refused).
int splitkv_call(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Sq, int Sk, int D, const long long* strides, int causal, float scale,
                 int dtype, float k_descale, float v_descale, int kv_elem_bytes, int n_split,
                 void* workspace, size_t workspace_bytes, void* stream,
                 bool use_scratch = false) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || B > 65535 || H > 65535 || n_split < 0 ||
      Sk > INT32_MAX - 1024)
    return FA2_ERR_SHAPE;
  if (causal && Sq > Sk) return FA2_ERR_SHAPE;  // the first queries would have no key
  if (dtype != FA2_F16 && dtype != FA2_BF16) return FA2_ERR_DTYPE;
  if (!(D == 64 || D == 128 || D == 256)) return FA2_ERR_HEADDIM;
  const SkvStrides st =
      strides ? SkvStrides{strides[0], strides[1], strides[2], strides[3], strides[4],
                           strides[5], strides[6], strides[7], strides[8], strides[9],
                           strides[10], strides[11]}
              : contiguous_strides(H, Sq, Sk, D);
  if (strides) {
    // strides in [0, 2^40]; rows 16-byte aligned (8 elements of q and o, and
    // of 16-bit K and V; 16 FP8 codes); sequence strides at least D
    for (int i = 0; i < 12; ++i) {
      const long long x = strides[i];
      const bool kv = i >= 3 && i < 9;
      const long long align = kv && kv_elem_bytes == 1 ? 16 : 8;
      if (x < 0 || x > (1LL << 40) || x % align) return FA2_ERR_STRIDE;
      if (i % 3 == 2 && x < D) return FA2_ERR_STRIDE;
    }
  }
  // the elements of every tensor within int64, the 256 rows of K or V one
  // tile load spans within 31-bit offsets from the tile's start (a head
  // itself may span any size), query rows of the whole call indexed in 32
  // bits
  if (!elements_fit_int64(B, H, Sk, D) || 256LL * st.ks * kv_elem_bytes > (long long)INT32_MAX ||
      256LL * st.vs * kv_elem_bytes > (long long)INT32_MAX)
    return FA2_ERR_SHAPE;
  if ((long long)B * H * Sq > (long long)INT32_MAX / 4) return FA2_ERR_SHAPE;
  if (strides && !rows_disjoint(B, H, Sq, D, st.ob, st.oh, st.os)) return FA2_ERR_STRIDE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA2_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA2_ERR_ALIGN;
  if (!std::isfinite(scale)) return FA2_ERR_SCALE;
  if (!std::isfinite(k_descale) || !(k_descale > 0.f) || !std::isfinite(v_descale) ||
      !(v_descale > 0.f))
    return FA2_ERR_SCALE;
  // the default split count needs the device's size; an explicit one lets
  // every argument be checked before the device is looked up
  int n_cu = 0;
  bool device_checked = false;
  if (n_split == 0) {
    const int dev = check_device(&n_cu);
    if (dev != FA2_OK) return dev;
    device_checked = true;
    n_split = splitkv_default_splits(B, H, Sq, Sk, n_cu, kv_elem_bytes == 1);
  }
  if (n_split > 65536) return FA2_ERR_SHAPE;
  const size_t need = chunk_workspace_bytes(B, H, Sq, D, n_split);
  if (use_scratch) {
    if (need > (size_t)FA2_SCRATCH_BYTES) return FA2_ERR_SCRATCH;
    if (!device_checked) {
      const int dev = check_device(&n_cu);
      if (dev != FA2_OK) return dev;
      device_checked = true;
    }
    const int got = scratch_here(&workspace);
    if (got != FA2_OK) return got;
    workspace_bytes = FA2_SCRATCH_BYTES;
  }
  if (!workspace || ((uintptr_t)workspace & 15u) || workspace_bytes < need) return FA2_ERR_WORKSPACE;
  // overlap, by the byte range each tensor spans
  const size_t q_bytes = extent_bytes(B, H, Sq, D, st.qb, st.qh, st.qs, 2);
  const size_t k_bytes = extent_bytes(B, H, Sk, D, st.kb, st.kh, st.ks, kv_elem_bytes);
  const size_t v_bytes = extent_bytes(B, H, Sk, D, st.vb, st.vh, st.vs, kv_elem_bytes);
  const size_t o_bytes = extent_bytes(B, H, Sq, D, st.ob, st.oh, st.os, 2);
  const size_t lse_bytes = (size_t)B * H * Sq * sizeof(float);
  if (overlaps(o, o_bytes, q, q_bytes) || overlaps(o, o_bytes, k, k_bytes) ||
      overlaps(o, o_bytes, v, v_bytes) || overlaps(lse, lse_bytes, q, q_bytes) ||
      overlaps(lse, lse_bytes, k, k_bytes) || overlaps(lse, lse_bytes, v, v_bytes) ||
      overlaps(lse, lse_bytes, o, o_bytes) || overlaps(workspace, need, q, q_bytes) ||
      overlaps(workspace, need, k, k_bytes) || overlaps(workspace, need, v, v_bytes) ||
      overlaps(workspace, need, o, o_bytes) || overlaps(workspace, need, lse, lse_bytes))
    return FA2_ERR_ALIAS;
  if (!device_checked) {
    const int dev = check_device(&n_cu);
    if (dev != FA2_OK) return dev;
  }

  (void)hipGetLastError();
  const hipStream_t hs = (hipStream_t)stream;
  const hipError_t err =
      kv_elem_bytes == 1
          ? launch_splitkv_any<true>(D, dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale,
                                     k_descale, v_descale, st, n_split, workspace, hs)
          : launch_splitkv_any<false>(D, dtype, causal, q, k, v, o, lse, B, H, Sq, Sk, scale, 1.f,
                                      1.f, st, n_split, workspace, hs);
  return err == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

}  // namespace

namespace {
int default_splits_here(int B, int H, int Sq, int Sk, bool kv8) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return 1;
  int n_cu = 0;
  if (check_device(&n_cu) != FA2_OK) n_cu = 256;
  return splitkv_default_splits(B, H, Sq, Sk, n_cu, kv8);
}
}  // namespace

extern "C" int fa2_splitkv_splits(int B, int H, int Sq, int Sk) {
  return default_splits_here(B, H, Sq, Sk, false);
}

extern "C" int fa2_splitkv_splits_fp8(int B, int H, int Sq, int Sk) {
  return default_splits_here(B, H, Sq, Sk, true);
}

extern "C" size_t fa2_splitkv_workspace_bytes(int B, int H, int Sq, int Sk, int D, int n_split) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || n_split < 0) return 0;
  if (!(D == 64 || D == 128 || D == 256)) return 0;
  // n_split = 0: enough for the default of either entry point (the FP8
  // default is never below the 16-bit one)
  if (n_split == 0) n_split = default_splits_here(B, H, Sq, Sk, true);
  return chunk_workspace_bytes(B, H, Sq, D, n_split);
}

extern "C" int fa2_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Sq, int Sk, int D, int causal, float scale,
                               int dtype, int n_split, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return splitkv_call(q, k, v, o, lse, B, H, Sq, Sk, D, nullptr, causal, scale, dtype, 1.f, 1.f, 2,
                      n_split, workspace, workspace_bytes, stream);
}

extern "C" int fa2_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int H, int Sq, int Sk, int D, int causal,
                                       float scale, int dtype, int n_split, void* stream) {
  return splitkv_call(q, k, v, o, lse, B, H, Sq, Sk, D, nullptr, causal, scale, dtype, 1.f, 1.f, 2,
                      n_split, nullptr, 0, stream, true);
}

extern "C" int fa2_fwd_splitkv_fp8(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int H, int Sq, int Sk, int D, int causal,
                                   float scale, float k_descale, float v_descale, int dtype,
                                   int n_split, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return splitkv_call(q, k, v, o, lse, B, H, Sq, Sk, D, nullptr, causal, scale, dtype, k_descale,
                      v_descale, 1, n_split, workspace, workspace_bytes, stream);
}

extern "C" int fa2_fwd_splitkv_strided(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int H, int Sq, int Sk, int D,
                                       const long long* strides, int causal, float scale,
                                       int dtype, int kv_fp8, float k_descale, float v_descale,
                                       int n_split, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!q || !k || !v || !o || !lse || !strides) return FA2_ERR_NULL;
  if (kv_fp8 != 0 && kv_fp8 != 1) return FA2_ERR_DTYPE;
  return splitkv_call(q, k, v, o, lse, B, H, Sq, Sk, D, strides, causal, scale, dtype,
                      kv_fp8 ? k_descale : 1.f, kv_fp8 ? v_descale : 1.f, kv_fp8 ? 1 : 2, n_split,
                      workspace, workspace_bytes, stream);
}
