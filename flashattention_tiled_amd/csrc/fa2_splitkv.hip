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
// workgroups. The merge is the guide's rescaling algebra applied across
// chunks: with M = max_g m_g and w_g = 2^(m_g - M),
//   O = sum_g w_g O~_g / sum_g w_g l'_g,   lse = ln2 (M + log2 sum_g w_g l_g),
// l_g summing P as computed and l'_g summing P as rounded for the P V
// product (the two sums of the prefill kernel).
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

#include "fa2_tile.h"
#include "fa2_host.h"

using fa2_host::check_device;
using fa2_host::overlaps;

namespace {

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

}  // namespace

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
