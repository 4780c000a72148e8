// Merge of key-chunk partials into O and lse, shared by the split-KV
// decoding path and the key-split prefill.
//
// When the keys of a query row are cut into chunks that run in different
// workgroups, each chunk g leaves its unnormalised O~_g, the base-2
// reference max m_g its P was taken against, l_g (the sum of P as computed)
// and l'_g (the sum of P as rounded for the P V product). The rescaling
// algebra of the infra.bea.ai FlashAttention V2 guide ("Optimization 2:
// Delay Rescaling"), applied across chunks instead of across tiles, merges
// them: with M = max_g m_g and w_g = 2^(m_g - M),
//   O = sum_g w_g O~_g / sum_g w_g l'_g,   lse = ln2 (M + log2 sum_g w_g l_g).
// That is the split-then-combine of jared-hpc Lecture 6 ("FA2 change 2")
// moved from warps to workgroups.
//
// Workspace layout (fp32), for rows row0 .. Sq - 1 of every (b, h), with
// Sr = Sq - row0:
//   part_o  [B*H][n_split][Sr][D]   O~ of each chunk
//   part_ml [B*H][n_split][Sr][3]   m (base 2), l, l'
// Row i has n_split chunks (kc = 0), or min(n_split, i / kc + 1) (kc > 0:
// the causal key split of the prefill, whose chunks are kc keys long and
// start at or before the first row of the row's query tile).
#pragma once

#include "fa2_plan.h"
#include "fa2_tile.h"

namespace {

// One wave per row, D / 64 columns per lane. The chunks' (m, l, l') are
// read 64 at a time, one chunk per lane, and reduced across the wave; the
// weighted O~ rows are then summed four chunks at a time, so that their
// loads overlap. A chunk with l' = 0 saw no key and has no weight. O is
// written through element strides (ob, oh, os); lse is (B, H, Sq).
template <int D, int DT>
__global__ __launch_bounds__(256) void fa2_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, uint16_t* __restrict__ o,
    float* __restrict__ lse, int n_rows, int H, int Sq, int row0, int kc, int n_split,
    long long ob, long long oh, long long os) {
  using E = Elem<DT>;
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;  // whole waves leave together
  const int Sr = Sq - row0;
  const int bh = r / Sr, i = row0 + r % Sr;
  const int n_ch = kc > 0 ? min(n_split, i / kc + 1) : n_split;
  const size_t first = (size_t)bh * n_split * Sr + (i - row0);  // partial row of chunk 0
  // M = max of m over the chunks that saw a key
  float mx = -INFINITY;
  for (int g = lane; g < n_ch; g += 64) {
    const float* ml = part_ml + (first + (size_t)g * Sr) * 3;
    if (ml[2] > 0.f) mx = fmaxf(mx, ml[0]);
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  float den = 0.f, lsum = 0.f;
  for (int g0 = 0; g0 < n_ch; g0 += 64) {
    // this lane's chunk of the block: w = 2^(m - M), and its share of the sums
    float w = 0.f;
    if (g0 + lane < n_ch) {
      const float* ml = part_ml + (first + (size_t)(g0 + lane) * Sr) * 3;
      if (ml[2] > 0.f) {
        w = __builtin_amdgcn_exp2f(ml[0] - mx);
        lsum += w * ml[1];
        den += w * ml[2];
      }
    }
    const int nb = min(64, n_ch - g0);
    int j = 0;
    for (; j + 4 <= nb; j += 4) {
      float wj[4], val[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wj[u] = __shfl(w, j + u);
        const float* po = part_o + (first + (size_t)(g0 + j + u) * Sr) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) val[u][e] = po[e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] += wj[u] * val[u][e];
    }
    for (; j < nb; ++j) {
      const float wj = __shfl(w, j);
      const float* po = part_o + (first + (size_t)(g0 + j) * Sr) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) num[e] += wj * po[e];
    }
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) {
    lsum += __shfl_xor(lsum, s);
    den += __shfl_xor(den, s);
  }
  const float inv = 1.0f / den;
  uint16_t* orow = o + (size_t)((bh / H) * ob + (bh % H) * oh + (long long)i * os);
#pragma unroll
  for (int e = 0; e < PER; e += 2) {
    const uint32_t pk = E::pack2(num[e] * inv, (e + 1 < PER ? num[e + 1] : 0.f) * inv);
    if (PER >= 2) {
      *(uint32_t*)(orow + lane * PER + e) = pk;
    } else {
      orow[lane] = (uint16_t)(pk & 0xffffu);
    }
  }
  if (lane == 0) lse[(size_t)bh * Sq + i] = (mx + __builtin_amdgcn_logf(lsum)) * kLn2;
}

// Launch the merge of rows row0 .. Sq - 1 of B*H heads.
template <int D, int DT>
hipError_t launch_combine(const float* part_o, const float* part_ml, void* o, float* lse, int BH,
                          int H, int Sq, int row0, int kc, int n_split, long long ob, long long oh,
                          long long os, hipStream_t stream) {
  const int n_rows = BH * (Sq - row0);
  fa2_combine_kernel<D, DT><<<dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream>>>(
      part_o, part_ml, (uint16_t*)o, lse, n_rows, H, Sq, row0, kc, n_split, ob, oh, os);
  return hipGetLastError();
}

}  // namespace
