// Launch planning of the library, in plain C++ with no HIP dependency: the
// prefill tile configurations, the key split of small prefill grids, the
// split-KV chunking and default split count, the workspace sizes, and the
// byte-range checks on strided tensors. The entry points use these to shape
// their launches; a CPU harness compiles the same header to check the plans
// (every work item, chunk and partial row accounted for) with the address
// and undefined-behaviour sanitizers.
//
// split_item and causal_split_item also run on the GPU (the prefill kernel
// decodes its work item with them); they are declared __host__ __device__,
// which the HIP compiler provides and a plain C++ build defines away before
// including this header.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace {

// ---- prefill tile configurations ----------------------------------------
// Tile configuration per head dimension:
//   kWaves         waves per workgroup (they share the LDS rings)
//   kRowBlocks     32-row MFMA blocks per wave
//   kBc            keys per tile
//   kWavesPerSimd  waves per SIMD the register budget is sized for
//   kLoadEvery     phase-1 k-steps between this wave's tile-load blocks (0: all
//                  at the start of the step)
//   kStages        stages of the K ring and of the V ring (default 2)
//   kPipelined     1: a wave computes tile j + 1's scores beside tile j's
//                  softmax (two score buffers); 0: scores, softmax and P V of
//                  tile j in sequence, one score buffer, and the other waves
//                  of the SIMD fill the gaps (for registers too tight for two)
//   kKeyGroups     groups of kWaves / kKeyGroups waves that split the key
//                  tiles of one query tile between them (default 1). Each
//                  group owns all B_r rows and streams its own key range
//                  through its own rings; at the end the groups' (m, l, O~)
//                  are merged through LDS, as the pages' split of the keys
//                  across warps merges them.
// Pipelined, iteration j reads K of tile j + 1 and V of tile j while K of
// tile j + kStages and V of tile j + kStages - 1 load; unpipelined, it reads
// K and V of tile j while those of tile j + kStages - 1 load. Either way a
// tile's loads have kStages - 1 iterations to land. Two stages fit two workgroups per compute
// unit at D <= 128. At D = 256 two score buffers leave registers for one wave
// per SIMD only; one buffer (the unpipelined loop) fits two, and two
// workgroups of 32-key tiles with two stages (2 x 2 x 16 KiB each) share a
// unit's LDS.
// The defaults are the best of a sweep over these values on the benchmark
// shapes (flashattention_tiled_amd/tune.py); FA2_TILE_D<D> overrides one, as
// "waves, row blocks, keys, waves per SIMD, load spacing[, stages[,
// pipelined[, key groups]]]". D = 64 and D = 128 have other (ALT)
// configurations. D = 64's first (ALT 1) is for sequences of at least
// FA2_D64_LONG_S: 32-key tiles at four waves per SIMD, 2-4% faster there and
// up to 20% slower on short sequences. The key-group tiles (D = 128's ALT 1,
// D = 64's ALT 2) are for causal grids whose workgroups of the main tile are
// all resident at once (d128_alt, d64_kg): there the longest query tiles set
// the time, run at one wave per SIMD once their compute unit's other
// workgroup is done (or from the start, at one workgroup per unit). These
// tiles split each query tile's keys between two groups of four waves, one
// workgroup per unit, so that every query tile runs at two waves per SIMD to
// its end and the units take the tiles longest first.
template <int W, int RB, int BC, int WPS, int LE, int NST = 2, int PIPE = 1, int KG = 1>
struct TileCfg {
  static constexpr int kWaves = W, kRowBlocks = RB, kBc = BC, kWavesPerSimd = WPS, kLoadEvery = LE,
                       kStages = NST, kPipelined = PIPE, kKeyGroups = KG;
};
#ifndef FA2_TILE_D64
#define FA2_TILE_D64 4, 1, 64, 2, 1
#endif
#ifndef FA2_TILE_D64_LONG
#define FA2_TILE_D64_LONG 4, 1, 32, 4, 0
#endif
#ifndef FA2_D64_LONG_S
#define FA2_D64_LONG_S 8192
#endif
#ifndef FA2_TILE_D64_KG
#define FA2_TILE_D64_KG 8, 1, 64, 2, 1, 2, 1, 2
#endif
#ifndef FA2_TILE_D128
#define FA2_TILE_D128 4, 1, 64, 2, 2
#endif
#ifndef FA2_TILE_D128_ALT
#define FA2_TILE_D128_ALT 8, 1, 64, 2, 2, 2, 1, 2
#endif
#ifndef FA2_TILE_D256
#define FA2_TILE_D256 4, 1, 32, 2, 1, 2, 0
#endif
template <int D, int ALT = 0> struct Tile;
template <> struct Tile<64> : TileCfg<FA2_TILE_D64> {};
template <> struct Tile<64, 1> : TileCfg<FA2_TILE_D64_LONG> {};
template <> struct Tile<64, 2> : TileCfg<FA2_TILE_D64_KG> {};
template <> struct Tile<128> : TileCfg<FA2_TILE_D128> {};
template <> struct Tile<128, 1> : TileCfg<FA2_TILE_D128_ALT> {};
template <> struct Tile<256> : TileCfg<FA2_TILE_D256> {};

template <int D, int ALT = 0> struct Shape {
  static constexpr int kWaves = Tile<D, ALT>::kWaves;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKeyGroups = Tile<D, ALT>::kKeyGroups;
  static constexpr int kGroupWaves = kWaves / kKeyGroups;  // waves of one key group
  static constexpr int kRB = Tile<D, ALT>::kRowBlocks;
  static constexpr int kRowsPerWave = 32 * kRB;
  static constexpr int kBr = kGroupWaves * kRowsPerWave;  // query rows per workgroup
  static constexpr int kBc = Tile<D, ALT>::kBc;
  static constexpr int kChunksPerRow = D / 8;        // 16-byte chunks per key row
  static constexpr int kTileBytes = kBc * D * 2;     // one K or one V tile
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / kGroupWaves;  // per K (or V) tile
  static constexpr int kStages = Tile<D, ALT>::kStages;
  static constexpr bool kPipelined = Tile<D, ALT>::kPipelined != 0;
  static constexpr int kRingBytes = 2 * kStages * kTileBytes;  // one group's K ring + V ring
  // the merge of the key groups: per wave and group, the half of its O~
  // the other group finishes (D / 4 floats per lane) and its m, l and l'
  // per lane, laid out lane-major
  static constexpr int kMergeFloats = D / 4 + 3;
  static constexpr int kMergeBytes =
      kKeyGroups > 1 ? kKeyGroups * kGroupWaves * kMergeFloats * 64 * 4 : 0;
  // Q reaches the registers through LDS in the prologue when the query tile
  // is two key tiles of rows (32 rows per wave, two-stage pipelined rings):
  // its first half in the second stage of a V ring, which the prologue
  // leaves free, its second in the other group's (with key groups) or in a
  // region after the ring
  static constexpr bool kQStaged = kPipelined && kStages == 2 && kRB == 1 && kBr == 2 * kBc;
  static constexpr int kQExtraBytes = kQStaged && kKeyGroups == 1 ? kTileBytes : 0;
  // Unpipelined two-stage tiles whose query tile is the four ring stages'
  // rows (D = 256) load Q through the ring before its first key tiles.
  static constexpr bool kQThroughRing = !kPipelined && kStages == 2 && kRB == 1 && kBr == 4 * kBc;
  static constexpr int kLdsBytes = kKeyGroups * kRingBytes + kQExtraBytes > kMergeBytes
                                       ? kKeyGroups * kRingBytes + kQExtraBytes
                                       : kMergeBytes;
  static_assert(kWaves % kKeyGroups == 0 && kKeyGroups <= 2, "key groups");
  static_assert(kTileBytes % (1024 * kGroupWaves) == 0, "tile must split into 1 KiB wave loads");
  static_assert(kStages >= 2 && (kStages - 2) * 2 * kLoadsPerWave < 64, "ring depth");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// ---- chunk partials (shared by the split-KV path and the key split) ------
// part_o [B*H][n_split][Sr][D] fp32, rounded up to 256 bytes, then
// part_ml [B*H][n_split][Sr][3] fp32 (m in base 2, l, l').
size_t chunk_part_o_bytes(int B, int H, int Sr, int D, int n_split) {
  const size_t b = (size_t)B * H * n_split * Sr * D * sizeof(float);
  return (b + 255) / 256 * 256;
}
size_t chunk_workspace_bytes(int B, int H, int Sr, int D, int n_split) {
  return chunk_part_o_bytes(B, H, Sr, D, n_split) + (size_t)B * H * n_split * Sr * 3 * sizeof(float);
}

// ---- key split of small prefill grids ------------------------------------
// The key split of a launch (ct = 0: none). When there are too few query
// tiles to keep every compute unit busy to the end -- under causal masking
// the last tile of a head has twice the average's keys -- the keys of a
// query tile are cut into chunks of ct key tiles that run as separate
// workgroups, and rows whose tile has more than one chunk leave the chunk
// partials for the merge. Causal: chunks are m query tiles' worth of keys
// (ct = m B_r / B_c), so chunk c of tile qt exists iff c <= qt / m and
// starts at or before the tile's first row, and the rows from row0 = m B_r
// on are merged. Non-causal: every tile has n_split chunks and every row is
// merged (row0 = 0).
struct KeySplit {
  int ct, m, n_qt, n_split, row0;
  float* part_o;
  float* part_ml;
};

// Work item u of one (b, h) under the causal key split, in launch order:
// first the chunks of a full ct tiles, chunk by chunk, then the shorter
// last chunks, longest first (the last chunk of tile qt = c m + r holds
// r + 1 query tiles' worth of keys), so that compute units take the long
// items first and the short ones fill in at the end.
__host__ __device__ __forceinline__ void causal_split_item(int u, int n_qt, int m, int& qt, int& c) {
  for (c = 0;; ++c) {
    const int first = c * m + m - 1;  // the first tile with a full chunk c
    if (first >= n_qt) break;
    if (u < n_qt - first) {
      qt = first + u;
      return;
    }
    u -= n_qt - first;
  }
  for (int r = m - 2; r >= 0; --r) {
    const int p = r < n_qt ? (n_qt - 1 - r) / m + 1 : 0;  // tiles c m + r < n_qt
    if (u < p) {
      c = u;
      qt = c * m + r;
      return;
    }
    u -= p;
  }
  qt = 0;  // not reached: u is below the item count
  c = 0;
}

// Query tile qt and key chunk c of work item u of one (b, h) under a key
// split (ks.ct > 0): the causal order above, or, non-causal, chunk by chunk
// over all n_qt tiles.
__host__ __device__ __forceinline__ void split_item(int u, const KeySplit& ks, bool causal, int& qt,
                                                    int& c) {
  if (causal) {
    causal_split_item(u, ks.n_qt, ks.m, qt, c);
  } else {
    c = u / ks.n_qt;
    qt = u - c * ks.n_qt;
  }
}

// Work items per (b, h) of a launch with n_qt query tiles: the tiles, or
// under a key split every (tile, chunk) pair.
long long split_items_per_head(const KeySplit& ks, int n_qt, bool causal) {
  if (ks.ct == 0) return n_qt;
  if (!causal) return (long long)n_qt * ks.n_split;
  long long n = 0;
  for (int t = 0; t < n_qt; ++t) n += t / ks.m + 1;
  return n;
}

// Shortest key chunk, in keys.
constexpr int kSplitMinChunkKeys = 512;
// The cost model a split must win by kSplitMargin, from measurements on
// MI355X. A compute unit computes about kCuFlopsAlone[D] FLOP/s for a
// workgroup it holds alone (one wave per SIMD) and kCuFlopsFull[D] when
// full, shared among its workgroups (index 0, 1, 2: D = 64, 128, 256). The
// merge reads the partials back and writes O at about kMergeBytesPerSec
// after a fixed kMergeFixedSec, and writing the partials costs the prefill
// kernel about their bytes at kPartialWriteBytesPerSec.
constexpr double kCuFlopsAlone[3] = {2.3e12, 3.7e12, 3.9e12};
constexpr double kCuFlopsFull[3] = {3.3e12, 3.9e12, 3.9e12};
constexpr double kMergeBytesPerSec = 3.0e12;
constexpr double kPartialWriteBytesPerSec = 6.0e12;
constexpr double kMergeFixedSec = 3.0e-6;
constexpr double kSplitMargin = 1.5;

// The key split for a launch of (B, H, S) on n_cu compute units (ct = 0:
// none; the buffers are left unset). Causal grids that leave compute units
// with a single workgroup (one wave per SIMD) -- at most half the
// workgroups the GPU holds at once, or one round where a unit holds just
// one -- end on their longest workgroup, the last query tile of a head
// with all S keys, twice the average. (Causal grids of up to one round on
// units that hold two are kept balanced per unit by the kernel's
// heavy-light tile order, and a split does not speed them up.) Non-causal
// grids are even and only gain where at least half the compute units would
// otherwise idle. The split cuts every tile's keys into chunks: causal, of
// about T / slots key tiles, T being all the tiles of the launch;
// non-causal, into n_cu / tiles chunks per tile, one per compute unit. A
// launch takes at least its longest workgroup's tiles (unsplit: alone on
// its compute unit; split: sharing it with the unit's other workgroups)
// and at least all its work at the whole GPU's rate; the split is taken
// when the time it saves by that estimate beats the merge's cost by
// kSplitMargin.
template <int D, int ALT>
KeySplit plan_split_for(int B, int H, int S, bool causal, int n_cu) {
  using SH = Shape<D, ALT>;
  KeySplit ks{};
  const long long Br = SH::kBr, Bc = SH::kBc, rho = Br / Bc;
  const long long slots = (long long)n_cu * Tile<D, ALT>::kWavesPerSimd * 4 / SH::kWaves;
  const long long n_qt = (S + Br - 1) / Br, n_bh = (long long)B * H, n_t = (S + Bc - 1) / Bc;
  const long long n_wg = n_qt * n_bh;
  const bool one_per_cu = Tile<D, ALT>::kWavesPerSimd * 4 / SH::kWaves < 2;
  const long long max_wg = !causal ? n_cu / 2 : one_per_cu ? slots : slots / 2;
  if (slots < 1 || n_qt < 2 || n_wg > max_wg) return ks;
  long long ct, m = 0, n_split, row0;
  // merged rows x chunks (the partials), merged rows, and all key tiles
  double part_rows, merged_rows, all_tiles;
  if (causal) {
    const long long tiles = n_bh * (rho * (n_qt - 1) * n_qt / 2 + n_t);
    all_tiles = (double)tiles;
    const long long per_slot = (tiles + slots - 1) / slots;
    m = (per_slot + rho / 2) / rho;
    const long long m_min = (kSplitMinChunkKeys + Br - 1) / Br;
    if (m < m_min) m = m_min;
    if (m >= n_qt) return ks;
    ct = m * rho;
    n_split = (n_qt - 1) / m + 1;
    row0 = m * Br;
    double pr = 0;
    for (long long t = m; t < n_qt; ++t) pr += (double)(t / m + 1) * (double)Br;
    part_rows = pr * (double)n_bh;
    merged_rows = (double)(S - row0) * (double)n_bh;
  } else {
    const long long per_tile = n_cu / n_wg;  // chunks per query tile, one per compute unit
    ct = (n_t + per_tile - 1) / per_tile;
    const long long ct_min = (kSplitMinChunkKeys + Bc - 1) / Bc;
    if (ct < ct_min) ct = ct_min;
    n_split = (n_t + ct - 1) / ct;
    if (n_split < 2) return ks;
    row0 = 0;
    merged_rows = (double)S * (double)n_bh;
    part_rows = merged_rows * (double)n_split;
    all_tiles = (double)n_wg * (double)n_t;
  }
  const int di = D == 64 ? 0 : D == 128 ? 1 : 2;
  const long long per_cu = slots / n_cu > 0 ? slots / n_cu : 1;  // workgroups a unit holds
  const double tile_flops = 4.0 * (double)Br * (double)Bc * D;
  const double gpu_sec = all_tiles * tile_flops / ((double)n_cu * kCuFlopsFull[di]);
  // a causal chunk shares its unit with the unit's other workgroups; a
  // non-causal one has it alone
  const double chunk_sec = causal ? (double)ct * tile_flops * (double)per_cu / kCuFlopsFull[di]
                                  : (double)ct * tile_flops / kCuFlopsAlone[di];
  const double saved =
      std::max((double)n_t * tile_flops / kCuFlopsAlone[di], gpu_sec) - std::max(chunk_sec, gpu_sec);
  const double part_bytes = part_rows * (D * 4.0 + 12.0);
  const double merge = kMergeFixedSec + (part_bytes + merged_rows * D * 2.0) / kMergeBytesPerSec +
                       part_bytes / kPartialWriteBytesPerSec;
  if (saved < kSplitMargin * merge) return ks;
  ks.m = (int)m;
  ks.ct = (int)ct;
  ks.n_split = (int)n_split;
  ks.row0 = (int)row0;
  ks.n_qt = (int)n_qt;
  return ks;
}

// Whether a D = 128 launch takes the ALT tile (key groups): causal, not
// split, and the main tile's workgroups all resident at once with at least
// one per compute unit (with fewer, the tiles are short and the split of
// their keys does not pay for the merge). FA2_D128_ALT overrides the rule:
// 0 never, 2 whenever not split.
#ifndef FA2_D128_ALT
#define FA2_D128_ALT 1
#endif
bool d128_alt(int B, int H, int S, bool causal, bool split, int n_cu) {
  using SH = Shape<128>;
  if (FA2_D128_ALT == 0 || split) return false;
  if (FA2_D128_ALT == 2) return true;
  const long long slots = (long long)n_cu * Tile<128>::kWavesPerSimd * 4 / SH::kWaves;
  const long long n_wg = (long long)((S + SH::kBr - 1) / SH::kBr) * B * H;
  return causal && n_wg >= n_cu && n_wg <= slots;
}

// The same rule for the D = 64 key-group tile (below FA2_D64_LONG_S, where
// the long-sequence tile takes over).
bool d64_kg(int B, int H, int S, bool causal, bool split, int n_cu) {
  using SH = Shape<64>;
  if (split || S >= FA2_D64_LONG_S) return false;
  const long long slots = (long long)n_cu * Tile<64>::kWavesPerSimd * 4 / SH::kWaves;
  const long long n_wg = (long long)((S + SH::kBr - 1) / SH::kBr) * B * H;
  return causal && n_wg >= n_cu && n_wg <= slots;
}

KeySplit plan_split(int D, int B, int H, int S, bool causal, int n_cu) {
  switch (D) {
    case 64:
      return S >= FA2_D64_LONG_S ? plan_split_for<64, 1>(B, H, S, causal, n_cu)
                                 : plan_split_for<64, 0>(B, H, S, causal, n_cu);
    case 128: return plan_split_for<128, 0>(B, H, S, causal, n_cu);
    default: return plan_split_for<256, 0>(B, H, S, causal, n_cu);
  }
}

// Workspace bytes of a key split (0 for none).
size_t split_workspace_bytes(const KeySplit& ks, int B, int H, int S, int D) {
  return ks.ct == 0 ? 0 : chunk_workspace_bytes(B, H, S - ks.row0, D, ks.n_split);
}

// ---- split-KV decoding ---------------------------------------------------
// KV8: K and V hold FP8 e4m3 codes (one byte per element) instead of 16-bit
// values.
template <int D, bool KV8 = false> struct SplitTile {
  static constexpr int kBc = 32;
  static constexpr int kTileBytes = kBc * D * (KV8 ? 1 : 2);
  static constexpr int kLoadsPerWave = kTileBytes / 1024;  // one wave loads the whole tile
  static constexpr int kLdsBytes = 4 * kTileBytes;         // K and V, two stages each
  static_assert(kTileBytes % 1024 == 0, "a tile is whole 1 KiB wave loads");
};

// Default number of key chunks per (b, h): about two one-wave workgroups
// per compute unit for 16-bit K and V, four for FP8 (a chunk holds half the
// bytes), each chunk at least 4 tiles long. Measured on decode shapes:
// more, shorter chunks lose bandwidth.
int splitkv_default_splits(int B, int H, int Sq, int Sk, int n_cu, bool kv8) {
  const long long n_qblk = (Sq + 31) / 32;
  const long long n_tiles = (Sk + SplitTile<64>::kBc - 1) / SplitTile<64>::kBc;
  const long long target = (kv8 ? 4LL : 2LL) * n_cu;
  long long want = (target + (long long)B * H * n_qblk - 1) / ((long long)B * H * n_qblk);
  const long long cap = n_tiles / 4 > 0 ? n_tiles / 4 : 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  if (want > 1024) want = 1024;
  return (int)want;
}

// The chunks a split-KV launch runs for Sk keys asked to split n_split ways:
// chunks of chunk_tiles whole tiles of Bc keys, the trailing ones that
// would be empty dropped, leaving n_eff <= n_split chunks.
void splitkv_chunking(int Sk, int Bc, int n_split, int& chunk_tiles, int& n_eff) {
  const int n_tiles = (Sk + Bc - 1) / Bc;
  chunk_tiles = (n_tiles + n_split - 1) / n_split;
  n_eff = (n_tiles + chunk_tiles - 1) / chunk_tiles;
}

}  // namespace

// ---- byte ranges of strided tensors --------------------------------------
namespace fa2_host {
namespace {

// Whether byte ranges [a, a + na) and [b, b + nb) overlap.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Whether the rows (b, h, s) of a (B, H, S, D) tensor with these element
// strides (head dim contiguous) are sure to be pairwise disjoint: taking
// the dims of size > 1 in ascending stride order, each stride must reach
// past the span of the dims before it. That holds for every permutation of
// a contiguous tensor and of a padded one; a layout whose rows interleave
// without overlapping is refused too (a sufficient test, not a necessary
// one).
bool rows_disjoint(int B, int H, int S, int D, long long sb, long long sh, long long ss) {
  long long n[3] = {B, H, S}, st[3] = {sb, sh, ss};
  for (int i = 1; i < 3; ++i)
    for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
      const long long tn = n[j], ts = st[j];
      n[j] = n[j - 1];
      st[j] = st[j - 1];
      n[j - 1] = tn;
      st[j - 1] = ts;
    }
  long long span = D;
  for (int i = 0; i < 3; ++i) {
    if (n[i] < 2) continue;
    if (st[i] < span) return false;
    span += st[i] * (n[i] - 1);
  }
  return true;
}

// Whether B * H * S * D elements (and twice that in bytes) fit in int64.
bool elements_fit_int64(long long B, long long H, long long S, long long D) {
  if (B < 1 || H < 1 || S < 1 || D < 1) return false;
  const long long lim = 0x3fffffffffffffffLL;  // int64 max / 2
  long long n = B;
  for (long long f : {H, S, D}) {
    if (n > lim / f) return false;
    n *= f;
  }
  return true;
}

// Bytes from a strided (B, H, S, D) tensor's base pointer to the end of its
// last element.
size_t extent_bytes(int B, int H, int S, int D, long long sb, long long sh, long long ss,
                    int elem_bytes) {
  return (size_t)(((long long)(B - 1) * sb + (long long)(H - 1) * sh + (long long)(S - 1) * ss +
                   D) * elem_bytes);
}

}  // namespace
}  // namespace fa2_host
