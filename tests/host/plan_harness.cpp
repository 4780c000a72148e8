// CPU harness for the library's launch planning (csrc/fa2_plan.h), built
// with g++ under the address and undefined-behaviour sanitizers by
// tests/test_plan_harness.py. It walks every plan the library can make over
// a grid of shapes and device sizes and checks what the kernels rely on:
//
// key split of the prefill (fa2_fwd_balanced):
//   - every (query tile, key chunk) pair is one work item, exactly once;
//   - the chunks of a tile cover its key tiles exactly once, none empty,
//     and (causal) each starts at or before the tile's first row, so its
//     first tile holds a key every row keeps;
//   - every partial row the prefill kernel writes lies inside the
//     workspace the entry point asks for, and the merge's chunk count per
//     row is the number of chunks that wrote it;
//   - the grid stays within 32-bit workgroup indices;
// split-KV decoding (fa2_fwd_splitkv):
//   - the chunks cover the key tiles exactly once, none empty, at most the
//     requested count, and their partial rows fit the workspace;
//   - the default split count stays in [1, 1024] and leaves chunks of at
//     least four tiles;
// strided tensors:
//   - every layout rows_disjoint accepts has disjoint rows by a brute-force
//     check of every element, every nested layout is accepted, and
//     extent_bytes is the largest element offset, on small shapes.
//
// Exit status 0 and a summary line on success; the first failure prints
// what it was and exits 1.
#define __host__
#define __device__
#define __forceinline__ inline
#include "fa2_plan.h"

#include <cstdio>
#include <cstdlib>
#include <set>
#include <utility>
#include <vector>

namespace {

long long g_checks = 0;

#define CHECK(cond, ...)                                            \
  do {                                                              \
    ++g_checks;                                                     \
    if (!(cond)) {                                                  \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                            \
      std::fprintf(stderr, "\n");                                   \
      std::exit(1);                                                 \
    }                                                               \
  } while (0)

template <int D, bool LONG>
int check_key_split(int B, int H, int S, bool causal, int n_cu) {
  using SH = Shape<D, LONG>;
  const KeySplit ks = plan_split(D, B, H, S, causal, n_cu);
  const int Br = SH::kBr, Bc = SH::kBc;
  const int n_qt = (S + Br - 1) / Br;
  const char* fmt = "D=%d B=%d H=%d S=%d causal=%d n_cu=%d";
#define ARGS D, B, H, S, (int)causal, n_cu
  if (ks.ct == 0) {
    CHECK(split_workspace_bytes(ks, B, H, S, D) == 0, fmt, ARGS);
    CHECK(split_items_per_head(ks, n_qt, causal) == n_qt, fmt, ARGS);
    return 0;
  }
  const int n_t = (S + Bc - 1) / Bc;
  CHECK(ks.n_qt == n_qt && ks.ct >= 1 && ks.n_split >= 2, fmt, ARGS);
  if (causal) {
    CHECK(ks.m >= 1 && ks.ct == ks.m * (Br / Bc) && ks.row0 == ks.m * Br, fmt, ARGS);
    CHECK(ks.n_split == (n_qt - 1) / ks.m + 1 && ks.row0 < S, fmt, ARGS);
  } else {
    CHECK(ks.row0 == 0 && ks.n_split == (n_t + ks.ct - 1) / ks.ct, fmt, ARGS);
  }
  const long long items = split_items_per_head(ks, n_qt, causal);
  CHECK(items * H * B < (1LL << 31), fmt, ARGS);
  auto n_chunks = [&](int qt) { return causal ? qt / ks.m + 1 : ks.n_split; };
  // every (tile, chunk) pair exactly once
  std::vector<std::vector<int>> seen(n_qt);
  for (int qt = 0; qt < n_qt; ++qt) seen[qt].assign(n_chunks(qt), 0);
  for (long long u = 0; u < items; ++u) {
    int qt = -1, c = -1;
    split_item((int)u, ks, causal, qt, c);
    CHECK(qt >= 0 && qt < n_qt && c >= 0 && c < n_chunks(qt), "%s item %lld -> (%d, %d)",
          "bad item", u, qt, c);
    CHECK(seen[qt][c] == 0, "item %lld repeats (tile %d, chunk %d); D=%d S=%d", u, qt, c, D, S);
    seen[qt][c] = 1;
  }
  for (int qt = 0; qt < n_qt; ++qt)
    for (int c = 0; c < n_chunks(qt); ++c)
      CHECK(seen[qt][c] == 1, "tile %d chunk %d never launched; D=%d S=%d", qt, c, D, S);
  // key coverage, chunk starts, partial rows and the merge's chunk counts
  const int Sr = S - ks.row0;
  const size_t ws = split_workspace_bytes(ks, B, H, S, D);
  CHECK(ws == chunk_workspace_bytes(B, H, Sr, D, ks.n_split), fmt, ARGS);
  const size_t o_bytes = chunk_part_o_bytes(B, H, Sr, D, ks.n_split);
  const size_t ml_bytes = ws - o_bytes;
  for (int qt = 0; qt < n_qt; ++qt) {
    const int kv_end = causal ? std::min((qt + 1) * Br, S) : S;
    const int t_all = (kv_end + Bc - 1) / Bc;
    int next = 0;  // the key tile the next chunk must start at
    for (int c = 0; c < n_chunks(qt); ++c) {
      const int t0 = c * ks.ct, t_stop = std::min(t_all, t0 + ks.ct);
      CHECK(t0 == next && t0 < t_stop, "tile %d chunk %d keys [%d, %d) after %d; D=%d S=%d", qt,
            c, t0, t_stop, next, D, S);
      if (causal) CHECK(t0 * Bc <= qt * Br, "chunk %d of tile %d starts past its first row", c, qt);
      next = t_stop;
    }
    CHECK(next == t_all, "tile %d: chunks end at key tile %d of %d; D=%d S=%d", qt, next, t_all,
          D, S);
    const int r_end = std::min((qt + 1) * Br, S);
    for (int row = qt * Br; row < r_end; ++row) {
      const bool merged = n_chunks(qt) > 1;
      CHECK(merged == (row >= ks.row0), "row %d: merged %d but row0 %d", row, (int)merged,
            ks.row0);
      if (!merged) continue;
      const int kc = causal ? ks.row0 : 0;
      const int n_ch = kc > 0 ? std::min(ks.n_split, row / kc + 1) : ks.n_split;
      CHECK(n_ch == n_chunks(qt), "row %d: merge reads %d chunks, %d wrote", row, n_ch,
            n_chunks(qt));
      // the first and the last (b, h): partial rows grow with bh
      for (int bh : {0, B * H - 1}) {
        for (int c = 0; c < n_chunks(qt); ++c) {
          const size_t prow = ((size_t)bh * ks.n_split + c) * (size_t)Sr + (size_t)(row - ks.row0);
          CHECK((prow + 1) * D * sizeof(float) <= o_bytes, "partial O row past the workspace");
          CHECK((prow + 1) * 3 * sizeof(float) <= ml_bytes, "partial (m, l) past the workspace");
        }
      }
    }
  }
#undef ARGS
  return 1;
}

int check_key_split_any(int D, int B, int H, int S, bool causal, int n_cu) {
  switch (D) {
    case 64:
      return S >= FA2_D64_LONG_S ? check_key_split<64, true>(B, H, S, causal, n_cu)
                                 : check_key_split<64, false>(B, H, S, causal, n_cu);
    case 128: return check_key_split<128, false>(B, H, S, causal, n_cu);
    default: return check_key_split<256, false>(B, H, S, causal, n_cu);
  }
}

void check_splitkv(int B, int H, int Sq, int Sk, int D, int n_split) {
  const int Bc = SplitTile<64>::kBc;
  int chunk_tiles = 0, n_eff = 0;
  splitkv_chunking(Sk, Bc, n_split, chunk_tiles, n_eff);
  const int n_tiles = (Sk + Bc - 1) / Bc;
  CHECK(chunk_tiles >= 1 && n_eff >= 1 && n_eff <= n_split, "Sk=%d n_split=%d", Sk, n_split);
  int next = 0;
  for (int c = 0; c < n_eff; ++c) {
    const int t0 = c * chunk_tiles, t1 = std::min(n_tiles, t0 + chunk_tiles);
    CHECK(t0 == next && t0 < t1, "Sk=%d n_split=%d chunk %d empty or misplaced", Sk, n_split, c);
    next = t1;
  }
  CHECK(next == n_tiles, "Sk=%d n_split=%d: chunks end at %d of %d tiles", Sk, n_split, next,
        n_tiles);
  // the partial rows of the last (b, h), last chunk, last row fit the
  // workspace sized for n_split chunks (the kernel lays them out for n_eff)
  const size_t ws = chunk_workspace_bytes(B, H, Sq, D, n_split);
  const size_t o_bytes = chunk_part_o_bytes(B, H, Sq, D, n_eff);
  const size_t prow = ((size_t)(B * H - 1) * n_eff + (n_eff - 1)) * Sq + (Sq - 1);
  CHECK((prow + 1) * D * sizeof(float) <= o_bytes, "split-KV partial O row past its region");
  CHECK(o_bytes + (prow + 1) * 3 * sizeof(float) <= ws, "split-KV partial (m, l) past the workspace");
}

void check_default_splits(int B, int H, int Sq, int Sk, int n_cu) {
  for (bool kv8 : {false, true}) {
    const int n = splitkv_default_splits(B, H, Sq, Sk, n_cu, kv8);
    const int n_tiles = (Sk + 31) / 32;
    CHECK(n >= 1 && n <= 1024, "default splits %d", n);
    CHECK(n == 1 || n <= n_tiles / 4, "default splits %d leave chunks under 4 tiles (%d tiles)",
          n, n_tiles);
  }
  CHECK(splitkv_default_splits(B, H, Sq, Sk, n_cu, true) >=
            splitkv_default_splits(B, H, Sq, Sk, n_cu, false),
        "the FP8 default is below the 16-bit one (the workspace query sizes for the FP8 one)");
}

// Brute force over every element of a small strided tensor. rows_disjoint
// is a sufficient test: it may refuse a layout whose rows interleave without
// overlapping (the entry points then reject it), but a layout it accepts
// must have disjoint rows, and a nested one -- each stride of a dim of size
// > 1 past the span of the smaller ones, as every permutation of a
// contiguous tensor is -- must be accepted.
void check_strides(unsigned seed, long long& n_accepted, long long& n_refused_disjoint) {
  std::srand(seed);
  for (int trial = 0; trial < 20000; ++trial) {
    const int B = 1 + std::rand() % 3, H = 1 + std::rand() % 3, S = 1 + std::rand() % 4;
    const int D = 8 * (1 + std::rand() % 2);
    const long long sb = 8 * (std::rand() % 10), sh = 8 * (std::rand() % 10),
                    ss = 8 * (std::rand() % 6);
    std::set<long long> all;
    bool disjoint = true;
    long long max_off = 0;
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int s = 0; s < S; ++s)
          for (int d = 0; d < D; ++d) {
            const long long off = b * sb + h * sh + s * ss + d;
            max_off = std::max(max_off, off);
            if (!all.insert(off).second) disjoint = false;
          }
    const bool accepted = fa2_host::rows_disjoint(B, H, S, D, sb, sh, ss);
    CHECK(!accepted || disjoint,
          "rows_disjoint accepts overlapping rows: B=%d H=%d S=%d D=%d sb=%lld sh=%lld ss=%lld", B,
          H, S, D, sb, sh, ss);
    n_accepted += accepted ? 1 : 0;
    n_refused_disjoint += (!accepted && disjoint) ? 1 : 0;
    for (int eb : {1, 2}) {
      CHECK(fa2_host::extent_bytes(B, H, S, D, sb, sh, ss, eb) == (size_t)(max_off + 1) * eb,
            "extent_bytes(B=%d H=%d S=%d D=%d sb=%lld sh=%lld ss=%lld)", B, H, S, D, sb, sh, ss);
    }
    // the six nested (permuted contiguous) layouts of the same sizes
    const int n[3] = {B, H, S};
    const int perms[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2}, {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
    for (const auto& p : perms) {
      long long st[3], span = D;
      for (int i = 2; i >= 0; --i) {  // p[2] innermost
        st[p[i]] = span;
        span *= n[p[i]];
      }
      CHECK(fa2_host::rows_disjoint(B, H, S, D, st[0], st[1], st[2]),
            "nested layout refused: B=%d H=%d S=%d D=%d strides %lld %lld %lld", B, H, S, D, st[0],
            st[1], st[2]);
    }
  }
}

}  // namespace

int main() {
  const int s_list[] = {1,    2,    63,   64,   127,  128,  129,  255,  256,   511,   512,  600,
                        1000, 1024, 1500, 2047, 2048, 2049, 3000, 4096, 4097,  6000,  8191, 8192,
                        8193, 9000, 12001, 16384, 16385, 20000, 32768, 65537};
  const int n_cu_list[] = {256, 304, 228, 120, 80, 64, 32, 8, 1};
  long long plans = 0, shapes = 0;
  for (int D : {64, 128, 256})
    for (int n_cu : n_cu_list)
      for (int B : {1, 2, 3, 4})
        for (int H : {1, 2, 3, 4, 5, 8, 16})
          for (int S : s_list)
            for (bool causal : {false, true}) {
              ++shapes;
              plans += check_key_split_any(D, B, H, S, causal, n_cu);
            }
  long long skv = 0;
  for (int Sk : {1, 2, 31, 32, 33, 100, 127, 128, 129, 1000, 4097, 32768, 131072})
    for (int n_split = 1; n_split <= 70; ++n_split)
      for (int Sq : {1, 16, 33}) {
        check_splitkv(3, 5, Sq, Sk, 128, n_split);
        ++skv;
      }
  for (int n_cu : n_cu_list)
    for (int B : {1, 4, 8})
      for (int H : {1, 8, 32})
        for (int Sq : {1, 16, 70})
          for (int Sk : {1, 100, 4096, 131072, 1 << 20}) check_default_splits(B, H, Sq, Sk, n_cu);
  long long accepted = 0, refused_disjoint = 0;
  check_strides(12345u, accepted, refused_disjoint);
  std::printf("plan harness OK: %lld prefill shapes, %lld key-split plans, %lld split-KV plans, "
              "%lld strided layouts accepted (%lld disjoint ones refused), %lld checks\n",
              shapes, plans, skv, accepted, refused_disjoint, g_checks);
  return 0;
}
