// FlashAttention-2 forward pass with FP8 (OCP e4m3) Q, K and V for MI355X
// (gfx950 / CDNA4), on the FP8 matrix cores.
//
// The infra.bea.ai FlashAttention V2 guide names FP8 as the way
// FlashAttention-3 gets more throughput ("FlashAttention-3 and Beyond").
// Here both products of the forward pass run on gfx950's e4m3 matrix-core
// instruction v_mfma_f32_32x32x64_f8f6f4, twice the rate of the 16-bit one:
//   S^T = K_j Q^T      (A = K_j e4m3 codes from LDS, B = Q^T codes resident in
//                       registers; 64 head dims per product)
//   O~^T += V_j^T P8^T (A = V_j^T codes read transposed from LDS, B = P8^T,
//                       64 keys per product)
// with the values being codes times per-tensor descales: the score scale c
// = scale * log2(e) * q_descale * k_descale multiplies the fp32 products,
// and v_descale multiplies O~ in the epilogue.
//
// The online softmax is the 16-bit kernel's (fa2_fwd.hip): base-2 logits,
// a lazily moved reference max m, l summed in fp32 over P as computed (for
// lse), O~ normalised in the epilogue by a second sum, of P as rounded. What
// FP8 changes:
//  - P is rounded to e4m3 for the P V product as P8 = 2^(t - m + kP8Exp),
//    so that the largest P of a row, 2^kP8Exp, sits well inside e4m3's
//    normal range and small P keep their precision longer before they fall
//    into the subnormals. A tile is redone with a raised m whenever its
//    row max of t passes m + kP8Headroom, which keeps every P8 at most 448,
//    e4m3's largest finite value.
//  - The sum of P8 as rounded comes from one more product per tile, a row
//    of e4m3 ones against P8^T (there is no FP8 dot instruction on gfx950),
//    so O is divided by exactly the weights it was accumulated with.
//
// Operand layouts (lane l, l32 = l % 32, hi = l / 32): for the 32x32x64
// product, A and B lanes hold row / column l32 and k = 32 hi .. 32 hi + 31,
// one byte each; C is the 16-bit kernel's 32x32 accumulator (register r of
// lane l: row 8 (r / 4) + 4 hi + r % 4, column l32). P8^T byte e of a lane
// is accumulator register e % 16 of key block e / 16, i.e. key
// 32 (e / 16) + 8 ((e % 16) / 4) + 4 hi + e % 4, and the V^T operand gathers
// the same keys: each of its four ds_read_b64_tr_b8 reads (key block kb,
// half h) gives a lane 8 keys of its head dim (see fa2_splitkv.hip for the
// read's lane mapping). K and V tiles are rows of D codes with the
// 16-byte-chunk swizzles of fa2_tile.h's FP8 helpers.

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// P8 = 2^(t - m + kP8Exp): m's own P8 is 64.
constexpr int kP8Exp = 6;
// A tile is redone when its row max of t exceeds m by more than this:
// 64 * 2^2.75 = 430.5 <= 448, with room for the fp32 rounding of t - m.
constexpr float kP8Headroom = 2.75f;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // operand formats 0, 0: e4m3 both; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Tile shape of the FP8 kernel: 4 waves of 32 query rows, 64-key tiles,
// two waves per SIMD, two-stage K and V rings. At D = 256 the key loop is
// unpipelined (one score buffer: a second does not fit beside Q^T and O~ in
// 256 registers), as in the 16-bit kernel.
template <int D> struct Fp8Shape {
  static constexpr int kWaves = 4, kThreads = 256, kBr = 128, kBc = 64;
  static constexpr bool kSerial = D == 256;
  static constexpr int kTileBytes = kBc * D;  // one K or V tile of codes
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;
  // K and V rings, two stages each; with the pipelined loop also a region
  // for the second half of Q (loaded through LDS in the prologue: its first
  // half goes to V's second stage, which the prologue leaves free)
  static constexpr int kLdsBytes = (kSerial ? 4 : 5) * kTileBytes;
  static constexpr int kKSteps = D / 64;            // products per 32-key block of S^T
  static_assert(kLoadsPerWave >= 1 && kTileBytes % (1024 * kWaves) == 0, "wave loads");
};

// Tile max of t = c_eff * scores per row. c_eff is never negative here: the
// kernel takes a negative scale as its magnitude with Q's codes negated
// (masked tiles are scaled already, c_eff = 1).
template <int NKB>
__device__ __forceinline__ float fp8_tile_max(const f32x16 (&acc)[1][NKB], float c_eff) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, acc[0][kb][r]), acc[0][kb][r + 1]);
  return xor32_max(mx * c_eff);
}

// P8 of one tile for this lane's row: 32 values 2^(t - m + kP8Exp), their
// fp32 sum, and their e4m3 codes packed as the B operand (byte e = register
// e % 16 of key block e / 16).
template <int NKB>
__device__ __forceinline__ void fp8_probs(const f32x16 (&acc)[1][NKB], float c_eff, float m8,
                                          float& tsum, i32x8& pb) {
  static_assert(NKB == 2, "one 64-key product per tile");
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int kb = w / 4, r = 4 * (w % 4);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(acc[0][kb][r], c_eff, -m8));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(acc[0][kb][r + 1], c_eff, -m8));
    const float p2 = __builtin_amdgcn_exp2f(fmaf(acc[0][kb][r + 2], c_eff, -m8));
    const float p3 = __builtin_amdgcn_exp2f(fmaf(acc[0][kb][r + 3], c_eff, -m8));
    s0 += p0 + p1;
    s1 += p2 + p3;
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
    pb[w] = x;
  }
  tsum = s0 + s1;
}

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa2_fwd_fp8_kernel(
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ k,
    const unsigned char* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int S,
    float c /* scale * log2(e) * q_descale * k_descale */, float v_mult, int pair_split,
    int tk_from, unsigned int* __restrict__ tk) {
  using SH = Fp8Shape<D>;
  constexpr int Br = SH::kBr, Bc = SH::kBc, TB = SH::kTileBytes, LPW = SH::kLoadsPerWave;
  constexpr int NKB = Bc / 32, NKS = SH::kKSteps, NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SH::kLdsBytes];
  constexpr uint32_t kK0 = 0, kK1 = TB, kV0 = 2 * TB, kV1 = 3 * TB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // workgroup -> (query tile, batch * head): the 16-bit kernel's order
  // (longest causal tiles first, a head's tiles H * B apart in launch order,
  // the second half ascending when the grid is resident at once, and the
  // last quarter of a multi-round grid by ticket, in the order they start)
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
  const int n_qt = gridDim.x;
  const int qt =
      (pair_split > 0 && lin >= pair_split) ? (lin - pair_split) / n_bh : n_qt - 1 - lin_t / n_bh;
  const int q0 = qt * Br;
  const int wave_row0 = q0 + wave * 32;
  const size_t head = (size_t)bh * (size_t)S * D;

  // Q^T operands: k-step s of this lane's row, dims 64 s + 32 hi .. + 31.
  // A negative scale is taken as its magnitude with every Q code negated
  // (the sign bit flipped: exact), so the score scale c is never negative.
  const int q_sign = c < 0.f ? (int)0x80808080 : 0;
  c = fabsf(c);
  i32x8 qf[NKS];
  if constexpr (SH::kSerial) {
    const int row = wave_row0 + l32;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qf[s] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (row < S) qf[s] = *(const i32x8*)(q + head + (size_t)row * D + 64 * s + 32 * hi) ^ q_sign;
    }
  }

  constexpr int kv_cap = 0x7fffffff / D;  // rows one tile load may reach
  const unsigned char* k_head = k + head;
  const unsigned char* v_head = v + head;
  uint32_t k_off[LPW], v_off[LPW];
  tile_load_offsets8<D, LPW, false>(wave, lane, D, k_off);
  tile_load_offsets8<D, LPW, true>(wave, lane, D, v_off);

  // K operand of (key block kb, k-step s): row 32 kb + l32, chunks
  // 4 s + 2 hi and 4 s + 2 hi + 1, swizzled (the swizzle does not depend on kb)
  const int ksw = swz_k8<D>(l32);
  uint32_t k_rd[NKS][2];
#pragma unroll
  for (int s = 0; s < NKS; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      k_rd[s][u] = (uint32_t)(l32 * D + 16 * ((4 * s + 2 * hi + u) ^ ksw));
  // V^T source address of this lane: key row R(e) = 8 (e / 4) + 4 hi + e % 4
  // of each 16-key half, e = (lane % 16) / 2; dims 16 ((lane / 16) % 2) +
  // 8 (lane % 2) of each 32-dim block, whose chunk pair is XORed with the
  // row's swizzle
  const int e8 = (lane & 15) >> 1, grp8 = (lane >> 4) & 1;
  const int r8 = 8 * (e8 >> 2) + 4 * hi + (e8 & 3);
  const uint32_t v8_base = (uint32_t)(r8 * D + 16 * grp8 + 8 * (lane & 1));
  const uint32_t v8_x = (uint32_t)(16 * swz_v8<D>(r8));
  i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
  // The empty asm hides the constant from the optimiser, so it stays in eight
  // registers for the whole loop instead of being rebuilt before each use
  // (saves about 14 moves per key tile). At D = 256 no registers are spare.
  if constexpr (!SH::kSerial) __asm__ volatile("" : "+v"(ones));

  f32x16 acc_o[NDB], acc_l;
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  acc_l = f32x16{};
  float m_run = 0.f, l_run = 0.f;  // reference max (base 2), this lane's share of l (P8 units)

  const int kv_end = CAUSAL ? min(q0 + Br, S) : S;
  const int n_tiles = (kv_end + Bc - 1) / Bc;
  const int n_act = CAUSAL ? min(n_tiles, (wave_row0 + 32 + Bc - 1) / Bc) : n_tiles;

  auto k_tile = [&](int rows, int t) { return tile_rsrc_rows(k_head, rows, t * Bc, D, kv_cap); };
  auto v_tile = [&](int rows, int t) { return tile_rsrc_rows(v_head, rows, t * Bc, D, kv_cap); };

  auto scores = [&](uint32_t k_stage, f32x16 (&acc)[1][NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      acc[0][kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const unsigned char* base = smem + k_stage + kb * 32 * D;
        const u32x4 lo = *(const u32x4*)(base + k_rd[s][0]);
        const u32x4 up = *(const u32x4*)(base + k_rd[s][1]);
        const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
        acc[0][kb] = mfma_fp8(a, qf[s], acc[0][kb]);
      }
    }
  };
  auto pv = [&](uint32_t v_stage, const i32x8& pb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      i32x8 a;
#pragma unroll
      for (int t = 0; t < 4; ++t) {  // (key block, half) = (t / 2, t % 2)
        const uint32_t addr = v_stage + (uint32_t)((16 * t) * D) + v8_base +
                              ((uint32_t)(32 * db) ^ v8_x);
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(smem + addr));
        a[2 * t] = raw[0];
        a[2 * t + 1] = raw[1];
      }
      acc_o[db] = mfma_fp8(a, pb, acc_o[db]);
    }
    acc_l = mfma_fp8(ones, pb, acc_l);
  };

  // the headroom test on a tile's scores: raise m to the tile's row max
  // first if any row of the wave needs it (rare, wave-uniform)
  auto headroom = [&](const f32x16 (&sc)[1][NKB], float ce) {
    const float tmax = fp8_tile_max<NKB>(sc, ce);
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kP8Headroom) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      acc_l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
  };

  if constexpr (SH::kSerial) {
    // Unpipelined: iteration j computes tile j from stage j % 2 (scores,
    // headroom test, P8, P V) after its loads (issued in iteration j - 1)
    // have landed and every wave is done with iteration j - 1, whose stages
    // then take tile j + 1.
    load_tile_rsrc<LPW>(k_tile(S, 0), smem + kK0, wave, k_off);
    load_tile_rsrc<LPW>(v_tile(S, 0), smem + kV0, wave, v_off);
    auto step_s = [&](auto par, int j) {
      constexpr int PAR = decltype(par)::value;
      const uint32_t k_cur = PAR ? kK1 : kK0, k_free = PAR ? kK0 : kK1;
      const uint32_t v_cur = PAR ? kV1 : kV0, v_free = PAR ? kV0 : kV1;
      wait_vm_lgkm0<0>();
      workgroup_barrier();
      load_tile_rsrc<LPW>(k_tile(j + 1 < n_tiles ? S : 0, j + 1), smem + k_free, wave, k_off);
      load_tile_rsrc<LPW>(v_tile(j + 1 < n_tiles ? S : 0, j + 1), smem + v_free, wave, v_off);
      if (j < n_act) {
        f32x16 sc[1][NKB];
        float ce[1];
        scores(k_cur, sc);
        if (tile_needs_mask<1, NKB, CAUSAL>(j * Bc, wave_row0, S))
          tile_mask<1, NKB, CAUSAL>(sc, j * Bc, wave_row0, S, c, l32, hi, ce);
        else
          ce[0] = c;
        // m starts at the row max of tile 0, which holds key 0 <= every row
        if (j == 0) m_run = fp8_tile_max<NKB>(sc, ce[0]);
        headroom(sc, ce[0]);
        float tsum;
        i32x8 pb;
        fp8_probs<NKB>(sc, ce[0], m_run - (float)kP8Exp, tsum, pb);
        l_run += tsum;
        pv(v_cur, pb);
      }
    };
    for (int j = 0; j < n_tiles; j += 2) {
      step_s(std::integral_constant<int, 0>{}, j);
      if (j + 1 < n_tiles) step_s(std::integral_constant<int, 1>{}, j + 1);
    }
  } else {
    // prologue: Q in whole 1 KiB blocks through LDS (rows Bc h .. Bc h +
    // Bc - 1 in K's layout: half 0 into V's second stage, which the first
    // step refills after every wave has read it, half 1 into the region
    // after the rings), K and V of tile 0 and K of tile 1; then Q and K of
    // tile 0 before the first scores
    static_assert(Br == 2 * Bc, "Q is two key tiles of rows");
    const unsigned char* q_head = q + head;
    load_tile_rsrc<LPW>(tile_rsrc_rows(q_head, S, q0, D, kv_cap), smem + kV1, wave, k_off);
    load_tile_rsrc<LPW>(tile_rsrc_rows(q_head, S, q0 + Bc, D, kv_cap), smem + 4 * TB, wave, k_off);
    load_tile_rsrc<LPW>(k_tile(S, 0), smem + kK0, wave, k_off);
    load_tile_rsrc<LPW>(v_tile(S, 0), smem + kV0, wave, v_off);
    if (n_tiles > 1) load_tile_rsrc<LPW>(k_tile(S, 1), smem + kK1, wave, k_off);

    f32x16 s_a[1][NKB], s_b[1][NKB];
    float ce_a[1], ce_b[1];
    if (n_tiles > 1)
      wait_vm_lgkm0<2 * LPW>();
    else
      wait_vm_lgkm0<LPW>();
    workgroup_barrier();
    {
      // this wave's rows: rows 32 (wave % 2) .. + 31 of half wave / 2
      const unsigned char* qb = smem + (wave / 2 == 0 ? kV1 : 4 * TB) + (wave % 2) * 32 * D;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const u32x4 lo = *(const u32x4*)(qb + k_rd[s][0]);
        const u32x4 up = *(const u32x4*)(qb + k_rd[s][1]);
        qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)up[0], (int)up[1], (int)up[2], (int)up[3]} ^ q_sign;
      }
    }
    if (n_act > 0) {
      // m starts at the row max of tile 0, which holds key 0 <= every row
      scores(kK0, s_a);
      tile_mask<1, NKB, CAUSAL>(s_a, 0, wave_row0, S, c, l32, hi, ce_a);
      m_run = fp8_tile_max<NKB>(s_a, ce_a[0]);
    }

    // One step for tile j (parity PAR): scores of tile j + 1 beside the
    // probabilities of tile j, the headroom test, then P V of tile j.
    auto step = [&](auto par, int j, f32x16 (&cur)[1][NKB], float (&ce_cur)[1],
                    f32x16 (&nxt)[1][NKB], float (&ce_nxt)[1]) {
      constexpr int PAR = decltype(par)::value;
      const uint32_t k_next = PAR ? kK0 : kK1, k_free = PAR ? kK1 : kK0;
      const uint32_t v_cur = PAR ? kV1 : kV0, v_free = PAR ? kV0 : kV1;
      wait_vm_lgkm0<0>();
      workgroup_barrier();
      // K of tile j + 2 into tile j's K stage, V of tile j + 1 into tile
      // j - 1's V stage (tiles past the last get zero-length buffers)
      load_tile_rsrc<LPW>(k_tile(j + 2 < n_tiles ? S : 0, j + 2), smem + k_free, wave,
                          k_off);
      load_tile_rsrc<LPW>(v_tile(j + 1 < n_tiles ? S : 0, j + 1), smem + v_free, wave,
                          v_off);
      if (j < n_act) {
        scores(k_next, nxt);
        headroom(cur, ce_cur[0]);
        float tsum;
        i32x8 pb;
        fp8_probs<NKB>(cur, ce_cur[0], m_run - (float)kP8Exp, tsum, pb);
        l_run += tsum;
        pv(v_cur, pb);
        if (j + 1 < n_act) {
          if (tile_needs_mask<1, NKB, CAUSAL>((j + 1) * Bc, wave_row0, S))
            tile_mask<1, NKB, CAUSAL>(nxt, (j + 1) * Bc, wave_row0, S, c, l32, hi, ce_nxt);
          else
            ce_nxt[0] = c;
        }
      }
    };
    for (int j = 0; j < n_tiles; j += 2) {
      step(std::integral_constant<int, 0>{}, j, s_a, ce_a, s_b, ce_b);
      if (j + 1 < n_tiles) step(std::integral_constant<int, 1>{}, j + 1, s_b, ce_b, s_a, ce_a);
    }
  }
  wait_vm_lgkm0<0>();

  // Epilogue: O = O~ v_descale / (sum of P8 as rounded), rounded once to the
  // output dtype; lse = ln2 (m + log2 l - kP8Exp), l the fp32 sum of P8.
  const int row = wave_row0 + l32;
  const float l_tot = xor32_sum(l_run);
  if (row < S) {
    const float inv = v_mult / acc_l[0];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      store_o_block<DT>(o + head + (size_t)row * D + 32 * db, acc_o[db], inv, hi);
    if (hi == 0)
      lse[(size_t)bh * S + row] =
          (m_run + __builtin_amdgcn_logf(l_tot) - (float)kP8Exp) * kLn2;
  }
}

template <int D, int DT, bool CAUSAL>
hipError_t launch_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int S, float c, float v_mult, int n_cu, unsigned int* tk,
                      hipStream_t stream) {
  using SH = Fp8Shape<D>;
  const int n_qt = (S + SH::kBr - 1) / SH::kBr;
  const long long slots = (long long)n_cu * 2;  // two 4-wave workgroups per compute unit
  const long long n_wg = (long long)n_qt * H * B;
  const int pair_split =
      (CAUSAL && n_qt > 1 && n_wg <= slots) ? (int)(((n_qt + 1) / 2) * (long long)H * B) : 0;
  // tickets for the last quarter of multi-round grids (not at D = 256: the
  // unpipelined tile measured 0.4-1.6% slower with them)
  const int tk_from = (tk && !SH::kSerial && n_wg > slots) ? (int)(n_wg - n_wg / 4) : INT32_MAX;
  fa2_fwd_fp8_kernel<D, DT, CAUSAL><<<dim3((unsigned)n_qt, (unsigned)H, (unsigned)B),
                                      dim3(SH::kThreads), 0, stream>>>(
      (const unsigned char*)q, (const unsigned char*)k, (const unsigned char*)v, (uint16_t*)o, lse,
      S, c, v_mult, pair_split, tk_from, tk);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fp8_any(int dtype, int causal, const void* q, const void* k, const void* v,
                          void* o, float* lse, int B, int H, int S, float c, float v_mult,
                          int n_cu, unsigned int* tk, hipStream_t stream) {
  if (dtype == FA2_F16)
    return causal ? launch_fp8<D, FA2_F16, true>(q, k, v, o, lse, B, H, S, c, v_mult, n_cu, tk,
                                                 stream)
                  : launch_fp8<D, FA2_F16, false>(q, k, v, o, lse, B, H, S, c, v_mult, n_cu, tk,
                                                  stream);
  return causal ? launch_fp8<D, FA2_BF16, true>(q, k, v, o, lse, B, H, S, c, v_mult, n_cu, tk,
                                                stream)
                : launch_fp8<D, FA2_BF16, false>(q, k, v, o, lse, B, H, S, c, v_mult, n_cu, tk,
                                                 stream);
}

}  // namespace

extern "C" int fa2_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int S, int D, int causal, float scale, float q_descale,
                           float k_descale, float v_descale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (B < 1 || H < 1 || S < 1 || B > 65535 || H > 65535 || S > INT32_MAX - 1024)
    return FA2_ERR_SHAPE;
  if (dtype != FA2_F16 && dtype != FA2_BF16) return FA2_ERR_DTYPE;
  if (!(D == 64 || D == 128 || D == 256)) return FA2_ERR_HEADDIM;
  // the elements within int64 (a head may span any size: tiles are
  // addressed from 64-bit starts); the grid's linear block index in 32 bits
  if (!fa2_host::elements_fit_int64(B, H, S, D)) return FA2_ERR_SHAPE;
  if ((((long long)S + 127) / 128) * H * B > (long long)INT32_MAX) return FA2_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA2_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA2_ERR_ALIGN;
  if (!std::isfinite(scale)) return FA2_ERR_SCALE;
  for (float d : {q_descale, k_descale, v_descale})
    if (!std::isfinite(d) || !(d > 0.f)) return FA2_ERR_SCALE;
  const float c = scale * kLog2e * q_descale * k_descale;
  if (!std::isfinite(c)) return FA2_ERR_SCALE;
  const size_t n = (size_t)B * H * S * D;
  const size_t lse_bytes = (size_t)B * H * S * sizeof(float);
  if (fa2_host::overlaps(o, 2 * n, q, n) || fa2_host::overlaps(o, 2 * n, k, n) ||
      fa2_host::overlaps(o, 2 * n, v, n) || fa2_host::overlaps(lse, lse_bytes, q, n) ||
      fa2_host::overlaps(lse, lse_bytes, k, n) || fa2_host::overlaps(lse, lse_bytes, v, n) ||
      fa2_host::overlaps(lse, lse_bytes, o, 2 * n))
    return FA2_ERR_ALIAS;
  int n_cu = 0;
  const int dev = fa2_host::check_device(&n_cu);
  if (dev != FA2_OK) return dev;
  (void)hipGetLastError();
  unsigned int* const tk = ticket_counter((hipStream_t)stream);
  const hipError_t err =
      D == 64    ? launch_fp8_any<64>(dtype, causal, q, k, v, o, lse, B, H, S, c, v_descale, n_cu,
                                      tk, (hipStream_t)stream)
      : D == 128 ? launch_fp8_any<128>(dtype, causal, q, k, v, o, lse, B, H, S, c, v_descale,
                                       n_cu, tk, (hipStream_t)stream)
                 : launch_fp8_any<256>(dtype, causal, q, k, v, o, lse, B, H, S, c, v_descale,
                                       n_cu, tk, (hipStream_t)stream);
  return err == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}
