// FlashAttention-2 forward pass for MI355X (gfx950 / CDNA4).
//
// One workgroup owns a tile of B_r query rows of one (batch, head); the grid
// is (ceil(S / B_r), H, B), the sequence-parallel grid of FlashAttention-2
// (jared-hpc Lecture 6, "FA2 change 1"). Inside the workgroup every 64-lane
// wavefront owns 32 query rows outright and runs the whole key loop on them,
// so waves never exchange softmax state (infra.bea.ai FlashAttention V2 guide,
// "Optimization 3: Warp-Level Work Partitioning", split-Q). K and V tiles of
// B_c keys are staged in LDS once per workgroup and read by all its waves.
//
// Per key tile j the wave computes (infra.bea.ai guide, "Optimization 2:
// Delay Rescaling"; the cookbook notebook's Triton kernel loop):
//   S   = Q K_j^T                              (matrix cores, fp32 accumulate)
//   m'  = max(m, rowmax(c * S)),  c = scale * log2(e)
//   P   = 2^(c * S - m'),  alpha = 2^(m - m')
//   l   = alpha * l + rowsum(P)
//   O~  = alpha * O~ + P V_j                   (matrix cores, P rounded to the
//                                               input dtype, fp32 accumulate)
// and only the epilogue divides by l and writes lse = ln2 * (m + log2 l).
// Base-2 exponentials with scale*log2(e) folded into one FMA give the same
// values as exp(scale*S - m) since 2^(x log2 e) = e^x.
//
// Matrix-core formulation. The wave computes the transposed products
//   S^T = K_j Q^T   (A = K_j from LDS,  B = Q^T resident in registers)
//   O^T = V_j^T P^T (A = V_j^T from LDS, B = P^T straight from S^T's registers)
// with v_mfma_f32_32x32x16_{f16,bf16}. Output column n of a 32x32 block lives
// in lane n (mod 32), so each lane holds one query row: the row max and row
// sum need only in-lane reductions plus one exchange with the lane 32 away,
// and the per-row rescale by alpha is a per-lane scalar multiply.
//
// MFMA 32x32x16 lane layouts used below (lane l, l32 = l % 32, hi = l / 32):
//   A (32 x 16): lane l holds row l32, 8 consecutive k values of half hi.
//   B (16 x 32): lane l holds column l32, the same 8 k values.
//   C (32 x 32): register r of lane l holds row 8*(r/4) + 4*hi + r%4, column l32.
// Any bijection between (hi, element) and k is valid as long as A and B use
// the same one, which is how P^T is fed from the S^T accumulator registers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
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

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Element-type specific pieces: the matrix-core product and the RNE packing
// of two fp32 values into the input dtype.
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
};

// Tile shape per head dimension.
template <int D> struct Tile {
  static constexpr int kWaves = 4;             // waves per workgroup
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRowsPerWave = 32;      // query rows owned by one wave
  static constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
  static constexpr int kBc = 64;               // keys per tile
  static constexpr int kKPitch = D + 8;        // K tile row pitch in LDS (elements)
  static constexpr int kVPitch = kBc + 4;      // V^T tile row pitch in LDS (elements)
  // Waves per SIMD the register budget is sized for: two at D <= 128 (256
  // VGPRs each), one at D = 256 (O~ alone takes 128 registers per lane).
  static constexpr int kMinWavesPerSimd = D <= 128 ? 2 : 1;
};

// Value of x held by the lane 32 away, combined with x by max or by sum.
__device__ __forceinline__ float max_with_other_half(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  return x + __shfl_xor(x, 32);
}

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(Tile<D>::kThreads, Tile<D>::kMinWavesPerSimd) void fa2_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int S, float c /* scale * log2(e) */) {
  using T = Tile<D>;
  using E = Elem<DT>;
  constexpr int Bc = T::kBc, Br = T::kBr, KP = T::kKPitch, VP = T::kVPitch;
  constexpr int NKB = Bc / 32;  // 32-key blocks per tile
  constexpr int NDS = D / 16;   // k-steps of 16 over the head dim (S^T product)
  constexpr int NDB = D / 32;   // 32-wide head-dim blocks of O^T

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[Bc * KP];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroup -> (query tile, batch*head). Tiles are taken in descending
  // query-tile order across all heads, so under causal masking the longest
  // tiles start first; consecutive workgroups of one (b, h) are H*B apart in
  // launch order, which keeps them on one XCD when H*B is a multiple of 8.
  const int n_qt = gridDim.x;
  const int n_bh = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int bh = lin % n_bh;
  const int qt = n_qt - 1 - lin / n_bh;
  const int q0 = qt * Br;
  const size_t head = (size_t)bh * (size_t)S * D;

  const int wave_row0 = q0 + wave * T::kRowsPerWave;
  const int row = wave_row0 + l32;  // the query row this lane owns

  // Q^T operand: lane holds Q[row][16 s + 8 hi .. +7] for every k-step s.
  u32x4 qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    qf[s] = u32x4{0, 0, 0, 0};
    if (row < S) qf[s] = *(const u32x4*)(q + head + (size_t)row * D + 16 * s + 8 * hi);
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY;  // running max of c*S (base-2 units)
  float l_run = 0.f;        // this lane's share of the running sum

  const int kv_end = CAUSAL ? min(q0 + Br, S) : S;
  const int n_tiles = (kv_end + Bc - 1) / Bc;

  for (int j = 0; j < n_tiles; ++j) {
    const int key0 = j * Bc;
    __syncthreads();  // every wave is done reading the previous tile

    // K tile, row-major [key][d]; keys >= S are zero.
    constexpr int kChunks = Bc * D / 8;  // 16-byte chunks
#pragma unroll
    for (int ci = tid; ci < kChunks; ci += T::kThreads) {
      const int r = ci / (D / 8), c8 = ci % (D / 8);
      u32x4 val = {0, 0, 0, 0};
      if (key0 + r < S) val = *(const u32x4*)(k + head + (size_t)(key0 + r) * D + c8 * 8);
      *(u32x4*)(k_lds + r * KP + c8 * 8) = val;
    }
    // V tile, transposed to [d][key]: a thread loads 4 keys x 8 dims and
    // writes 8 rows of 4 keys.
    constexpr int kVGroups = (Bc / 4) * (D / 8);
#pragma unroll
    for (int g = tid; g < kVGroups; g += T::kThreads) {
      const int kq = g / (D / 8), dc = g % (D / 8);
      u32x4 x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 4 * kq + r;
        x[r] = u32x4{0, 0, 0, 0};
        if (key < S) x[r] = *(const u32x4*)(v + head + (size_t)key * D + dc * 8);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 even = {(x[0][w] & 0xffffu) | (x[1][w] << 16),
                            (x[2][w] & 0xffffu) | (x[3][w] << 16)};
        const u32x2 odd = {(x[0][w] >> 16) | (x[1][w] & 0xffff0000u),
                           (x[2][w] >> 16) | (x[3][w] & 0xffff0000u)};
        *(u32x2*)(vt_lds + (8 * dc + 2 * w) * VP + 4 * kq) = even;
        *(u32x2*)(vt_lds + (8 * dc + 2 * w + 1) * VP + 4 * kq) = odd;
      }
    }
    __syncthreads();

    // Under causal masking a wave whose rows all precede the tile's first key
    // has nothing to do for this tile (it still joins the barriers above).
    if (CAUSAL && key0 > wave_row0 + T::kRowsPerWave - 1) continue;

    // S^T = K_j Q^T: NKB blocks of 32 keys x 32 rows.
    f32x16 acc_s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      acc_s[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        const u32x4 a = *(const u32x4*)(k_lds + (32 * kb + l32) * KP + 16 * s + 8 * hi);
        acc_s[kb] = E::mfma(a, qf[s], acc_s[kb]);
      }
    }

    // Mask keys >= S (ragged tail) and, under causal masking, keys > row.
    // Masked tiles are scaled first and masked in the scaled (base-2)
    // domain, so a zero scale never meets a -inf score; c_eff is then 1.
    float c_eff = c;
    const bool need_mask =
        (key0 + Bc > S) || (CAUSAL && key0 + Bc - 1 > wave_row0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 8 * (r / 4) + 4 * hi + (r % 4);
          const bool masked = key >= S || (CAUSAL && key > row);
          acc_s[kb][r] = masked ? -INFINITY : acc_s[kb][r] * c;
        }
      c_eff = 1.f;
    }

    // Online softmax for this lane's row.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[kb][r]);
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(m_run, mx * c_eff);
    // A row with no unmasked key so far keeps m = -inf; use 0 as its
    // exponent reference so that no -inf - (-inf) is formed.
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;

    uint32_t pk[NKB][8];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(acc_s[kb][r], c_eff, -m_ref));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(acc_s[kb][r + 1], c_eff, -m_ref));
        l_run += p0 + p1;
        pk[kb][r / 2] = E::pack2(p0, p1);
      }

    // O^T += V_j^T P^T. B operand element e of step (kb, h) is accumulator
    // register 8h + e, i.e. key 32 kb + 16 h + 8 (e / 4) + 4 hi + e % 4;
    // the A operand gathers V^T at the same keys.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 b = {pk[kb][4 * h], pk[kb][4 * h + 1], pk[kb][4 * h + 2], pk[kb][4 * h + 3]};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* base = vt_lds + (32 * db + l32) * VP + 32 * kb + 16 * h + 4 * hi;
          const u32x2 a0 = *(const u32x2*)base;
          const u32x2 a1 = *(const u32x2*)(base + 8);
          const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
          acc_o[db] = E::mfma(a, b, acc_o[db]);
        }
      }
    m_run = m_new;
  }

  // Epilogue: O = O~ / l, rounded once to the input dtype; lse = ln2 (m + log2 l).
  const float l_tot = sum_with_other_half(l_run);
  if (row < S) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 out = {E::pack2(acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv),
                           E::pack2(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv)};
        *(u32x2*)(o + head + (size_t)row * D + 32 * db + 8 * g + 4 * hi) = out;
      }
    if (hi == 0) lse[(size_t)bh * S + row] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

template <int D, int DT, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int S, float scale, hipStream_t stream) {
  using T = Tile<D>;
  const dim3 grid((unsigned)((S + T::kBr - 1) / T::kBr), (unsigned)H, (unsigned)B);
  const dim3 block(T::kThreads);
  fa2_fwd_kernel<D, DT, CAUSAL><<<grid, block, 0, stream>>>(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, S,
      scale * kLog2e);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_causal(int causal, const void* q, const void* k, const void* v, void* o,
                         float* lse, int B, int H, int S, float scale, hipStream_t stream) {
  return causal ? launch<D, DT, true>(q, k, v, o, lse, B, H, S, scale, stream)
                : launch<D, DT, false>(q, k, v, o, lse, B, H, S, scale, stream);
}

template <int D>
hipError_t launch_dtype(int dtype, int causal, const void* q, const void* k, const void* v,
                        void* o, float* lse, int B, int H, int S, float scale,
                        hipStream_t stream) {
  return dtype == FA2_F16
             ? launch_causal<D, FA2_F16>(causal, q, k, v, o, lse, B, H, S, scale, stream)
             : launch_causal<D, FA2_BF16>(causal, q, k, v, o, lse, B, H, S, scale, stream);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Per-device verdict on whether the device is gfx950: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];

int check_device() {
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
    g_device_ok[dev].store(verdict, std::memory_order_release);
  }
  return verdict == 1 ? FA2_OK : FA2_ERR_NO_DEVICE;
}

}  // namespace

extern "C" int fa2_supported(int D, int dtype) {
  return (D == 64 || D == 128 || D == 256) && (dtype == FA2_F16 || dtype == FA2_BF16);
}

extern "C" int fa2_rows_per_workgroup(int D) {
  switch (D) {
    case 64: return Tile<64>::kBr;
    case 128: return Tile<128>::kBr;
    case 256: return Tile<256>::kBr;
    default: return 0;
  }
}

extern "C" const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL: return "a tensor pointer is NULL";
    case FA2_ERR_SHAPE: return "B, H and S must be >= 1, B and H <= 65535, and B*H*S*D must fit in int64";
    case FA2_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA2_ERR_DTYPE: return "dtype must be FA2_F16 or FA2_BF16";
    case FA2_ERR_ALIGN: return "q, k, v and o must be 16-byte aligned and lse 4-byte aligned";
    case FA2_ERR_SCALE: return "scale must be finite and >= 0";
    case FA2_ERR_NO_DEVICE: return "no current HIP device, or it is not a gfx950 (MI355X)";
    case FA2_ERR_LAUNCH: return "the HIP runtime reported an error at kernel launch";
    case FA2_ERR_ALIAS: return "o or lse overlaps q, k, v or each other";
    default: return "unknown fa2 status";
  }
}

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int S, int D, int causal, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (B < 1 || H < 1 || S < 1 || B > 65535 || H > 65535) return FA2_ERR_SHAPE;
  if (dtype != FA2_F16 && dtype != FA2_BF16) return FA2_ERR_DTYPE;
  if (!(D == 64 || D == 128 || D == 256)) return FA2_ERR_HEADDIM;
  // B, H <= 65535, S < 2^31, D <= 256: B*H*S*D < 2^71 can overflow int64.
  const unsigned __int128 elems = (unsigned __int128)B * H * S * D;
  if (elems > (unsigned __int128)(INT64_MAX / 2)) return FA2_ERR_SHAPE;
  // the kernel linearises its block index in a 32-bit int
  const unsigned long long blocks =
      (unsigned long long)(((long long)S + fa2_rows_per_workgroup(D) - 1) / fa2_rows_per_workgroup(D)) *
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
  const int dev = check_device();
  if (dev != FA2_OK) return dev;

  (void)hipGetLastError();  // start from a clean error state
  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  switch (D) {
    case 64: err = launch_dtype<64>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st); break;
    case 128: err = launch_dtype<128>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st); break;
    default: err = launch_dtype<256>(dtype, causal, q, k, v, o, lse, B, H, S, scale, st); break;
  }
  return err == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}
