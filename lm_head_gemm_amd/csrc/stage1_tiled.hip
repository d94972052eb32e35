// Stage 1 on the tiled weight layout: FlashSampling's fused kernel (arXiv
// 2603.15854, Section 3, "Stage 1 (Fused Kernel)") reading W from a one-time
// repacked copy laid out for CDNA4's matrix cores.
//
// Tiled layout (weights are static, so the LM head is repacked once):
//   W is cut into blocks of 16 vocab rows x 256 columns (8 KiB of bf16).
//   Block (m, c) covers rows 16m .. 16m+15 and columns 256c .. 256c+255.
//   Eight consecutive row blocks form a group, and a group is stored column
//   step by column step: block (m, c) sits at block index
//   ((m / 8) * nC + c) * 8 + m % 8   (nC = ceil(D / 256)).
//   Inside a block, step t (0..7) holds 64 pieces of 16 bytes; piece `lane`
//   = (r, q) = (lane % 16, lane / 16) is W[16m + r][256c + 32t + 8q .. +8],
//   exactly the A operand of v_mfma_f32_16x16x32_bf16 for K step t. Rows past
//   V (up to a whole group) and columns past D are zero.
// Consequences: a wave load of one step is 1 KiB contiguous and already in
// operand layout (no LDS transpose), and the waves of a workgroup, one row
// block each, read adjacent blocks, so at each column step the workgroup
// streams 32 or 64 KiB of contiguous memory: the access pattern HBM serves
// best (measured: 86% of peak, against 75% for 16-row interleaved reads).
//
// Four kernels read it:
//  * GEMV (B <= 2, when asked for: the MFMA kernel streams this layout
//    faster): each lane accumulates bf16 dot products of its row piece with
//    H (staged once in LDS; the four lanes of a row share nothing but the
//    reduction), then two butterfly steps finish each row's sum;
//  * MFMA (B up to 64): the A operand comes straight from the loads; H
//    chunks are staged in LDS and shared by the workgroup's waves, one row
//    block per wave; the tiles of a nearly empty last round run as 64-row
//    tiles whose two wave halves split the K loop;
//  * wide MFMA (B 65 .. 128, and above when D is not a multiple of 256): two
//    row blocks per wave and 128-column batch tiles, H staged in sub-chunks
//    and the B operands read one K step ahead;
//  * the wide tile in few registers (B > 128, D a multiple of 256): the B
//    operands through a short register ring, so that two workgroups share a
//    CU (128-column batch tiles) or one 256-column batch tile fits.
// (An opt-in 256 x 256 tile with both operands copied into LDS exists for
// measurement; it is never chosen by itself.)
// Row-major W whose D is a multiple of 256 is read by three more kernels:
// mfma_rows_kernel (B up to 64) and mfma_rows_wide_kernel (B up to 128), with
// 256-byte row runs per wave load moved to operand order through a
// wave-private LDS region, and above that the wide kernel in its ROWS form
// (four neighbouring lanes load 64 contiguous bytes of a row, a lane
// permutation puts the pieces in A-operand order).
// All end in the same register epilogue: l * (1/T) + Gumbel(Philox word),
// a running maximum per batch row, one candidate key per (row, vocab tile);
// optionally the tile's log-mass (grouped variant) and the logits (stored
// through LDS as whole row segments).
#include <atomic>
#include <type_traits>

#include "fs_common.h"

namespace fs {
namespace {

constexpr int kBK = 256;            // columns per block
constexpr int kKS = 8;              // K steps of 32 per block
constexpr int kBlock16 = kKS * 64;  // 16-byte pieces per block
// Padded H row in LDS (elements). The 32-byte pad makes the row stride an odd
// multiple of 32 bytes, which measured free of bank conflicts for the B
// operand reads (16 lanes of 16 rows per access); a 16-byte pad conflicts
// 2-way on gfx950.
constexpr int kLdsRow = kBK + 16;
constexpr int kGroup = 8;           // row blocks per group in the tiled layout
constexpr int64_t kMaxHLds = 159 * 1024;  // LDS bytes for staged H rows (the rest: reduction arrays)

// First 16-byte piece of block (m, c) of the tiled layout.
__device__ __forceinline__ int64_t block_piece(int m, int c, int nC) {
  return (((int64_t)(m / kGroup) * nC + c) * kGroup + (m % kGroup)) * kBlock16;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>) in order: a
// loop whose index is a compile-time constant in its body, whatever the body's
// size (register arrays indexed by it then stay in registers).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float dot8_bf16(const uint4& w, const uint4& h, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, h.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, h.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, h.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, h.w), acc, false);
  return acc;
}

// ---------------------------------------------------------------- pack
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W, int64_t ldw, int32_t V,
                                                   int32_t D, int32_t nC, int64_t n16,
                                                   uint4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const int lane = (int)(i & 63);
  const int t = (int)((i >> 6) & (kKS - 1));
  const int64_t blk = i / kBlock16;                 // ((g * nC) + c) * 8 + m % 8
  const int64_t g = blk / ((int64_t)kGroup * nC);
  const int rem = (int)(blk - g * kGroup * nC);
  const int c = rem / kGroup;
  const int m = (int)(g * kGroup) + rem % kGroup;
  const int row = 16 * m + (lane & 15);
  const int k = kBK * c + 32 * t + 8 * (lane >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < V && k < D) v = *reinterpret_cast<const uint4*>(W + (int64_t)row * ldw + k);
  out[i] = v;
}

// ---------------------------------------------------------------- GEMV
template <int BB, int NW, bool SAMPLE, bool STORE>
__global__ __launch_bounds__(64 * NW) void gemv_tiled_kernel(Stage1Args a) {
  static_assert(BB == 1 || BB == 2 || BB == 4, "batch tile");
  extern __shared__ uint4 lds_h[];          // [BB][D / 8] pieces of H
  __shared__ uint64_t red[NW][BB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int vt = blockIdx.x;
  const int b0 = blockIdx.y * BB;
  const int D = a.D;
  const int nC = (D + kBK - 1) / kBK;
  const int nM = (a.V + 15) / 16;
  const int d8 = D / 8;

  for (int i = tid; i < BB * d8; i += 64 * NW) {
    const int b = i / d8;
    const int c = i - b * d8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (b0 + b < a.B)
      v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.H) + (int64_t)(b0 + b) * a.ldh + 8 * c);
    lds_h[i] = v;
  }
  __syncthreads();

  const int m = vt * NW + wave;
  const bool has_rows = m < nM;
  const int mc = min(m, nM - 1);
  const uint4* wt = static_cast<const uint4*>(a.W) + lane;

  float acc[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) acc[b] = 0.f;

  // two blocks (16 KiB per wave) in flight per iteration
  for (int c0 = 0; c0 < nC; c0 += 2) {
    uint4 w[2][kKS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < kKS; ++t) {
        w[u][t] = make_uint4(0u, 0u, 0u, 0u);
        if (has_rows && c0 + u < nC) w[u][t] = load_stream16(wt + block_piece(mc, c0 + u, nC) + t * 64);
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u;
#pragma unroll
      for (int t = 0; t < kKS; ++t) {
        const int k8 = 32 * c + 4 * t + q;   // 16-byte piece of H this lane pairs with
        if (c < nC && 8 * k8 < D) {
#pragma unroll
          for (int b = 0; b < BB; ++b) acc[b] = dot8_bf16(w[u][t], lds_h[b * d8 + k8], acc[b]);
        }
      }
    }
  }

#pragma unroll
  for (int b = 0; b < BB; ++b) {
    acc[b] += __shfl_xor(acc[b], 16);
    acc[b] += __shfl_xor(acc[b], 32);
  }
  // lane (r, q) now handles row 16m + r of batch row b0 + q
  float l = acc[0];
#pragma unroll
  for (int b = 1; b < BB; ++b)
    if (q == b) l = acc[b];
  const int v = 16 * m + r;
  const int batch = b0 + q;
  const bool valid = has_rows && v < a.V && q < BB && batch < a.B;

  if constexpr (STORE) {
    if (valid) {
      const int64_t off = (int64_t)batch * a.ld_logits + v;
      if (a.logits_bf16) static_cast<uint16_t*>(a.logits)[off] = f32_to_bf16_rne(l);
      else static_cast<float*>(a.logits)[off] = l;
    }
  }
  if constexpr (SAMPLE) {
    float s = l;
    if (!a.greedy) {
      const uint4 words = philox_quad(a.nk, (uint32_t)(v >> 2), (uint32_t)batch);
      s = score2(l, a.score_scale, pick_word(words, r & 3));
    }
    uint64_t best = valid ? pack_key(s, (uint32_t)v) : 0ull;
#pragma unroll
    for (int mk = 1; mk < 16; mk <<= 1) best = umax64(best, shfl_xor_u64(best, mk));
    if (r == 0 && q < BB) red[wave][q] = best;
    __syncthreads();
    uint64_t k = 0ull;
    if (tid < BB) {
      k = red[0][tid];
#pragma unroll
      for (int w = 1; w < NW; ++w) k = umax64(k, red[w][tid]);
    }
    publish_candidates(a, vt, b0, min(BB, a.B - b0), k, tid, 64 * NW);
  }
}

// Tile log-mass (grouped variant). A lane holds N values x = l / T of one
// batch column (NaN marks an entry past V or a NaN logit, both skipped) and
// their maximum m; lane_mass adds sum e^(x - m). mass_reduce_store merges the
// four lanes of the column (q = 0..3) and the q = 0 lane leaves the pair in
// the workgroup's LDS slot; publish_mass merges the waves' pairs and writes
// ln(sum e^x) of the tile per batch row to mass[tile, b].
template <int N>
__device__ __forceinline__ void lane_mass(const float (&x)[N], float m, float& s) {
  constexpr float kLog2e = 1.4426950408889634f;
  s = 0.f;
  if (m == __builtin_inff()) {
    s = 1.f;
  } else if (m != -__builtin_inff()) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (x[i] == x[i]) s += __builtin_amdgcn_exp2f((x[i] - m) * kLog2e);
  }
}

__device__ __forceinline__ void mass_reduce_store(float2* slot, int col, int q, float m, float s) {
  lse_merge(m, s, __shfl_xor(m, 16), __shfl_xor(s, 16));
  lse_merge(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32));
  if (q == 0) slot[col] = make_float2(m, s);
}

template <int NW, int BN>
__device__ __forceinline__ void publish_mass(const Stage1Args& a, const float2 (&red_mass)[NW][BN], int tile,
                                             int b0, int n_rows, int tid) {
  if (tid < n_rows) {
    float m = -__builtin_inff(), s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) lse_merge(m, s, red_mass[w][tid].x, red_mass[w][tid].y);
    a.mass[(int64_t)tile * a.B + b0 + tid] = lse_value(m, s);
  }
}

// Logits store of the MFMA kernels, staged through LDS. In the accumulator
// layout lane (r, q) of wave w holds, per 16-column batch block, the logits of
// vocab rows v_base + 16w + 4q .. +3 for one batch column, so a direct store
// writes 8- or 16-byte pieces of 16 different logits rows per instruction.
// Here each pass moves NBC column blocks: the fragments go to a [16 NBC][16 NW]
// fp32 tile in LDS (row pitch 16 NW + 8 floats, an odd multiple of 32 bytes),
// then the workgroup writes whole row segments of 16 NW logits. The caller
// must have synchronised the workgroup before the first pass (T reuses the H
// buffers). Rows past B and vocab entries past V are not written.
template <int NW, int NBC>
__device__ __forceinline__ void store_logits_staged(const Stage1Args& a, float* T, int v_base, int b_base,
                                                    const f32x4 (&vals)[NBC], int tid) {
  constexpr int VW = 16 * NW;          // vocab rows of the tile
  constexpr int PITCH = VW + 8;
  constexpr int PER_ROW = VW / 4;      // float4 per staged row
  const int lane = tid & 63, wave = tid >> 6, r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int i = 0; i < NBC; ++i)
    *reinterpret_cast<f32x4*>(T + (16 * i + r) * PITCH + 16 * wave + 4 * q) = vals[i];
  __syncthreads();
  for (int p = tid; p < 16 * NBC * PER_ROW; p += 64 * NW) {
    const int row = p / PER_ROW, c4 = p - row * PER_ROW;
    const int b = b_base + row;
    if (b < a.B) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(T + row * PITCH + 4 * c4);
      const float l[4] = {x[0], x[1], x[2], x[3]};
      store_logits4(a, b, v_base + 4 * c4, a.V, l);
    }
  }
  __syncthreads();
}

// Column blocks whose sums wave half kh (0 or 1) of a 64-row tile finishes:
// the first half of the blocks for kh = 0, the rest for kh = 1.
template <int NB>
__device__ __forceinline__ bool half_owns(int nb, int kh) {
  return NB == 1 ? kh == 0 : (nb < NB / 2) == (kh == 0);
}

// Epilogue of the kernels in which each wave owns one 16-row block of a
// 16 NW-row vocab tile and the workgroup one 16 NB-column batch tile: the
// optional logits store (staged through `stage`, STAGE_BYTES of LDS the
// main loop no longer needs), then per batch row the tile's maximiser as one
// key (and the tile's log-mass with MASS), published for Stage 2 or the
// single-pass reduction. With HALF the tile is a 64-row one (tile index vt,
// first row block rb0): waves w and w + 4 hold row block rb0 + w mod 4, and
// wave half kh scores only the column blocks half_owns gives it.
template <int NB, int NW, bool SAMPLE, bool STORE, bool MASS, int STAGE_BYTES, bool HALF = false>
__device__ __forceinline__ void narrow_epilogue(const Stage1Args& a, const f32x4 (&acc)[NB], int vt, int b0,
                                                float* stage, uint64_t (&red)[NW][16 * NB],
                                                float2 (&red_mass)[MASS ? NW : 1][MASS ? 16 * NB : 1],
                                                int rb0 = 0, int kh = 0) {
  static_assert(!HALF || (NW == 8 && SAMPLE && !STORE && !MASS), "64-row tiles only sample");
  constexpr int BN = 16 * NB;
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int m = HALF ? rb0 + (wave & 3) : vt * NW + wave;
  const int v0 = 16 * m + 4 * q;   // this lane's four consecutive vocab rows
  if constexpr (STORE) {
    constexpr int NBC = NB < 2 ? NB : 2;   // 16-column blocks per staging pass
    static_assert(16 * NBC * (16 * NW + 8) * 4 <= STAGE_BYTES, "staging tile fits the caller's LDS");
    __syncthreads();                        // every wave is done with the main loop's LDS
    float* T = stage;
#pragma unroll
    for (int p = 0; p < NB / NBC; ++p) {
      f32x4 vals[NBC];
#pragma unroll
      for (int i = 0; i < NBC; ++i) vals[i] = acc[p * NBC + i];
      store_logits_staged<NW, NBC>(a, T, vt * NW * 16, b0 + p * NBC * 16, vals, tid);
    }
  }
  if constexpr (SAMPLE) {
    // As in the wide kernel: running maximum over the lane's four rows in
    // vocab order, bound check on v only in the last vocab tile, no noise
    // when greedy; columns past B are dropped by publish_candidates.
    auto tile_max = [&](auto greedy_c, auto full_c) {
      constexpr bool kGreedy = decltype(greedy_c)::value;
      constexpr bool kFull = decltype(full_c)::value;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (HALF && !half_owns<NB>(nb, kh)) {
          if (q == 0) red[wave][nb * 16 + r] = 0ull;   // the other wave half's
          continue;
        }
        const int b = b0 + nb * 16 + r;
        uint4 words = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (!kGreedy) words = philox_quad(a.nk, (uint32_t)(v0 >> 2), (uint32_t)b);
        RunMax best = runmax_init();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float l = acc[nb][j];
          const float s = kGreedy ? l : score2(l, a.score_scale, pick_word(words, j));
          if (kFull || v0 + j < a.V) runmax_take(best, s, v0 + j);
        }
        uint64_t key = runmax_key(best);
        key = umax64(key, shfl_xor_u64(key, 16));
        key = umax64(key, shfl_xor_u64(key, 32));
        if (q == 0) red[wave][nb * 16 + r] = key;
        if constexpr (MASS && !kGreedy) {
          float x[4], mx = -__builtin_inff(), sm = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[j] = (kFull || v0 + j < a.V) ? acc[nb][j] * a.inv_t : __builtin_nanf("");
            mx = fmaxf(mx, x[j]);   // NaN entries are skipped
          }
          lane_mass(x, mx, sm);
          mass_reduce_store(red_mass[wave], nb * 16 + r, q, mx, sm);
        }
      }
    };
    const bool full = HALF ? (int64_t)(rb0 + 4) * 16 <= a.V : (int64_t)(vt + 1) * NW * 16 <= a.V;
    if (a.greedy) {
      if (full) tile_max(std::true_type{}, std::true_type{});
      else tile_max(std::true_type{}, std::false_type{});
    } else {
      if (full) tile_max(std::false_type{}, std::true_type{});
      else tile_max(std::false_type{}, std::false_type{});
    }
    __syncthreads();
    uint64_t k = 0ull;
    if (tid < BN) {
      k = red[0][tid];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) k = umax64(k, red[w2][tid]);
    }
    if constexpr (MASS) publish_mass<NW>(a, red_mass, vt, b0, min(BN, a.B - b0), tid);
    publish_candidates(a, vt, b0, min(BN, a.B - b0), k, tid, NT);
  }
}

// ---------------------------------------------------------------- MFMA
// Each lane takes the 16 bytes held by lane addr / 4 (ds_bpermute per dword).
__device__ __forceinline__ uint4 lane_gather(const uint4& v, int addr) {
  return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.x),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.y),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.z),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.w));
}

template <int NB>
__device__ __forceinline__ void tiled_half_tile(const Stage1Args& a, int vt, int rb0, uint4* lds_h4,
                                                uint64_t (&red)[8][16 * NB], float2 (&red_mass)[1][1]);

// With HALF (sampling, one batch tile of 32 or 64 columns), the last
// a.half_tiles vocab tiles hold 64 rows each (tiled_half_tile); the others
// are the kernel's own. That variant is held to 128 registers (four waves per
// SIMD, two workgroups per CU), the occupancy of the variant without.
template <int NB, int NW, bool SAMPLE, bool STORE, bool MASS = false, bool HALF = false>
__global__ __launch_bounds__(64 * NW, HALF ? 4 : 1) void mfma_tiled_kernel(Stage1Args a,
                                                                                             int32_t n_bt) {
  constexpr int BN = 16 * NB;
  constexpr int NT = 64 * NW;
  constexpr int HP = BN * (kBK / 8) / NT;   // 16-byte pieces of H per thread per block
  static_assert(HP >= 1 && HP * NT == BN * (kBK / 8), "batch tile vs workgroup size");

  __shared__ uint4 lds_h4[2 * BN * kLdsRow / 8];
  __shared__ uint64_t red[NW][BN];
  __shared__ float2 red_mass[MASS ? NW : 1][MASS ? BN : 1];
  uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_h4);

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup
  if constexpr (HALF) {
    static_assert(NW == 8 && NB >= 2 && SAMPLE && !STORE && !MASS, "64-row tiles: sampling, 32-64 columns");
    const int whole = a.n_tiles - a.half_tiles;
    if (vt >= whole) {
      tiled_half_tile<NB>(a, vt, 8 * whole + 4 * (vt - whole), lds_h4, red, red_mass);
      return;
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b0 = bt * BN;
  const int D = a.D;
  const int nC = (D + kBK - 1) / kBK;
  const int nM = (a.V + 15) / 16;
  const int m = vt * NW + wave;
  const int mc = min(m, nM - 1);
  // first 16-byte piece of this lane in K block c; K step t is 64 pieces further
  constexpr int kTStride = 64;
  const uint4* wt = static_cast<const uint4*>(a.W) + lane;
  auto wblock = [&](int c) { return wt + block_piece(mc, c, nC); };
  auto wload = [&](const uint4* p) { return load_stream16(p); };   // read once: non-temporal
  const uint16_t* H = static_cast<const uint16_t*>(a.H);

  // This thread's share of each H block: rows hn[i], columns hk[i] .. +8;
  // pieces past B or D are zero. (Predicated loads measured faster here than
  // clamped-address loads followed by a select.)
  int hn[HP], hk[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = tid + NT * i;
    hn[i] = p / (kBK / 8);
    hk[i] = 8 * (p % (kBK / 8));
  }
  auto load_h = [&](int c, uint4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const int k = c * kBK + hk[i];
      h[i] = make_uint4(0u, 0u, 0u, 0u);
      if (b0 + hn[i] < a.B && k < D) h[i] = *reinterpret_cast<const uint4*>(H + (int64_t)(b0 + hn[i]) * a.ldh + k);
    }
  };
  auto store_h = [&](int buf, const uint4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i)
      *reinterpret_cast<uint4*>(lds_h + buf * BN * kLdsRow + hn[i] * kLdsRow + hk[i]) = h[i];
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Rolling prefetch: the register holding K step t of block c is reloaded
  // with step t of block c+1 as soon as its MFMAs have been issued, so one
  // block (8 KiB per wave) stays in flight with a single register set; W
  // loads are unconditional (clamped row block) so the compiler can count
  // them. H for block c+1 is loaded during block c and written to the other
  // LDS buffer before the workgroup barrier.
  uint4 w[kKS];
  uint4 hreg[HP];
  {
    const uint4* p = wblock(0);
#pragma unroll
    for (int t = 0; t < kKS; ++t) w[t] = wload(p + t * kTStride);
  }
  load_h(0, hreg);
  store_h(0, hreg);
  __syncthreads();

  // Block c's math; with `more`, block c+1's loads are issued on the way.
  // The last block is peeled off so no load is ever issued for nothing.
  constexpr bool kPinLoads = NB == 2;
  auto step = [&](int c, bool more) {
    if (more) load_h(c + 1, hreg);
    const uint4* p = wblock(more ? c + 1 : c);
    const uint16_t* hb = lds_h + (c & 1) * BN * kLdsRow;
#pragma unroll
    for (int t = 0; t < kKS; ++t) {
      const uint4 x = w[t];
      // With two column blocks the reload goes after the step's matrix
      // instructions and stays there (no matrix instruction or memory load
      // crosses the scheduling barrier), so the new value can take the old
      // one's registers; left free, the compiler issues the block's loads
      // late into other registers and waits for all of them at the loop's
      // back edge. Measured 1-4 us faster at B = 17-32 on four heads, equal
      // or up to 1 us slower with one or four column blocks.
      if (!kPinLoads && more) w[t] = wload(p + t * kTStride);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 bfrag = *reinterpret_cast<const uint4*>(hb + (nb * 16 + r) * kLdsRow + 32 * t + 8 * q);
        acc[nb] = mfma16x16x32(x, bfrag, acc[nb]);
      }
      if (kPinLoads && more) {
        __builtin_amdgcn_sched_barrier(0x786);   // ALU and LDS instructions may cross
        w[t] = wload(p + t * kTStride);
      }
    }
    if (more) {
      store_h((c + 1) & 1, hreg);
      __syncthreads();
    }
  };
  for (int c = 0; c + 1 < nC; ++c) step(c, true);
  step(nC - 1, false);

  narrow_epilogue<NB, NW, SAMPLE, STORE, MASS, (int)sizeof(lds_h4)>(a, acc, vt, b0, reinterpret_cast<float*>(lds_h4),
                                                                     red, red_mass);
}

// A 64-row vocab tile of the sampling kernel (tile index vt, row blocks
// rb0 .. rb0 + 3, one batch tile of 16 NB columns, NB = 2 or 4), for the
// tiles of a last round of workgroups that would leave most of the chip idle.
// Waves w and w + 4 hold row block rb0 + w mod 4 and split each K block
// between them (K steps 0-3 and 4-7): the workgroup does half of a 128-row
// tile's matrix work and reads half of its W, none of it twice. H is staged
// as in the 128-row tile. The two partial sums of a row block meet in LDS,
// each wave half finishing half of the column blocks; a logit is the sum of
// its two halves, within fp32 rounding of the 128-row tile's.
template <int NB>
__device__ __forceinline__ void tiled_half_tile(const Stage1Args& a, int vt, int rb0, uint4* lds_h4,
                                                uint64_t (&red)[8][16 * NB], float2 (&red_mass)[1][1]) {
  constexpr int NW = 8;
  constexpr int BN = 16 * NB;
  constexpr int NT = 64 * NW;
  constexpr int HP = BN * (kBK / 8) / NT;
  constexpr int KH = kKS / 2;        // K steps of a block per wave half
  constexpr int kTStride = 64;
  static_assert(4 * NB * 64 * 16 <= 2 * BN * kLdsRow * 2, "partial sums fit the H buffers");
  uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_h4);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int kh = wave >> 2;
  const int D = a.D;
  const int nC = (D + kBK - 1) / kBK;
  const int nM = (a.V + 15) / 16;
  const int mc = min(rb0 + (wave & 3), nM - 1);
  const uint4* wt = static_cast<const uint4*>(a.W) + lane + KH * kh * kTStride;
  auto wblock = [&](int c) { return wt + block_piece(mc, c, nC); };
  const uint16_t* H = static_cast<const uint16_t*>(a.H);

  int hn[HP], hk[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = tid + NT * i;
    hn[i] = p / (kBK / 8);
    hk[i] = 8 * (p % (kBK / 8));
  }
  auto load_h = [&](int c, uint4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const int k = c * kBK + hk[i];
      h[i] = make_uint4(0u, 0u, 0u, 0u);
      if (hn[i] < a.B && k < D) h[i] = *reinterpret_cast<const uint4*>(H + (int64_t)hn[i] * a.ldh + k);
    }
  };
  auto store_h = [&](int buf, const uint4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i)
      *reinterpret_cast<uint4*>(lds_h + buf * BN * kLdsRow + hn[i] * kLdsRow + hk[i]) = h[i];
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // W two K blocks ahead (register set c mod 2 holds block c, reloaded with
  // block c + 2 as its matrix instructions issue), so that up to 8 KiB per
  // wave are in flight as in the 128-row tile, in as many registers.
  constexpr int KD = 2;
  uint4 w[KD][KH];
  uint4 hreg[HP];
#pragma unroll
  for (int s = 0; s < KD; ++s) {
    const uint4* p = wblock(s < nC ? s : 0);
#pragma unroll
    for (int t = 0; t < KH; ++t)
      if (s < nC) w[s][t] = load_stream16(p + t * kTStride);
  }
  load_h(0, hreg);
  store_h(0, hreg);
  __syncthreads();
  // Block c's math from register set S; with MORE, block c+1's H is staged on
  // the way, with AHEAD block c+KD's W is loaded. Both are compile-time in
  // every call, so the compiler can count the loads in flight (a load under
  // a run-time condition makes it wait for all of them at each barrier).
  auto step = [&](int c, auto set_c, auto more_c, auto ahead_c) {
    constexpr int S = decltype(set_c)::value;
    constexpr bool kMore = decltype(more_c)::value;
    constexpr bool kAhead = decltype(ahead_c)::value;
    if (kMore) load_h(c + 1, hreg);
    const uint4* p = wblock(kAhead ? c + KD : c);
    const uint16_t* hb = lds_h + (c & 1) * BN * kLdsRow + 32 * KH * kh + 8 * q;
#pragma unroll
    for (int t = 0; t < KH; ++t) {
      const uint4 x = w[S][t];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 bfrag = *reinterpret_cast<const uint4*>(hb + (nb * 16 + r) * kLdsRow + 32 * t);
        acc[nb] = mfma16x16x32(x, bfrag, acc[nb]);
      }
      // the reload stays behind its register's matrix instructions (only ALU
      // and LDS instructions cross), so it can take the same registers
      // instead of being copied into them at the loop's back edge
      if (kAhead) {
        __builtin_amdgcn_sched_barrier(0x786);
        w[S][t] = load_stream16(p + t * kTStride);
      }
    }
    if (kMore) {
      store_h((c + 1) & 1, hreg);
      __syncthreads();
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using Y = std::true_type;
  using N = std::false_type;
  int c = 0;
  for (; c + 3 < nC; c += 2) {
    step(c, S0{}, Y{}, Y{});
    step(c + 1, S1{}, Y{}, Y{});
  }
  // the last one to three blocks
  if (c + 2 < nC) {
    step(c, S0{}, Y{}, Y{});
    step(c + 1, S1{}, Y{}, N{});
    step(c + 2, S0{}, N{}, N{});
  } else if (c + 1 < nC) {
    step(c, S0{}, Y{}, N{});
    step(c + 1, S1{}, N{}, N{});
  } else {
    step(c, S0{}, N{}, N{});
  }

  // each wave hands the column blocks it does not finish to its partner
  __syncthreads();   // every wave is done with H
  f32x4* X = reinterpret_cast<f32x4*>(lds_h4);   // [row block][column block][lane]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    if (!half_owns<NB>(nb, kh)) X[((wave & 3) * NB + nb) * 64 + lane] = acc[nb];
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    if (half_owns<NB>(nb, kh)) acc[nb] += X[((wave & 3) * NB + nb) * 64 + lane];
  narrow_epilogue<NB, NW, true, false, false, 0, true>(a, acc, vt, 0, nullptr, red, red_mass, rb0, kh);
}

// ------------------------------------------------------- MFMA, row-major W
// Row-major bf16 W [V, D] (stride ldw, D a multiple of 128), B up to 64: the
// same tile as mfma_tiled_kernel (wave w owns row block vt * NW + w, the
// workgroup one 16 NB-column batch tile), fed from row-major memory.
//  * W is read in K blocks of 128 columns: per block and wave, four 16-byte
//    non-temporal wave loads, load j covering rows 4j .. 4j+3 of the wave's
//    block with 16 lanes (256 contiguous bytes) per row. Runs of 256 bytes
//    per row stream from HBM about as fast as the tiled layout's (measured:
//    6.8-6.95 TB/s against 5.8-6.3 for 64-byte runs of 16 rows).
//  * Each wave moves its block through a private 4 KiB LDS region (16 rows x
//    16 pieces of 16 bytes, piece p of row rho stored at p ^ rho, which keeps
//    both the row writes and the operand reads free of bank conflicts) into
//    the A-operand order: K step s of the block is pieces 4s .. 4s+3.
//  * Two K blocks of W (8 KiB per wave) are in flight: block i + 2 is loaded
//    into the registers of block i as soon as those are in LDS.
//  * H is staged in LDS by the workgroup, 128 columns per block, double
//    buffered, one barrier per block.
//  * Workgroup vt starts its K loop at block vt mod (D / 128), so the
//    workgroups in flight read different offsets of their rows: with the
//    power-of-two row strides of 4096- and 8192-wide heads, rows read at one
//    offset concentrate on a few memory channels (measured: 6.2 TB/s without
//    the rotation, 6.8-6.9 with it). The accumulation order of a row's
//    logits depends on its tile, within fp32 rounding.
constexpr int kRowsBK = 128;               // columns per K block

template <int NB, int NW, bool SAMPLE, bool STORE, bool MASS>
__global__ __launch_bounds__(64 * NW, NW / 2) void mfma_rows_kernel(Stage1Args a, int32_t n_bt) {
  constexpr int BN = 16 * NB;
  constexpr int NT = 64 * NW;
  // W K blocks per H block: two (256 columns, one barrier per two W blocks)
  // where the LDS holds it beside the W regions at two workgroups per CU
  // (batch tiles up to 32), else one
  constexpr int HB = NB <= 2 ? 2 : 1;
  constexpr int HROW = HB * kRowsBK + 16;              // padded H row (elements): an odd multiple of 32 bytes
  constexpr int HPIECES = BN * HB * (kRowsBK / 8);     // 16-byte pieces of H per H block
  constexpr int HP = (HPIECES + NT - 1) / NT;          // per thread
  static_assert((HROW * 2 / 32) % 2 == 1, "H row stride an odd multiple of 32 bytes");

  __shared__ uint4 lds_w[NW * 16 * 16];                // per wave: 16 rows x 16 pieces
  __shared__ uint4 lds_h4[2 * BN * HROW / 8];
  __shared__ uint64_t red[NW][BN];
  __shared__ float2 red_mass[MASS ? NW : 1][MASS ? BN : 1];
  uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_h4);

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b0 = bt * BN;
  const int nM = (a.V + 15) / 16;
  const int mc = min(vt * NW + wave, nM - 1);
  const int nblk = a.D / kRowsBK;
  const int s0 = vt % nblk;
  auto blk = [&](int i) {   // i-th K block of this workgroup's rotated order (i < 2 nblk)
    const int c = s0 + i;
    return c >= nblk ? c - nblk : c;
  };

  // load j of a block: row 4j + q of the wave's block (clamped past V),
  // columns 8r .. 8r+7 of the block
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  const uint16_t* wsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wsrc[j] = W + (int64_t)min(16 * mc + 4 * j + q, a.V - 1) * a.ldw + 8 * r;
  auto wload = [&](int c, int j) { return load_stream16(wsrc[j] + c * kRowsBK); };
  uint4* region = lds_w + wave * 256;
  const uint16_t* H = static_cast<const uint16_t*>(a.H);

  // H block h holds the H columns of W blocks HB h .. HB h + HB - 1 side by
  // side; this thread's pieces: row hn, W block HB h + hh, columns hk .. +8
  int hn[HP], hh[HP], hk[HP];
  bool hv[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = tid + NT * i;
    hv[i] = p < HPIECES;
    hn[i] = p / (HB * kRowsBK / 8);
    const int k8 = p % (HB * kRowsBK / 8);
    hh[i] = k8 / (kRowsBK / 8);
    hk[i] = 8 * (k8 % (kRowsBK / 8));
  }
  uint4 hreg[HP];
  auto load_h = [&](int h) {
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const int wb = HB * h + hh[i];
      hreg[i] = make_uint4(0u, 0u, 0u, 0u);
      if (hv[i] && b0 + hn[i] < a.B && wb < nblk)
        hreg[i] = *reinterpret_cast<const uint4*>(H + (int64_t)(b0 + hn[i]) * a.ldh + blk(wb) * kRowsBK + hk[i]);
    }
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int i = 0; i < HP; ++i)
      if (hv[i])
        *reinterpret_cast<uint4*>(lds_h + buf * BN * HROW + hn[i] * HROW + hh[i] * kRowsBK + hk[i]) = hreg[i];
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // H of the first H block first, so its wait does not also wait for W;
  // then W blocks 0 and 1 (past the last block: the last one again, unused)
  uint4 w[2][4];
  load_h(0);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = blk(min(k, nblk - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) w[k][j] = wload(c, j);
  }
  store_h(0);
  __syncthreads();

  // W block i (register slot i & 1, position i % HB in its H block): into
  // the wave's LDS region, the slot refilled with block i + 2 (REFILL); at
  // the first block of an H block the next H block's loads are issued
  // (HLOAD), after the last its pieces go to the other H buffer and the
  // workgroup synchronises (HSTORE); four K steps of matrix instructions.
  auto step = [&](int i, auto slot_c, auto refill_c, auto hload_c, auto hstore_c) {
    constexpr int S = decltype(slot_c)::value;
    if constexpr (decltype(hload_c)::value) load_h(i / HB + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) region[(4 * j + q) * 16 + (r ^ (4 * j + q))] = w[S][j];
    if constexpr (decltype(refill_c)::value) {
      const int c2 = blk(i + 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) w[S][j] = wload(c2, j);
    }
    __builtin_amdgcn_wave_barrier();   // the region's writes before this wave's reads
    const uint16_t* hb = lds_h + ((i / HB) & 1) * BN * HROW + (HB == 2 ? S : 0) * kRowsBK;
#pragma unroll
    for (int t = 0; t < kRowsBK / 32; ++t) {
      const uint4 x = region[r * 16 + ((4 * t + q) ^ r)];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 bfrag = *reinterpret_cast<const uint4*>(hb + (nb * 16 + r) * HROW + 32 * t + 8 * q);
        acc[nb] = mfma16x16x32(x, bfrag, acc[nb]);
      }
    }
    __builtin_amdgcn_wave_barrier();   // this wave's reads before the next block's writes
    if constexpr (decltype(hstore_c)::value) {
      store_h((i / HB + 1) & 1);
      __syncthreads();
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  // Pairs of W blocks (i even); while blocks i .. i+3 exist every refill and
  // H block is there. The last 1 to 3 blocks: refills only while a block is
  // left to load, H loads only while an H block is left.
  int i = 0;
  for (; i + 3 < nblk; i += 2) {
    if constexpr (HB == 2) {
      step(i, I0{}, T{}, T{}, F{});
      step(i + 1, I1{}, T{}, F{}, T{});
    } else {
      step(i, I0{}, T{}, T{}, T{});
      step(i + 1, I1{}, T{}, T{}, T{});
    }
  }
  const int left = nblk - i;
  if constexpr (HB == 2) {
    if (left == 3) {
      step(i, I0{}, T{}, T{}, F{});
      step(i + 1, I1{}, F{}, F{}, T{});
      step(i + 2, I0{}, F{}, F{}, F{});
    } else if (left == 2) {
      step(i, I0{}, F{}, F{}, F{});
      step(i + 1, I1{}, F{}, F{}, F{});
    } else {
      step(i, I0{}, F{}, F{}, F{});
    }
  } else {
    if (left == 3) {
      step(i, I0{}, T{}, T{}, T{});
      step(i + 1, I1{}, F{}, T{}, T{});
      step(i + 2, I0{}, F{}, F{}, F{});
    } else if (left == 2) {
      step(i, I0{}, F{}, T{}, T{});
      step(i + 1, I1{}, F{}, F{}, F{});
    } else {
      step(i, I0{}, F{}, F{}, F{});
    }
  }

  narrow_epilogue<NB, NW, SAMPLE, STORE, MASS, (int)sizeof(lds_h4)>(a, acc, vt, b0, reinterpret_cast<float*>(lds_h4),
                                                                     red, red_mass);
}

// ------------------------------------------------------- MFMA, wide tiles
// Large batches (B > 64) make the contraction heavy enough that the vocab
// tile has to grow so that each byte of H staged in LDS feeds more matrix
// work: each of the 8 waves owns two row blocks (blocks vt*16 + w and
// vt*16 + 8 + w, i.e. one full group of the layout per half), giving a vocab
// tile of 256 rows and a batch tile of 128 columns.
//  * W: rolling prefetch kWidePD K steps ahead (4 registers of 16 bytes per
//    block), ordinary cached loads, because the batch tiles of one vocab tile
//    run back to back on one XCD (tile_of) and re-read it from L2; with one
//    or two batch tiles (B <= 256, STREAMW) non-temporal loads instead
//    (measured on the 4096 x 128256 head: 10% faster at B = 65 .. 128,
//    equal at 256, 1% slower at 1024).
//  * H: staged in sub-chunks of 64 columns, double-buffered in LDS with one
//    barrier per sub-chunk; each wave reads its B operands one K step ahead
//    into a second register set, and the reads for the next sub-chunk are
//    issued right after its barrier, before the last K step's MFMAs.
// Measured on the 4096 x 128256 head: 1.4-1.8x faster than the 128-row tile
// at B = 128 .. 1024.
constexpr int kWideNB = 8;                     // 16-column batch blocks: BN = 128
constexpr int kWideNW = 8;                     // waves
constexpr int kWideMB = 2;                     // row blocks per wave
constexpr int kWideKSub = 2;                   // K steps per H sub-chunk
constexpr int kWidePD = 4;                     // W prefetch distance in K steps
constexpr int kWideBN = 16 * kWideNB;
constexpr int kWideRows = 16 * kWideNW * kWideMB;

// Epilogue of the wide tile (wave w owns row blocks m[j] = vt * NW * MB + j * NW
// + w, j < MB, of a 16 NW MB-row vocab tile; the workgroup one 16 NB-column batch
// tile): the optional logits store staged through `stage` (STAGE_BYTES of LDS
// the main loop no longer needs), then per batch row the tile's maximiser as
// one key (and the tile's log-mass with MASS), published for Stage 2 or the
// single-pass reduction.
template <int NW, int MB, int NB, bool SAMPLE, bool STORE, bool MASS, int STAGE_BYTES>
__device__ __forceinline__ void wide_epilogue(const Stage1Args& a, const f32x4 (&acc)[MB][NB], const int (&m)[MB],
                                              int vt, int b0, float* stage, uint64_t (&red)[NW][16 * NB],
                                              float2 (&red_mass)[MASS ? NW : 1][MASS ? 16 * NB : 1]) {
  constexpr int BN = 16 * NB, NT = 64 * NW;
  static_assert(NT >= BN, "one thread per batch column for the workgroup reduction");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  if constexpr (STORE) {
    constexpr int NBC = 2;                  // 16-column blocks per staging pass
    static_assert(16 * NBC * (16 * NW + 8) * 4 <= STAGE_BYTES, "staging tile fits the caller's LDS");
    __syncthreads();                        // every wave is done with the main loop's LDS
    float* T = stage;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
#pragma unroll
      for (int p = 0; p < NB / NBC; ++p) {
        f32x4 vals[NBC];
#pragma unroll
        for (int i = 0; i < NBC; ++i) vals[i] = acc[j][p * NBC + i];
        store_logits_staged<NW, NBC>(a, T, 16 * (vt * NW * MB + j * NW), b0 + p * NBC * 16, vals, tid);
      }
    }
  }
  if constexpr (SAMPLE) {
    // Per batch column: the lane's 4 x MB candidates come in increasing
    // vocab order (a running maximum suffices), then the four lanes of the
    // column combine their keys. Batch columns past B are computed on zero
    // rows and dropped by publish_candidates. Only the last vocab tile needs
    // the bound check on v; greedy (T = 0) skips the noise entirely.
    auto tile_max = [&](auto greedy_c, auto full_c) {
      constexpr bool kGreedy = decltype(greedy_c)::value;
      constexpr bool kFull = decltype(full_c)::value;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int b = b0 + nb * 16 + r;
        RunMax best = runmax_init();
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          const int v0 = 16 * m[j] + 4 * q;   // this lane's four consecutive vocab rows
          uint4 words = make_uint4(0u, 0u, 0u, 0u);
          if constexpr (!kGreedy) words = philox_quad(a.nk, (uint32_t)(v0 >> 2), (uint32_t)b);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float l = acc[j][nb][e];
            const float sc = kGreedy ? l : score2(l, a.score_scale, pick_word(words, e));
            if (kFull || v0 + e < a.V) runmax_take(best, sc, v0 + e);
          }
        }
        uint64_t key = runmax_key(best);
        key = umax64(key, shfl_xor_u64(key, 16));
        key = umax64(key, shfl_xor_u64(key, 32));
        if (q == 0) red[wave][nb * 16 + r] = key;
        if constexpr (MASS && !kGreedy) {
          float x[4 * MB], mx = -__builtin_inff(), sm = 0.f;
#pragma unroll
          for (int j = 0; j < MB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 16 * m[j] + 4 * q + e;
              x[4 * j + e] = (kFull || v < a.V) ? acc[j][nb][e] * a.inv_t : __builtin_nanf("");
              mx = fmaxf(mx, x[4 * j + e]);   // NaN entries are skipped
            }
          lane_mass(x, mx, sm);
          mass_reduce_store(red_mass[wave], nb * 16 + r, q, mx, sm);
        }
      }
    };
    const bool full = (int64_t)(vt + 1) * (16 * NW * MB) <= a.V;
    if (a.greedy) {
      if (full) tile_max(std::true_type{}, std::true_type{});
      else tile_max(std::true_type{}, std::false_type{});
    } else {
      if (full) tile_max(std::false_type{}, std::true_type{});
      else tile_max(std::false_type{}, std::false_type{});
    }
    __syncthreads();
    uint64_t k = 0ull;
    if (tid < BN) {
      k = red[0][tid];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) k = umax64(k, red[w2][tid]);
    }
    if constexpr (MASS) publish_mass<NW>(a, red_mass, vt, b0, min(BN, a.B - b0), tid);
    publish_candidates(a, vt, b0, min(BN, a.B - b0), k, tid, NT);
  }
}

// ROWS: row-major W [V, D] (D a multiple of 256) read directly, as in the
// 16-rows-per-wave kernel: lane 4i + j of row block m loads
// W[16m + i][256c + 32t + 8j .. +8] (rows past V clamped), and the lane
// permutation moves it to lane i + 16j.
template <bool SAMPLE, bool STORE, bool MASS = false, bool ROWS = false, bool STREAMW = false>
__global__ __launch_bounds__(64 * kWideNW) void mfma_wide_kernel(Stage1Args a, int32_t n_bt) {
  constexpr int NB = kWideNB, NW = kWideNW, MB = kWideMB, KSUB = kWideKSub, PD = kWidePD;
  constexpr int BN = kWideBN, NT = 64 * NW, KH = 32 * KSUB, ROW = KH + 16;   // 160-byte rows: conflict-free reads
  constexpr int HP = BN * (KH / 8) / NT;       // 16-byte pieces of H per thread per sub-chunk
  constexpr int NSUB = kKS / KSUB;
  static_assert(HP >= 1 && HP * NT == BN * (KH / 8), "batch tile vs workgroup size");
  static_assert(kKS % PD == 0 && KSUB % 2 == 0 && kKS % KSUB == 0, "pipeline shape");

  __shared__ uint4 lds_h4[2 * BN * ROW / 8];
  __shared__ uint64_t red[NW][BN];
  __shared__ float2 red_mass[MASS ? NW : 1][MASS ? BN : 1];
  uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_h4);

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b0 = bt * BN;
  const int D = a.D;
  const int nC = (D + kBK - 1) / kBK;
  const int nM = (a.V + 15) / 16;
  int m[MB], mc[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    m[j] = vt * NW * MB + j * NW + wave;
    mc[j] = min(m[j], nM - 1);
  }
  const uint4* wt = static_cast<const uint4*>(a.W) + lane;
  const uint4* wrow[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
    wrow[j] = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.W) +
                                             (int64_t)min(16 * mc[j] + (lane >> 2), a.V - 1) * a.ldw +
                                             8 * (lane & 3));
  const int gather_addr = 4 * (4 * r + q);   // operand lane r + 16q takes run r, piece q
  // 16-byte piece of this lane for row block j, K block c, K step t
  auto wpiece = [&](int j, int c, int t) {
    if constexpr (ROWS) return wrow[j][c * (kBK / 8) + 4 * t];
    else if constexpr (STREAMW) return load_stream16(wt + block_piece(mc[j], c, nC) + t * 64);
    else return wt[block_piece(mc[j], c, nC) + t * 64];
  };
  const uint16_t* H = static_cast<const uint16_t*>(a.H);

  int hn[HP], hk[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = tid + NT * i;
    hn[i] = p / (KH / 8);
    hk[i] = 8 * (p % (KH / 8));
  }
  auto load_h = [&](int s, uint4 (&h)[HP]) {   // sub-chunk s = columns s*KH .. +KH
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const int k = s * KH + hk[i];
      h[i] = make_uint4(0u, 0u, 0u, 0u);
      if (b0 + hn[i] < a.B && k < D) h[i] = *reinterpret_cast<const uint4*>(H + (int64_t)(b0 + hn[i]) * a.ldh + k);
    }
  };
  auto store_h = [&](int buf, const uint4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i)
      *reinterpret_cast<uint4*>(lds_h + buf * BN * ROW + hn[i] * ROW + hk[i]) = h[i];
  };
  const uint16_t* lrd = lds_h + r * ROW + 8 * q;
  auto read_b = [&](int buf, int tt, uint4 (&dst)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      dst[nb] = *reinterpret_cast<const uint4*>(lrd + buf * BN * ROW + nb * 16 * ROW + 32 * tt);
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mm = [&](const uint4 (&x)[MB], const uint4 (&bf)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < MB; ++j) acc[j][nb] = mfma16x16x32(x[j], bf[nb], acc[j][nb]);
  };

  uint4 w[MB][PD];
  uint4 hreg[HP];
  uint4 bf[2][NB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int t = 0; t < PD; ++t) w[j][t] = wpiece(j, 0, t);
  load_h(0, hreg);
  store_h(0, hreg);
  __syncthreads();
  read_b(0, 0, bf[0]);

  // Block c's math. K step t takes W slot t % PD and refills it with step
  // t + PD (in block c + 1 once past the end of c); in the last block no
  // load is issued past the end.
  auto step = [&](int c, bool last) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int sidx = c * NSUB + s;
      const int buf = sidx & 1;
      const bool hmore = !last || s + 1 < NSUB;
      if (hmore) load_h(sidx + 1, hreg);
#pragma unroll
      for (int tt = 0; tt < KSUB; ++tt) {
        const int t = s * KSUB + tt;
        const int tn = t + PD;
        const bool refill = !last || tn < kKS;
        const int cn = tn < kKS ? c : c + 1;
        uint4 x[MB];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          x[j] = ROWS ? lane_gather(w[j][t % PD], gather_addr) : w[j][t % PD];
          if (refill) w[j][t % PD] = wpiece(j, cn, tn % kKS);
        }
        if (tt + 1 < KSUB) {
          read_b(buf, tt + 1, bf[(tt + 1) & 1]);
          mm(x, bf[tt & 1]);
        } else {
          if (hmore) {
            store_h(buf ^ 1, hreg);
            __syncthreads();
            read_b(buf ^ 1, 0, bf[0]);
          }
          mm(x, bf[(KSUB - 1) & 1]);
        }
      }
    }
  };
  for (int c = 0; c + 1 < nC; ++c) step(c, false);
  step(nC - 1, true);

  wide_epilogue<NW, MB, NB, SAMPLE, STORE, MASS, (int)sizeof(lds_h4)>(a, acc, m, vt, b0,
                                                                     reinterpret_cast<float*>(lds_h4), red, red_mass);
}

// ------------------------------------------------------- MFMA, row-major W, wide tiles
// Row-major bf16 W (D a multiple of 128), 64 < B <= 128: the wide tile (wave w owns
// row blocks m[j] = vt * 16 + j * 8 + w, j < 2: 256 vocab rows; the
// workgroup one 128-column batch tile) fed like mfma_rows_kernel: per
// 128-column K block and wave, eight 16-byte wave loads of 4 rows x 256
// contiguous bytes (one K block in flight), each wave's two row blocks moved
// to operand order through a private 8 KiB LDS region (piece p of row rho at
// p ^ rho), H staged per K block and double buffered, one barrier per K
// block, the K loop of workgroup (vt, bt) starting at block vt mod (D / 128).
// W loads are non-temporal with one or two batch tiles (the second reads the
// caches right after the first) and cached with more (later batch tiles of
// the vocab tile re-read W from L2); the plan uses it for one batch tile.
template <bool SAMPLE, bool STORE, bool MASS, bool STREAMW>
__global__ __launch_bounds__(64 * kWideNW) void mfma_rows_wide_kernel(Stage1Args a, int32_t n_bt) {
  constexpr int NB = kWideNB, NW = kWideNW, MB = kWideMB, BN = kWideBN, NT = 64 * NW;
  constexpr int HROW = kRowsBK + 16;                   // padded H row (elements): 288 bytes
  constexpr int HPIECES = BN * (kRowsBK / 8);
  constexpr int HP = HPIECES / NT;
  static_assert(HP * NT == HPIECES, "H pieces per thread");

  __shared__ uint4 lds_w[NW * MB * 16 * 16];           // per wave: MB blocks x 16 rows x 16 pieces
  __shared__ uint4 lds_h4[2 * BN * HROW / 8];
  __shared__ uint64_t red[NW][BN];
  __shared__ float2 red_mass[MASS ? NW : 1][MASS ? BN : 1];
  uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_h4);

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b0 = bt * BN;
  const int nM = (a.V + 15) / 16;
  int m[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) m[j] = vt * NW * MB + j * NW + wave;
  const int nblk = a.D / kRowsBK;
  const int s0 = vt % nblk;
  auto blk = [&](int i) {   // i-th K block of this workgroup's rotated order (i < 2 nblk)
    const int c = s0 + i;
    return c >= nblk ? c - nblk : c;
  };

  // load (j, i) of a block: row 4i + q of row block j (clamped past V), columns 8r .. 8r+7
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  const uint16_t* wsrc[MB][4];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wsrc[j][i] = W + (int64_t)min(16 * min(m[j], nM - 1) + 4 * i + q, a.V - 1) * a.ldw + 8 * r;
  auto wload = [&](int c, int j, int i) {
    if constexpr (STREAMW) return load_stream16(wsrc[j][i] + c * kRowsBK);
    else return *reinterpret_cast<const uint4*>(wsrc[j][i] + c * kRowsBK);
  };
  uint4* region = lds_w + wave * MB * 256;
  const uint16_t* H = static_cast<const uint16_t*>(a.H);

  int hn[HP], hk[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = tid + NT * i;
    hn[i] = p / (kRowsBK / 8);
    hk[i] = 8 * (p % (kRowsBK / 8));
  }
  uint4 hreg[HP];
  auto load_h = [&](int c) {
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      hreg[i] = make_uint4(0u, 0u, 0u, 0u);
      if (b0 + hn[i] < a.B)
        hreg[i] = *reinterpret_cast<const uint4*>(H + (int64_t)(b0 + hn[i]) * a.ldh + c * kRowsBK + hk[i]);
    }
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int i = 0; i < HP; ++i)
      *reinterpret_cast<uint4*>(lds_h + buf * BN * HROW + hn[i] * HROW + hk[i]) = hreg[i];
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // H of the first block first, so its wait does not also wait for W; then
  // W block 0. One K block of W (8 KiB per wave) stays in flight: block i + 1
  // is loaded into the registers of block i as soon as those are in LDS.
  uint4 w[MB][4];
  load_h(blk(0));
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) w[j][k] = wload(blk(0), j, k);
  store_h(0);
  __syncthreads();

  for (int i = 0; i < nblk; ++i) {
    const bool more = i + 1 < nblk;
    if (more) load_h(blk(i + 1));
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) region[(16 * j + 4 * k + q) * 16 + (r ^ (4 * k + q))] = w[j][k];
    {
      const int c2 = blk(more ? i + 1 : i);   // the last block reloads itself (in bounds, unused)
#pragma unroll
      for (int j = 0; j < MB; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) w[j][k] = wload(c2, j, k);
    }
    __builtin_amdgcn_wave_barrier();   // the region's writes before this wave's reads
    const uint16_t* hb = lds_h + (i & 1) * BN * HROW;
#pragma unroll
    for (int t = 0; t < kRowsBK / 32; ++t) {
      uint4 x[MB];
#pragma unroll
      for (int j = 0; j < MB; ++j) x[j] = region[(16 * j + r) * 16 + ((4 * t + q) ^ r)];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 bfrag = *reinterpret_cast<const uint4*>(hb + (nb * 16 + r) * HROW + 32 * t + 8 * q);
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[j][nb] = mfma16x16x32(x[j], bfrag, acc[j][nb]);
      }
    }
    __builtin_amdgcn_wave_barrier();   // this wave's reads before the next block's writes
    if (more) {
      store_h((i + 1) & 1);
      __syncthreads();
    }
  }

  wide_epilogue<NW, MB, NB, SAMPLE, STORE, MASS, (int)sizeof(lds_h4)>(a, acc, m, vt, b0,
                                                                     reinterpret_cast<float*>(lds_h4), red, red_mass);
}

// ------------------------------------------------------- MFMA, wide tiles in few registers
// Batches above 128 on the tiled layout (D a multiple of 256): the wide tile
// of mfma_wide_kernel (8 waves x two 16-row blocks = 256 vocab rows, wave w
// owns row blocks vt * 16 + 8 j + w) with NB 16-column batch blocks:
//  * NB = 8 (batch tile 128) in 128 registers, so two workgroups share each
//    CU and one's waits are covered by the other's matrix work (measured:
//    6-12% faster than mfma_wide_kernel at B = 384 .. 1024, up to 2% at
//    B = 129 .. 256; slower at one batch tile, where mfma_wide_kernel streams
//    W past the caches);
//  * NB = 16 (batch tile 256) in 246 registers, one workgroup per CU: for
//    B = 129 .. 256 W is streamed once instead of once per 128 columns
//    (measured: 2-5% faster than NB = 8 when the last round of workgroups is
//    nearly full, 10% slower when it is a third full, as with 594 tiles on
//    256 CUs: the launcher checks).
//  * W: the A operands straight from the tiled layout, ring_pd(NB) K steps
//    ahead (cached: the later batch tiles of a vocab tile run right after the
//    first on one XCD and find W in its L2).
//  * H: staged per 64-column sub-chunk in double-buffered LDS (160-byte
//    rows), one barrier per sub-chunk. The B operands of a K step pass
//    through a ring of kRingDepth registers instead of a full second set:
//    each slot is refilled right after the matrix instructions that read it,
//    the refills running on into the next K step (across the sub-chunk's
//    barrier), so kRingDepth reads are always in flight.
//  * Both operands are addressed from workgroup-uniform bases plus one 32-bit
//    offset per lane, and the H loads are branch-free (rows past B read row
//    B - 1, whose candidates are dropped; no column lies past D), so the
//    compiler counts loads in flight instead of draining them and keeps
//    few address registers.
constexpr int kRingDepth = 4;                  // B-operand reads in flight
constexpr int64_t kRingMaxLdh = int64_t(1) << 22;   // 32-bit H offsets within a batch tile
constexpr int kRingWideNB = 16;                // column blocks of the one-workgroup-per-CU form
// W prefetch distance in K steps: 2 in the 128-register form; 4 with 16
// column blocks, whose two waves per SIMD hide less latency (4 more
// registers, 246; measured 0.5-3% faster at B = 129-256 on the 4096-, 7168-
// and 8192-wide heads)
constexpr int ring_pd(int NB) { return NB == kRingWideNB ? 4 : 2; }

template <int NB, bool SAMPLE, bool STORE, bool MASS>
__global__ __launch_bounds__(64 * kWideNW, (NB == kWideNB ? 2 : 1) * kWideNW / 4) void mfma_ring_kernel(Stage1Args a,
                                                                                                    int32_t n_bt) {
  constexpr int NW = kWideNW, MB = kWideMB, KSUB = kWideKSub, PD = ring_pd(NB), R = kRingDepth;
  constexpr int BN = 16 * NB, NT = 64 * NW, KH = 32 * KSUB, ROW = KH + 16;   // 160-byte rows: conflict-free reads
  constexpr int HP = BN * (KH / 8) / NT;       // 16-byte pieces of H per thread per sub-chunk
  constexpr int NSUB = kKS / KSUB;
  constexpr int kGroupsPerTile = NW * MB / kGroup;
  static_assert(HP * NT == BN * (KH / 8), "H pieces per thread");
  static_assert(kKS % PD == 0 && kKS % KSUB == 0 && NB % R == 0 && R <= NB, "pipeline shape");
  static_assert(kGroup % NW == 0 && (NW * MB) % kGroup == 0, "row blocks of a tile fill whole groups");

  __shared__ uint4 lds_h4[2 * BN * ROW / 8];
  __shared__ uint64_t red[NW][BN];
  __shared__ float2 red_mass[MASS ? NW : 1][MASS ? BN : 1];
  uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_h4);

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b0 = bt * BN;
  const int D = a.D;
  const int nC = (D + kBK - 1) / kBK;
  const int nM = (a.V + 15) / 16;

  // W: row block j of this wave sits in group mc / kGroup (0 or 1 within the
  // tile), slot mc % kGroup; past V the last row block is read again
  const char* w_wg = reinterpret_cast<const char*>(a.W) + (int64_t)vt * kGroupsPerTile * nC * kGroup * kBlock16 * 16;
  int m[MB];
  uint32_t woff[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    m[j] = vt * NW * MB + j * NW + wave;
    const int mc = min(m[j], nM - 1);
    const int g = mc / kGroup - vt * kGroupsPerTile;
    woff[j] = (uint32_t)(((g * nC * kGroup + mc % kGroup) * kBlock16 + lane) * 16);
  }
  auto wpiece = [&](int j, int c, int t) {
    const uint4* p =
        reinterpret_cast<const uint4*>(w_wg + (woff[j] + (uint32_t)(c * kGroup * kBlock16 + t * 64) * 16u));
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
  };

  // H: piece i of this thread is row hn of the batch tile, columns hk .. +8
  // of the sub-chunk
  const char* h_wg = reinterpret_cast<const char*>(a.H) + (int64_t)b0 * a.ldh * 2;
  uint32_t hrow[HP];
  int hk[HP], hst[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = tid + NT * i;
    const int hn = p / (KH / 8);
    hk[i] = 8 * (p % (KH / 8));
    hrow[i] = (uint32_t)min(hn, a.B - 1 - b0) * (uint32_t)a.ldh;
    hst[i] = hn * ROW + hk[i];
  }
  auto load_h = [&](int s, uint4 (&h)[HP]) {   // sub-chunk s = columns s*KH .. +KH
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(h_wg + (hrow[i] + (uint32_t)(s * KH + hk[i])) * 2u);
      h[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  auto store_h = [&](int buf, const uint4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i) *reinterpret_cast<uint4*>(lds_h + buf * BN * ROW + hst[i]) = h[i];
  };
  const uint16_t* lrd = lds_h + r * ROW + 8 * q;
  auto read_b = [&](int buf, int tt, int nb) {
    return *reinterpret_cast<const uint4*>(lrd + buf * BN * ROW + nb * 16 * ROW + 32 * tt);
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 w[MB][PD];
  uint4 hreg[HP];
  uint4 ring[R];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int t = 0; t < PD; ++t) w[j][t] = wpiece(j, 0, t);
  load_h(0, hreg);
  store_h(0, hreg);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < R; ++i) ring[i] = read_b(0, 0, i);

  // K block c. K step t uses W slot t % PD and refills it with step t + PD
  // (in block c + 1 past the end of c; in the last block nothing is loaded
  // past the end). The sub-chunk and step indices are compile-time
  // constants (static_for), so every register array index is one.
  auto step = [&](int c, bool last) {
    static_for<NSUB>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      const int sidx = c * NSUB + s;
      const int buf = sidx & 1;
      const bool hmore = !last || s + 1 < NSUB;
      if (hmore) load_h(sidx + 1, hreg);
      static_for<KSUB>([&](auto tt_c) {
        constexpr int tt = decltype(tt_c)::value;
        constexpr int t = s * KSUB + tt;
        constexpr int tn = t + PD;
        const bool refill = !last || tn < kKS;
        const int cn = tn < kKS ? c : c + 1;
        constexpr bool in_sub = tt + 1 < KSUB;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int j = 0; j < MB; ++j) acc[j][nb] = mfma16x16x32(w[j][t % PD], ring[nb % R], acc[j][nb]);
          const int nn = nb + R;
          if (nn < NB) {
            ring[nb % R] = read_b(buf, tt, nn);
          } else if (in_sub) {
            ring[nb % R] = read_b(buf, tt + 1, nn - NB);
          } else if (hmore) {
            if (nn == NB) {
              store_h(buf ^ 1, hreg);
              __syncthreads();
            }
            ring[nb % R] = read_b(buf ^ 1, 0, nn - NB);
          }
          __builtin_amdgcn_sched_barrier(0);   // keep the ring order: R reads in flight, no more
        }
        if (refill) {
#pragma unroll
          for (int j = 0; j < MB; ++j) w[j][t % PD] = wpiece(j, cn, tn % kKS);
        }
      });
    });
  };
  for (int c = 0; c + 1 < nC; ++c) step(c, false);
  step(nC - 1, true);

  wide_epilogue<NW, MB, NB, SAMPLE, STORE, MASS, (int)sizeof(lds_h4)>(a, acc, m, vt, b0,
                                                                     reinterpret_cast<float*>(lds_h4), red, red_mass);
}

// ------------------------------------------------------- MFMA, 256 x 256 tiles
// Opt-in (batch_tile = 256; measured within 1-3% of the wide kernel at
// B = 512 .. 1024, not ahead of it, so the plan does not pick it by itself).
// Large batches on the tiled layout (D a multiple of 32): a workgroup of 8
// waves owns a 256-row vocab tile and a 256-column batch tile; wave w
// computes vocab quarter w & 3 (4 row blocks) x batch half w >> 2 (8 column
// blocks), 128 fp32 accumulators per lane. Per matrix operation this moves
// half the L2-to-CU bytes of the 256 x 128 wide tile.
//  * Both operands are copied straight from memory into LDS by the load
//    units (global_load_lds_dwordx4: each wave load fills 1 KiB of LDS, lane
//    i at byte 16 i), one K step (32 columns) per stage, in a ring of 4
//    stages with 3 in flight: no registers hold loads in flight.
//    W: one wave load per row block (its K step is already 1 KiB in A-operand
//    order). H: one wave load per 16 batch rows (64 bytes each), the four
//    16-byte pieces of row n stored in the order q ^ ((n >> 2) & 3) (the
//    counters still show 4 bank-conflict cycles per B-operand read with it;
//    H copied in operand order has none but its 16-row copies cost more).
//  * Each wave waits for its own copies with an explicit vmcnt, then the
//    workgroup barrier (s_barrier, no fence) publishes the stage; the LDS
//    operand reads are written in assembly and wait for themselves, so the
//    compiler does not insert a wait for every copy in flight before them.
//  * The two waves of each SIMD run a ping-pong schedule (one reads LDS while
//    the other issues matrix instructions; see the main loop). Measured
//    against the same tile with all waves in lockstep: 1-2% faster
//    (4096 x 128256 head B = 1024: 1073 against 1084 us); the sustained clock
//    under this load is about 1.71 GHz, which puts the bf16 matrix peak near
//    1.79 PFLOP/s.
//  * Epilogue as in the wide kernel, then the four vocab quarters of each
//    column meet in LDS.
constexpr int kBigRows = 256, kBigCols = 256, kBigWaves = 8, kBigNS = 4;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// s_waitcnt with only the vector-memory count (expcnt and lgkmcnt: no wait)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

__global__ __launch_bounds__(64 * kBigWaves) void mfma_big_kernel(Stage1Args a, int32_t n_bt) {
  constexpr int NT = 64 * kBigWaves;
  constexpr int W_ST = 16 * 64, H_ST = kBigCols * 4;   // uint4 per stage: W 16 KiB, H 16 KiB
  constexpr int MJ = 4, NJ = 8;                       // row blocks, column blocks per wave
  __shared__ uint4 lds_w[kBigNS * W_ST];
  __shared__ uint4 lds_hb[kBigNS * H_ST];
  __shared__ uint64_t red[4][kBigCols];

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int vw = wave & 3, bw = wave >> 2;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b0 = bt * kBigCols;
  const int D = a.D;
  const int nC = (D + kBK - 1) / kBK;
  const int nM = (a.V + 15) / 16;
  const int S = D / 32;                               // K steps = stages
  const uint4* Wt = static_cast<const uint4*>(a.W);
  const uint16_t* H = static_cast<const uint16_t*>(a.H);

  // this wave's copies of a stage: row blocks 2w, 2w + 1 of W; batch rows
  // 32w .. 32w + 31 of H (lane: row 16 i + lane / 4, stored piece lane & 3)
  const uint4* wsrc[2];
  const uint16_t* hsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = min(vt * 16 + 2 * wave + i, nM - 1);
    wsrc[i] = Wt + (((int64_t)(blk / kGroup) * nC) * kGroup + (blk % kGroup)) * kBlock16 + lane;
    const int row = 32 * wave + 16 * i + (lane >> 2);
    const int piece = (lane & 3) ^ ((row >> 2) & 3);
    hsrc[i] = H + (int64_t)min(b0 + row, a.B - 1) * a.ldh + 8 * piece;
  }
  auto issue = [&](int st) {
    const int c = st >> 3, t = st & 7;
    const int buf = st % kBigNS;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // block (blk, c) sits kGroup * kBlock16 pieces after block (blk, c - 1)
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + (int64_t)c * kGroup * kBlock16 + t * 64),
                                       (lds_void_t*)(lds_w + buf * W_ST + (2 * wave + i) * 64), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(hsrc[i] + 32 * st),
                                       (lds_void_t*)(lds_hb + buf * H_ST + (2 * wave + i) * 64), 16, 0, 0);
    }
  };

  f32x4 acc[MJ][NJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j)
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS byte addresses of this lane's operand pieces in stage buffer 0
  uint32_t aoff[MJ], boff[NJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j)
    aoff[j] = (uint32_t)(uintptr_t)(lds_w + (vw * MJ + j) * 64 + lane);
#pragma unroll
  for (int nb = 0; nb < NJ; ++nb) {
    const int n = bw * 128 + nb * 16 + r;
    boff[nb] = (uint32_t)(uintptr_t)(lds_hb + n * 4 + (q ^ ((n >> 2) & 3)));
  }

  // Ping-pong schedule. Waves w and w + 4 share a SIMD and sit in different
  // groups (grp = w >> 2). Each K step (stage) s of a wave is a memory phase
  // M(s) -- issue its copies for stage s + 3, read its stage-s operands from
  // LDS into registers -- and a compute phase C(s): its 32 matrix
  // instructions. Group 1 starts one phase late (one extra barrier), so
  // between consecutive workgroup barriers one wave of every SIMD computes
  // while the other reads LDS and issues copies:
  //   barrier 2s-1 .. 2s: group 0 M(s), group 1 C(s-1)
  //   barrier 2s .. 2s+1: group 0 C(s), group 1 M(s)
  // Stage s + 1 must be complete before barrier 2s+1 (group 0 reads it right
  // after): each wave waits for its own copies of it at the end of the phase
  // before that barrier (group 0: end of C(s); group 1: end of M(s)). The
  // copies for stage s + 3 overwrite the buffer of stage s - 1, whose last
  // reads ended before barrier 2s-1. Every wave passes 2 S + 2 barriers.
  const int grp = wave >> 2;
  auto wait_stage = [&](int st) {   // own copies of stage st done; later stages may stay in flight
    const int ahead = min(S - 1, st + 2) - st;
    if (ahead >= 2) wait_vmcnt<8>();
    else if (ahead == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
  };
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  u32x4v av[MJ], bv[NJ];
  auto read_operands = [&](int st) {
    const uint32_t wb = (uint32_t)((st % kBigNS) * W_ST * 16), hb = (uint32_t)((st % kBigNS) * H_ST * 16);
    asm volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %13\n\t"
        "ds_read_b128 %2, %14\n\t"
        "ds_read_b128 %3, %15\n\t"
        "ds_read_b128 %4, %16\n\t"
        "ds_read_b128 %5, %17\n\t"
        "ds_read_b128 %6, %18\n\t"
        "ds_read_b128 %7, %19\n\t"
        "ds_read_b128 %8, %20\n\t"
        "ds_read_b128 %9, %21\n\t"
        "ds_read_b128 %10, %22\n\t"
        "ds_read_b128 %11, %23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(av[0]), "=&v"(av[1]), "=&v"(av[2]), "=&v"(av[3]), "=&v"(bv[0]), "=&v"(bv[1]), "=&v"(bv[2]),
          "=&v"(bv[3]), "=&v"(bv[4]), "=&v"(bv[5]), "=&v"(bv[6]), "=&v"(bv[7])
        : "v"(aoff[0] + wb), "v"(aoff[1] + wb), "v"(aoff[2] + wb), "v"(aoff[3] + wb), "v"(boff[0] + hb),
          "v"(boff[1] + hb), "v"(boff[2] + hb), "v"(boff[3] + hb), "v"(boff[4] + hb), "v"(boff[5] + hb),
          "v"(boff[6] + hb), "v"(boff[7] + hb)
        : "memory");
  };
  auto compute = [&] {
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
      for (int j = 0; j < MJ; ++j)
        acc[j][nb] = mfma16x16x32(__builtin_bit_cast(uint4, av[j]), __builtin_bit_cast(uint4, bv[nb]), acc[j][nb]);
  };

  for (int st = 0; st < 3 && st < S; ++st) issue(st);
  wait_stage(0);
  barrier();                                          // stage 0 is in LDS for every wave
  if (grp == 1) barrier();
  for (int st = 0; st < S; ++st) {
    // M(st)
    if (st + 3 < S) issue(st + 3);                    // into the buffer of stage st - 1
    read_operands(st);
    if (grp == 1 && st + 1 < S) wait_stage(st + 1);
    barrier();
    // C(st)
    compute();
    if (grp == 0 && st + 1 < S) wait_stage(st + 1);
    barrier();
  }
  if (grp == 0) barrier();

  // epilogue: per batch column, the lane's 16 candidates (4 row blocks x 4
  // rows, increasing vocab order), then the 4 lanes of the column, then the
  // four vocab quarters
  auto tile_max = [&](auto greedy_c, auto full_c) {
    constexpr bool kGreedy = decltype(greedy_c)::value;
    constexpr bool kFull = decltype(full_c)::value;
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb) {
      const int col = bw * 128 + nb * 16 + r;
      const int b = b0 + col;
      RunMax best = runmax_init();
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        const int v0 = 16 * (vt * 16 + vw * MJ + j) + 4 * q;
        uint4 words = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (!kGreedy) words = philox_quad(a.nk, (uint32_t)(v0 >> 2), (uint32_t)b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float l = acc[j][nb][e];
          const float sc = kGreedy ? l : score2(l, a.score_scale, pick_word(words, e));
          if (kFull || v0 + e < a.V) runmax_take(best, sc, v0 + e);
        }
      }
      uint64_t key = runmax_key(best);
      key = umax64(key, shfl_xor_u64(key, 16));
      key = umax64(key, shfl_xor_u64(key, 32));
      if (q == 0) red[vw][col] = key;
    }
  };
  const bool full = (int64_t)(vt + 1) * kBigRows <= a.V;
  if (a.greedy) {
    if (full) tile_max(std::true_type{}, std::true_type{});
    else tile_max(std::true_type{}, std::false_type{});
  } else {
    if (full) tile_max(std::false_type{}, std::true_type{});
    else tile_max(std::false_type{}, std::false_type{});
  }
  __syncthreads();
  uint64_t k = 0ull;
  if (tid < kBigCols) k = umax64(umax64(red[0][tid], red[1][tid]), umax64(red[2][tid], red[3][tid]));
  publish_candidates(a, vt, b0, min(kBigCols, a.B - b0), k, tid, NT);
}

template <int BB, int NW>
hipError_t launch_gemv_bb(const Stage1Args& a, hipStream_t stream) {
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const dim3 grid(a.n_tiles, (a.B + BB - 1) / BB);
  const size_t lds = (size_t)BB * a.D * 2;
  void (*k)(Stage1Args) = nullptr;
  if (sample && store) k = gemv_tiled_kernel<BB, NW, true, true>;
  else if (sample) k = gemv_tiled_kernel<BB, NW, true, false>;
  else k = gemv_tiled_kernel<BB, NW, false, true>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  Stage1Args b = a;
  if ((int64_t)grid.x * grid.y > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // workgroup count is int32
  b.total_wgs = (int32_t)(grid.x * grid.y);
  return launch(k, grid, dim3(64 * NW), lds, stream, b);
}

template <int NW>
hipError_t launch_gemv_nw(const Stage1Args& a, hipStream_t stream) {
  int bb = a.B <= 1 ? 1 : a.B <= 2 ? 2 : 4;
  while (bb > 1 && (int64_t)bb * a.D * 2 > kMaxHLds) bb /= 2;   // BB rows of H must fit the LDS
  if (bb == 1) return launch_gemv_bb<1, NW>(a, stream);
  if (bb == 2) return launch_gemv_bb<2, NW>(a, stream);
  return launch_gemv_bb<4, NW>(a, stream);
}

int device_cu_count();

// Workgroups of kernel K (`threads` per workgroup, static LDS only) resident
// at once on the current device: queried once per device, 0 if unknown.
template <auto K>
int resident_wgs(int threads) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(K), threads, 0) !=
            hipSuccess ||
        per_cu <= 0)
      return 0;
    n = per_cu * device_cu_count();
    if (n > 0) cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Vocab tiles of the last round of workgroups, when a full round comes
// before it and the last round is at most a quarter full.
int64_t ragged_last_round(int64_t n_tiles, int64_t slots) {
  if (slots <= 0 || n_tiles <= slots) return 0;
  const int64_t rem = n_tiles % slots;
  return 4 * rem <= slots ? rem : 0;
}

template <int NB, int NW, bool SAMPLE, bool STORE, bool MASS>
hipError_t launch_mfma_nb_k(const Stage1Args& a, hipStream_t stream) {
  constexpr int BN = 16 * NB;
  const int n_bt = (a.B + BN - 1) / BN;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  if (a.half_tiles == 0)
    return launch(mfma_tiled_kernel<NB, NW, SAMPLE, STORE, MASS>, dim3((unsigned)grid), dim3(64 * NW), 0, stream, b,
                  (int32_t)n_bt);
  if constexpr (NW == 8 && NB >= 2 && SAMPLE && !STORE && !MASS) {
    if (n_bt == 1 && a.half_tiles <= a.n_tiles)
      return launch(mfma_tiled_kernel<NB, NW, true, false, false, true>, dim3((unsigned)grid), dim3(64 * NW), 0,
                    stream, b, (int32_t)1);
  }
  return hipErrorInvalidValue;   // 64-row tiles are planned only for this case
}

template <int NB, int NW>
hipError_t launch_mfma_nb(const Stage1Args& a, hipStream_t stream) {
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  if (a.mass)
    return store ? launch_mfma_nb_k<NB, NW, true, true, true>(a, stream)
                 : launch_mfma_nb_k<NB, NW, true, false, true>(a, stream);
  if (sample && store) return launch_mfma_nb_k<NB, NW, true, true, false>(a, stream);
  if (sample) return launch_mfma_nb_k<NB, NW, true, false, false>(a, stream);
  return launch_mfma_nb_k<NB, NW, false, true, false>(a, stream);
}

template <int NB, int NW>
hipError_t launch_rows_nb(const Stage1Args& a, hipStream_t stream) {
  constexpr int BN = 16 * NB;
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const int n_bt = (a.B + BN - 1) / BN;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  if (a.D % kRowsBK != 0) return hipErrorInvalidValue;
  void (*k)(Stage1Args, int32_t) = nullptr;
  if (a.mass) k = store ? mfma_rows_kernel<NB, NW, true, true, true> : mfma_rows_kernel<NB, NW, true, false, true>;
  else if (sample && store) k = mfma_rows_kernel<NB, NW, true, true, false>;
  else if (sample) k = mfma_rows_kernel<NB, NW, true, false, false>;
  else k = mfma_rows_kernel<NB, NW, false, true, false>;
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  return launch(k, dim3((unsigned)grid), dim3(64 * NW), 0, stream, b, (int32_t)n_bt);
}

template <int NW>
hipError_t launch_rows_nw(const Stage1Args& a, hipStream_t stream) {
  const int bn = a.batch_tile ? a.batch_tile : (a.B <= 16 ? 16 : a.B <= 32 ? 32 : 64);
  if (bn == 16) return launch_rows_nb<1, NW>(a, stream);
  if (bn == 32) return launch_rows_nb<2, NW>(a, stream);
  return launch_rows_nb<4, NW>(a, stream);
}

template <int NB>
hipError_t launch_mfma_ring_k(const Stage1Args& a, hipStream_t stream) {
  const int n_bt = (a.B + 16 * NB - 1) / (16 * NB);
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  if (a.ldh >= kRingMaxLdh || a.D % kBK != 0) return hipErrorInvalidValue;
  void (*k)(Stage1Args, int32_t) = nullptr;
  if (a.mass) k = store ? mfma_ring_kernel<NB, true, true, true> : mfma_ring_kernel<NB, true, false, true>;
  else if (sample && store) k = mfma_ring_kernel<NB, true, true, false>;
  else if (sample) k = mfma_ring_kernel<NB, true, false, false>;
  else k = mfma_ring_kernel<NB, false, true, false>;
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  return launch(k, dim3((unsigned)grid), dim3(64 * kWideNW), 0, stream, b, (int32_t)n_bt);
}

// Compute units of the current device (queried once per device; 0 if the
// query fails).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    cache[dev].store(n, std::memory_order_relaxed);
  return n > 0 ? n : 0;
}

// Only where the kernel with the 64-row tiles keeps as many workgroups
// resident as the one without.
template <int NB>
int64_t half_tiles_nb(int64_t n_tiles) {
  const int slots = resident_wgs<mfma_tiled_kernel<NB, 8, true, false, false, true>>(64 * 8);
  if (slots != resident_wgs<mfma_tiled_kernel<NB, 8, true, false, false>>(64 * 8)) return 0;
  return 2 * ragged_last_round(n_tiles, slots);
}

// One 256-column batch tile (one workgroup per CU) when it covers B and the
// last round of workgroups is empty or at least 9/16 full; else 128-column
// batch tiles at two workgroups per CU. Measured at B = 160 and 256 on
// 4096-wide heads: the 256-column tile 4-8% faster with the last round 59%
// and 65% full, the 128-column tiles 4-7% faster at 31, 40, 45 and 50%.
hipError_t launch_mfma_ring(const Stage1Args& a, hipStream_t stream) {
  if (a.B <= 16 * kRingWideNB) {
    const int cus = device_cu_count();
    const int64_t rem = cus > 0 ? a.n_tiles % cus : -1;
    if (rem == 0 || 16 * rem >= 9 * (int64_t)cus) return launch_mfma_ring_k<kRingWideNB>(a, stream);
  }
  return launch_mfma_ring_k<kWideNB>(a, stream);
}

template <bool ROWS, bool STREAMW>
hipError_t launch_mfma_wide_k(const Stage1Args& a, int n_bt, hipStream_t stream) {
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  void (*k)(Stage1Args, int32_t) = nullptr;
  if (a.mass)
    k = store ? mfma_wide_kernel<true, true, true, ROWS, STREAMW> : mfma_wide_kernel<true, false, true, ROWS, STREAMW>;
  else if (sample && store) k = mfma_wide_kernel<true, true, false, ROWS, STREAMW>;
  else if (sample) k = mfma_wide_kernel<true, false, false, ROWS, STREAMW>;
  else k = mfma_wide_kernel<false, true, false, ROWS, STREAMW>;
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  return launch(k, dim3((unsigned)grid), dim3(64 * kWideNW), 0, stream, b, (int32_t)n_bt);
}

template <bool STREAMW>
hipError_t launch_rows_wide_k(const Stage1Args& a, int n_bt, hipStream_t stream) {
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  if (a.D % kRowsBK != 0) return hipErrorInvalidValue;
  void (*k)(Stage1Args, int32_t) = nullptr;
  if (a.mass)
    k = store ? mfma_rows_wide_kernel<true, true, true, STREAMW> : mfma_rows_wide_kernel<true, false, true, STREAMW>;
  else if (sample && store) k = mfma_rows_wide_kernel<true, true, false, STREAMW>;
  else if (sample) k = mfma_rows_wide_kernel<true, false, false, STREAMW>;
  else k = mfma_rows_wide_kernel<false, true, false, STREAMW>;
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  return launch(k, dim3((unsigned)grid), dim3(64 * kWideNW), 0, stream, b, (int32_t)n_bt);
}

hipError_t launch_rows_wide(const Stage1Args& a, hipStream_t stream) {
  const int n_bt = (a.B + kWideBN - 1) / kWideBN;
  return n_bt <= 2 ? launch_rows_wide_k<true>(a, n_bt, stream) : launch_rows_wide_k<false>(a, n_bt, stream);
}

// Tiled W read by at most two batch tiles streams past the caches; row-major
// W keeps cached loads (the second half of each 128-byte line is the next K
// step's).
template <bool ROWS>
hipError_t launch_mfma_wide(const Stage1Args& a, hipStream_t stream) {
  // two or more batch tiles: the 128-register form, two workgroups per CU
  if (!ROWS && a.B > kWideBN && a.D % kBK == 0 && a.ldh < kRingMaxLdh) return launch_mfma_ring(a, stream);
  const int n_bt = (a.B + kWideBN - 1) / kWideBN;
  if (!ROWS && n_bt <= 2) return launch_mfma_wide_k<false, true>(a, n_bt, stream);
  return launch_mfma_wide_k<ROWS, false>(a, n_bt, stream);
}

// The 256 x 256 tile: tiled W with D a multiple of 32, sampling without
// stores or log-masses (the plan checks these before choosing it).
hipError_t launch_mfma_big(const Stage1Args& a, hipStream_t stream) {
  const int n_bt = (a.B + kBigCols - 1) / kBigCols;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  if (a.D % 32 != 0 || a.cand == nullptr || a.logits != nullptr || a.mass != nullptr)
    return hipErrorInvalidValue;
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  return launch(mfma_big_kernel, dim3((unsigned)grid), dim3(64 * kBigWaves), 0, stream, b, (int32_t)n_bt);
}

template <int NW>
hipError_t launch_mfma_nw(const Stage1Args& a, hipStream_t stream) {
  const int bn = a.batch_tile ? a.batch_tile : (a.B <= 16 ? 16 : a.B <= 32 ? 32 : 64);
  if (bn == 16) return launch_mfma_nb<1, NW>(a, stream);
  if (bn == 32) return launch_mfma_nb<2, NW>(a, stream);
  return launch_mfma_nb<4, NW>(a, stream);
}

}  // namespace

int64_t tiled_weights_bytes(int64_t V, int64_t D) {
  const int64_t groups = ((V + 15) / 16 + kGroup - 1) / kGroup;
  return groups * kGroup * ((D + kBK - 1) / kBK) * (int64_t)kBlock16 * 16;
}

hipError_t launch_pack_tiled(const void* W, int64_t ldw, int32_t V, int32_t D, void* out, hipStream_t stream) {
  const int nC = (D + kBK - 1) / kBK;
  const int64_t n16 = tiled_weights_bytes(V, D) / 16;
  if ((n16 + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((n16 + 255) / 256));
  return launch(pack_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(W), ldw, V, D, nC, n16,
                static_cast<uint4*>(out));
}

// Row-major bf16 W with D a multiple of 256, MFMA: the tiled-layout MFMA
// kernels reading their A operand straight from the rows (vocab tile 64 or
// 128 = 4 or 8 waves of one row block; 256 = the wide kernel).
bool rows_direct_ok(int64_t D) { return D % kBK == 0; }

hipError_t launch_stage1_rows_direct(const Stage1Args& a, hipStream_t stream) {
  // wide tile: the LDS-transposing row kernel for one batch tile (B <= 128),
  // the row-direct wide kernel above (measured, 4096 x 128256 head: B = 128
  // 200 us against 248-254; B = 256 360 against 329-333, where the matrix
  // cores bound the loop and the extra LDS traffic of the transpose costs)
  if (a.vocab_tile == kWideRows)
    return a.B <= kWideBN ? launch_rows_wide(a, stream) : launch_mfma_wide<true>(a, stream);
  return a.vocab_tile == 128 ? launch_rows_nw<8>(a, stream) : launch_rows_nw<4>(a, stream);
}

// Vocab tile = 16 rows per wave x waves per workgroup (4 or 8), or the
// 256-row wide tile (8 waves x 2 row blocks, MFMA only).
hipError_t launch_stage1_tiled(const Stage1Args& a, bool mfma, hipStream_t stream) {
  if (mfma && a.vocab_tile == kWideRows)
    return a.batch_tile == kBigCols ? launch_mfma_big(a, stream) : launch_mfma_wide<false>(a, stream);
  const bool eight = a.vocab_tile == 128;
  if (mfma) return eight ? launch_mfma_nw<8>(a, stream) : launch_mfma_nw<4>(a, stream);
  return eight ? launch_gemv_nw<8>(a, stream) : launch_gemv_nw<4>(a, stream);
}

// Sampling with 128-row tiles and one batch tile of 32 or 64 columns: the
// tiles of a last round of workgroups at most a quarter full run as two
// 64-row tiles each, in the same launch. Measured on 4096-wide heads with
// V = 69376, 72064, 78592 and 202048 (last round 6-20% full): 2-4% faster at
// B = 24 and 1-2% at B = 64 than the same tiles split by batch columns in a
// second launch, which in turn was 2-7% faster than no split. Not for a last
// round a third full (the 3584 x 152064 head: 3% slower) nor for 16-column
// batch tiles (2% slower at 16% full): a lone 128-row tile per CU already
// keeps more W in flight than its two halves do. Returns the number of
// 64-row tiles (twice the tiles so split).
int64_t tiled_half_tiles(int64_t n_tiles, int64_t B, int32_t batch_tile) {
  const int64_t bn = batch_tile ? batch_tile : (B <= 16 ? 16 : B <= 32 ? 32 : 64);
  if (B > bn || bn == 16) return 0;
  if (bn == 32) return half_tiles_nb<2>(n_tiles);
  return half_tiles_nb<4>(n_tiles);
}

}  // namespace fs
