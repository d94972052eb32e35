// Internal header shared by the HIP translation units of libflashsample.
//
// Device side: the noise (Philox4x32-10 -> uniform -> Gumbel, and the group
// stream of the grouped variant), log-mass pairs, the packed 64-bit candidate
// key and the running maximum, the logits store, candidate publication
// (two-stage and single-pass), and small wavefront helpers. Host side: the
// launch helper, the Stage-1 argument block and the declarations of each
// kernel family's launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "../../include/flashsample.h"

namespace fs {

// ------------------------------------------------------------------ noise
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11, Section 4): ten rounds of two 32x32->64-bit
// multiplies with the paper's multipliers, the key bumped by its Weyl
// constants between rounds.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct Key2 {
  uint32_t k0, k1;
};

// a ^ b ^ c in one gfx950 instruction (v_bitop3_b32 with the truth table of
// three-input parity, 0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c.x;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c.z;
    c = make_uint4(xor3((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1,
                   xor3((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0);
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return c;
}

// The four words for vocab indices 4q .. 4q+3 of batch row b.
struct NoiseKey {
  uint32_t seed_lo, seed_hi, step_lo, step_hi;
};

__device__ __forceinline__ uint4 philox_quad(const NoiseKey& nk, uint32_t q, uint32_t b) {
  return philox4x32_10(make_uint4(q, b, nk.step_lo, nk.step_hi), nk.seed_lo, nk.seed_hi);
}

__device__ __forceinline__ uint32_t pick_word(const uint4& w, int j) {
  return j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
}

// Standard Gumbel from a 32-bit word, u = (x + 1/2) 2^-32, g = -ln(-ln u),
// in base-2 units. The kernels compare perturbed scores
//     s2 = l * (1 / (T ln 2)) + g2,   g2 = -log2(e2),   e2 = -log2 u,
// which is s = l / T + g divided by ln 2 plus the constant log2(ln 2)
// (g = ln 2 * g2 - ln(ln 2)): a positive affine map of s, so neither the
// maximiser nor the order of any two scores changes, and the two scalings by
// ln 2 of the natural-log form drop out. Both logarithms are the hardware
// base-2 logarithm (v_log_f32). The inner one is taken two ways:
//  * u <= 1/2 (x < 2^31): directly, from u formed with one rounding;
//  * u >  1/2: from c = 1 - u = (~x + 1/2) 2^-32, formed from the integer
//    (the largest Gumbels live here, where u itself cannot resolve them).
//    With w = fl(1 - c), d = (1 - w) - c is exact (Sterbenz: 1 - w is c up
//    to the rounding of w, at most 2^-25), so 1 - c = w + d and
//    ln(1 - c) = ln w + ln(1 + d / w) = ln w + d (2 - w) + O(d (1 - w)^2),
//    an error below 2^-26 (first-order log1p, d / w ~ d (2 - w) on
//    [1/2, 1]). w == 1 (c < 2^-25) needs no special case: ln w = 0, d = -c.
// Each uniform carries one fp32 rounding (relative 2^-24), which moves g by
// about 1e-7; the bound checked against the fp64 definition is 1e-5.
constexpr float kInvLn2 = 1.44269504088896340736f;
constexpr float kLn2f = 0.693147180559945309f;
constexpr float kNegLnLn2 = 0.366512920581664327f;   // -ln(ln 2)

__device__ __forceinline__ float gumbel2_from_word(uint32_t x) {
  const bool low = x < 0x80000000u;
  // one conversion: v = u for x < 2^31, else v = c = 1 - u (from ~x)
  const float v = fmaf((float)(low ? x : ~x), 0x1p-32f, 0x1p-33f);
  const float w = 1.0f - v;
  const float d = (1.0f - w) - v;
  const float corr = low ? 0.0f : d * (2.0f - w);          // ln(1 - c) - ln w
  const float e2 = fmaf(corr, -kInvLn2, -__builtin_amdgcn_logf(low ? v : w));
  return -__builtin_amdgcn_logf(e2);
}

// The same Gumbel in natural units (group noise, the noise test entry).
__device__ __forceinline__ float gumbel_from_word(uint32_t x) {
  return fmaf(kLn2f, gumbel2_from_word(x), kNegLnLn2);
}

// Perturbed score of logit l in base-2 units (scale = 1 / (T ln 2)).
__device__ __forceinline__ float score2(float l, float scale, uint32_t word) {
  return fmaf(l, scale, gumbel2_from_word(word));
}

// Group stream of the grouped variant: the same key, counter word 0 tagged so
// it never meets a token counter (those are v >> 2 < 2^29).
constexpr uint32_t kGroupCounterTag = 0xC0000000u;

__device__ __forceinline__ float group_gumbel(const NoiseKey& nk, uint32_t k, uint32_t b) {
  const uint4 w = philox4x32_10(make_uint4(kGroupCounterTag | (k >> 2), b, nk.step_lo, nk.step_hi), nk.seed_lo,
                                nk.seed_hi);
  return gumbel_from_word(pick_word(w, (int)(k & 3u)));
}

// ------------------------------------------------------------------ log-mass
// A partial log-mass is a pair (m, s) standing for s * e^m: m the largest
// element seen (-inf: none), s the sum of e^(x - m) over the elements (>= 1
// once one is seen). Merging two pairs rescales to the larger m; the mass is
// m + ln s. +inf elements make the mass +inf.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -__builtin_inff()) return;   // both empty
  if (M == __builtin_inff()) {
    m = M;
    s = 1.0f;
    return;
  }
  constexpr float kLog2e = 1.4426950408889634f;
  s = s * __builtin_amdgcn_exp2f((m - M) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - M) * kLog2e);
  m = M;
}

__device__ __forceinline__ float lse_value(float m, float s) {
  constexpr float kLn2 = 0.693147180559945309f;
  return m == -__builtin_inff() || m == __builtin_inff() ? m : m + kLn2 * __builtin_amdgcn_logf(s);
}

// ------------------------------------------------------------------ candidate keys
// A candidate (score s, vocab index v) packs into one 64-bit key whose
// unsigned order is (s ascending, v descending):
//   key = ord(s) << 32 | (0xFFFFFFFF - v),
// ord() flips float bits into an order-preserving unsigned int. NaN scores
// and "no candidate" are key 0, which loses to every real candidate, so the
// maximum key is the highest score with the lowest index on ties.
__device__ __forceinline__ uint64_t pack_key(float s, uint32_t v) {
  const uint32_t bits = __float_as_uint(s);
  const uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  const uint64_t key = ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - v);
  return (s != s) ? 0ull : key;
}

// Running argmax of one lane over candidates presented in increasing vocab
// order: a strictly greater score replaces the best, so equal scores keep the
// lowest index; a NaN best (the initial state) is replaced by anything, and a
// NaN candidate never replaces a number. Its key equals the maximum of the
// candidates' pack_key values (0 when there were none or all were NaN).
struct RunMax {
  float s;
  int32_t v;
};

__device__ __forceinline__ RunMax runmax_init() { return RunMax{__builtin_nanf(""), -1}; }

__device__ __forceinline__ void runmax_take(RunMax& m, float s, int32_t v) {
  const bool take = s > m.s || m.s != m.s;
  m.s = take ? s : m.s;
  m.v = take ? v : m.v;
}

__device__ __forceinline__ uint64_t runmax_key(const RunMax& m) {
  return m.v < 0 ? 0ull : pack_key(m.s, (uint32_t)m.v);
}

__device__ __forceinline__ int32_t key_to_token(uint64_t key) {
  return key == 0ull ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)key);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask) {
  const uint32_t lo = __shfl_xor((uint32_t)x, mask);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}

// ------------------------------------------------------------------ streaming loads
// W is read exactly once per call: non-temporal 16-byte loads keep it from
// displacing reusable lines in L2 and stream measurably faster from HBM.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------------------ host
// Launch through hipLaunchKernel so the launch status comes back directly.
// A dispatch counts work-items in 32 bits per dimension: blocks x threads
// must stay below 2^32 (grids are sized in 64 bits and checked here before
// they are narrowed to dim3).
inline bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks > 0 && threads > 0 && blocks <= 0xFFFFFFFFll / threads;
}

template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, Args&&... args) {
  if (!grid_fits(grid.x, block.x) || !grid_fits(grid.y, block.y) || !grid_fits(grid.z, block.z))
    return hipErrorInvalidConfiguration;
  std::tuple<KArgs...> packed(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... a) {
        void* ptrs[] = {(void*)&a...};
        return hipLaunchKernel((const void*)kernel, grid, block, ptrs, lds, stream);
      },
      packed);
}

// Parameters common to the Stage-1 kernels.
struct Stage1Args {
  const void* H;
  int64_t ldh;
  const void* W;
  int64_t ldw;
  int32_t B, D, V;
  float inv_t;          // 1 / T (unused when greedy)
  float score_scale;    // 1 / (T ln 2): token scores are compared in base-2 units (score2)
  int32_t greedy;       // T == 0
  NoiseKey nk;
  int32_t vocab_tile;   // rows per tile
  int32_t n_tiles;
  int32_t batch_tile;   // MFMA: batch rows per workgroup (0: from B)
  uint64_t* cand;       // [n_tiles, B] keys, or null (store-only)
  float* mass;          // [n_tiles, B] tile log-masses of l / T (grouped variant), or null
  void* logits;         // [B, V] logits, or null
  int64_t ld_logits;
  int32_t logits_bf16;  // stored logits dtype
  // single-pass mode: Stage 2 folded into Stage 1
  int32_t single_pass;
  int32_t total_wgs;    // workgroups that publish candidates (set by the launcher)
  uint64_t* keys;       // [B] running maximum keys, zero between calls
  uint32_t* counter;    // finished-workgroup counters (kSpGroups + 1 slots), zero between calls
  int32_t* out;         // [B] tokens
  int32_t half_tiles;   // the last half_tiles vocab tiles hold half a vocab tile of rows each (from the plan)
};

// Stores l[0..3], the logits of batch row b at vocab rows v0 .. v0+3 (those
// below v_end), into the caller's logits buffer in its dtype. Logits are
// written once and read, if at all, by a later kernel: whole 8- or 16-byte
// pieces go out as non-temporal stores (measured: a third of the cost of
// ordinary stores when interleaved with the W stream).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_logits4(const Stage1Args& a, int b, int v0, int v_end, const float (&l)[4]) {
  const int64_t off = (int64_t)b * a.ld_logits + v0;
  if (a.logits_bf16) {
    uint16_t* p = static_cast<uint16_t*>(a.logits) + off;
    if (v0 + 3 < v_end && (off & 3) == 0) {
      const u32x2_t v = {(uint32_t)f32_to_bf16_rne(l[0]) | ((uint32_t)f32_to_bf16_rne(l[1]) << 16),
                         (uint32_t)f32_to_bf16_rne(l[2]) | ((uint32_t)f32_to_bf16_rne(l[3]) << 16)};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
    } else {
      for (int j = 0; j < 4; ++j)
        if (v0 + j < v_end) p[j] = f32_to_bf16_rne(l[j]);
    }
  } else {
    float* p = static_cast<float*>(a.logits) + off;
    if (v0 + 3 < v_end && (off & 3) == 0) {
      const u32x4_t v = {__float_as_uint(l[0]), __float_as_uint(l[1]), __float_as_uint(l[2]), __float_as_uint(l[3])};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
    } else {
      for (int j = 0; j < 4; ++j)
        if (v0 + j < v_end) p[j] = l[j];
    }
  }
}

// Launch index -> (vocab tile, batch tile) for the matrix-core kernels: the
// n_bt batch tiles of one vocab tile get consecutive slots on one XCD
// (workgroup i runs on XCD i mod 8), so the tile of W comes from HBM once and
// is re-read from that XCD's L2. Returns false for padding slots of a grid
// rounded up to a multiple of kXcds.
constexpr int kXcds = 8;

__device__ __forceinline__ bool tile_of(int L, int n_vt, int n_bt, int* vt, int* bt) {
  if (n_bt == 1) {
    *vt = L;
    *bt = 0;
    return L < n_vt;
  }
  const int G = n_vt * n_bt;
  const int per = (G + kXcds - 1) / kXcds;
  const int logical = (L % kXcds) * per + L / kXcds;
  if (logical >= G) return false;
  *vt = logical / n_bt;
  *bt = logical - *vt * n_bt;
  return true;
}

// Single-pass bookkeeping in the workspace after the [B] keys: one counter
// per group of vocab tiles (tile mod kSpGroups) and one for the groups, each
// in its own 256-byte slot (uint32 index kSpSlot * slot).
constexpr int kSpGroups = 32;
constexpr int kSpSlot = 64;

// Publishes one workgroup's best key per batch row (k is meaningful for
// tid < n_rows, rows b0 .. b0 + n_rows - 1; every thread of the workgroup
// must call this).
//  * Two-stage mode: candidate buffer [n_tiles, B], reduced by Stage 2.
//  * Single-pass mode (Stage 2 folded in): a device-scope atomic 64-bit
//    maximum into keys[b], skipped when a relaxed read of keys[b] already
//    holds a key at least as large (the maximum only grows, so the skipped
//    update could not have changed it); this keeps the number of
//    read-modify-writes per key near the number of record-breaking
//    candidates instead of one per workgroup. After its maxima have
//    completed, the workgroup counts itself finished in its group's counter;
//    the last of a group counts the group finished, and the workgroup that
//    finishes the last group decodes keys into tokens and returns keys and
//    counters to zero for the next call. Two levels keep the read-modify-
//    writes on any one counter to about n_workgroups / kSpGroups (one counter
//    for all workgroups serialises them: measured +17 to +31 us per call at
//    B <= 8). Every access to keys and counters is an atomic operation
//    performed where all XCDs see it, and each workgroup's maxima complete
//    before its increment is issued; the chain of increments that the last
//    workgroup's own increment observes therefore orders every maximum
//    before its exchanges, and no cache-flushing fence is needed. The
//    maximum is order independent: results equal the two-stage ones.
__device__ __forceinline__ void publish_candidates(const Stage1Args& a, int tile, int b0, int n_rows,
                                                   uint64_t k, int tid, int nthreads) {
  if (!a.single_pass) {
    if (tid < n_rows) a.cand[(int64_t)tile * a.B + b0 + tid] = k;
    return;
  }
  __shared__ int is_last;
  if (tid < n_rows && k != 0ull) {
    unsigned long long* slot = reinterpret_cast<unsigned long long*>(a.keys + b0 + tid);
    if (k > __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      __hip_atomic_fetch_max(slot, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the maxima have been performed
  __syncthreads();
  if (tid == 0) {
    // workgroups per group: the group's vocab tiles times the batch tiles
    const int g = tile % kSpGroups;
    const int n_bt = a.total_wgs / a.n_tiles;
    const uint32_t in_group = (uint32_t)(((a.n_tiles - g + kSpGroups - 1) / kSpGroups) * n_bt);
    const uint32_t groups = (uint32_t)min(a.n_tiles, kSpGroups);
    int last = 0;
    if (__hip_atomic_fetch_add(a.counter + kSpSlot * g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        in_group - 1)
      last = __hip_atomic_fetch_add(a.counter + kSpSlot * kSpGroups, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == groups - 1;
    is_last = last;
  }
  __syncthreads();
  if (is_last) {
    for (int b = tid; b < a.B; b += nthreads) {
      const uint64_t key = __hip_atomic_exchange(reinterpret_cast<unsigned long long*>(a.keys + b), 0ull,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.out[b] = key_to_token(key);
    }
    if (tid <= kSpGroups)
      __hip_atomic_exchange(a.counter + kSpSlot * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Launchers (each returns the hipError_t of its launches).
hipError_t launch_stage1_gemv(const Stage1Args& a, fs_dtype_t dtype, hipStream_t stream);
int gemv_batch_tile(int64_t B, int64_t D, fs_dtype_t dtype);
hipError_t launch_stage1_mfma(const Stage1Args& a, hipStream_t stream);
hipError_t launch_stage1_tiled(const Stage1Args& a, bool mfma, hipStream_t stream);
// Sampling on tiled W with n_tiles 128-row vocab tiles: how many 64-row tiles
// the last round of workgroups becomes (0: none), for the current device.
int64_t tiled_half_tiles(int64_t n_tiles, int64_t B, int32_t batch_tile);
bool rows_direct_ok(int64_t D);
hipError_t launch_stage1_rows_direct(const Stage1Args& a, hipStream_t stream);
hipError_t launch_stage1_mfma_f32(const Stage1Args& a, hipStream_t stream);
int32_t mfma_f32_tile_rows();
hipError_t launch_pack_tiled(const void* W, int64_t ldw, int32_t V, int32_t D, void* out, hipStream_t stream);
int64_t tiled_weights_bytes(int64_t V, int64_t D);
int mfma_tile_rows(int blocks_per_wave);
hipError_t launch_stage2(const uint64_t* cand, int32_t B, int32_t n_tiles, int32_t* out,
                         hipStream_t stream);
hipError_t launch_stage2_grouped(const uint64_t* cand, const float* mass, int32_t B, int32_t n_tiles,
                                 int32_t tiles_per_group, NoiseKey nk, int32_t* out, hipStream_t stream);
hipError_t launch_sample_logits(const void* logits, int64_t ld, int32_t logits_bf16, int32_t B,
                                int32_t V, float score_scale, int32_t greedy, NoiseKey nk,
                                uint64_t* partial, int32_t* n_parts_out, hipStream_t stream);
hipError_t launch_test_philox(NoiseKey nk, uint32_t b, int64_t v0, int64_t n, uint32_t* out,
                              hipStream_t stream);
hipError_t launch_test_gumbel(const uint32_t* words, int64_t n, float* out, hipStream_t stream);
hipError_t launch_fill_zero(uint64_t* p, int64_t n, hipStream_t stream);
hipError_t launch_probe_read(const void* src, int64_t bytes, int64_t chunk_bytes, uint32_t* sink,
                             hipStream_t stream);

}  // namespace fs
