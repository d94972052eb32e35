// Stage 2 of FlashSampling (arXiv 2603.15854, Section 3, "Stage 2
// (Reduction)"): per batch row, the maximum of the packed candidate keys over
// the vocab tiles, decoded to a token; the grouped variant's Stage 2 (group
// log-masses, the group draw, the chosen group's local sample). Also the
// unfused baseline's sampler
// (Gumbel-max over logits read back from device memory; the "sample from the
// logits" step of the same section's IO model) and the noise test hooks.
#include <type_traits>

#include "fs_common.h"

namespace fs {
namespace {

constexpr int kThreads = 256;

// Launch index -> batch row. The candidates of rows b .. b+15 for one tile
// share a 128-byte line, and workgroup L runs on XCD L mod kXcds; consecutive
// rows therefore get consecutive slots on one XCD, so each line is brought
// into one or two XCDs' L2 rather than into up to eight (measured on the
// 7168 x 129280 head at B = 1024: 6.6 us against 8.6 with one row per slot
// in order; 5.2-5.3 against 5.5-5.6 at B = 64 and 256). The grid is
// row_grid(B); returns false for its padding slots.
__device__ __forceinline__ bool row_of(int L, int B, int* row) {
  const int per = (B + kXcds - 1) / kXcds;
  *row = (L % kXcds) * per + L / kXcds;
  return *row < B;
}
unsigned row_grid(int32_t B) { return B <= kXcds ? (unsigned)B : (unsigned)((B + kXcds - 1) / kXcds * kXcds); }

// One workgroup per batch row; each lane folds its keys with four
// independent loads in flight, so a row of candidates costs about one memory
// round trip. 256 lanes cover up to 1024 tiles per round; rows with many
// more tiles (small vocab tiles) use 1024 lanes.
template <int NT>
__global__ __launch_bounds__(NT) void stage2_kernel(const uint64_t* __restrict__ cand, int32_t n_tiles,
                                                    int32_t B, int32_t* __restrict__ out) {
  __shared__ uint64_t red[NT / 64];
  int row;
  if (!row_of(blockIdx.x, B, &row)) return;  // whole workgroup
  const uint64_t* c = cand + row;   // candidate of tile t at c[t * B]
  uint64_t best = 0ull;
  for (int t0 = threadIdx.x; t0 < n_tiles; t0 += 4 * NT) {
    uint64_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * NT;
      k[u] = t < n_tiles ? c[(int64_t)t * B] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) best = umax64(best, k[u]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best = umax64(best, shfl_xor_u64(best, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x < 64) {
    uint64_t k = threadIdx.x < NT / 64 ? red[threadIdx.x] : 0ull;
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) k = umax64(k, shfl_xor_u64(k, m));
    if (threadIdx.x == 0) out[row] = key_to_token(k);
  }
}

// Stage 2 of the grouped variant, one workgroup per batch row: group g is the
// run of tiles [g tpg, (g+1) tpg). Each group's tiles are folded into its best
// key (the local sample) and log-mass; the group is scored t_g = mass_g + h_g
// with the group noise, and the largest (t_g, lowest g) key wins; that
// group's local sample is the token. Few large groups (tpg >= 16): a wave per
// group, lanes over its tiles, shuffle reductions. Many small groups: a
// thread per group, walking its tiles.
template <int NT>
__global__ __launch_bounds__(NT) void stage2_grouped_kernel(const uint64_t* __restrict__ cand,
                                                            const float* __restrict__ mass, int32_t n_tiles,
                                                            int32_t B, int32_t tpg, NoiseKey nk,
                                                            int32_t* __restrict__ out) {
  constexpr int NW = NT / 64;
  __shared__ uint64_t red_t[NT];
  __shared__ uint64_t red_k[NT];
  int row;
  if (!row_of(blockIdx.x, B, &row)) return;  // whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_groups = (n_tiles + tpg - 1) / tpg;
  uint64_t best_t = 0ull, best_key = 0ull;
  auto score_group = [&](int g, uint64_t key, float m, float s) {
    const float score = lse_value(m, s) + group_gumbel(nk, (uint32_t)g, (uint32_t)row);
    const uint64_t tk = pack_key(score, (uint32_t)g);
    if (tk > best_t) {
      best_t = tk;
      best_key = key;
    }
  };
  if (tpg >= 16) {
    for (int g = wave; g < n_groups; g += NW) {   // uniform per wave
      const int t1 = min(n_tiles, (g + 1) * tpg);
      uint64_t key = 0ull;
      float m = -__builtin_inff(), s = 0.f;
      for (int t = g * tpg + lane; t < t1; t += 64) {
        key = umax64(key, cand[(int64_t)t * B + row]);
        lse_merge(m, s, mass[(int64_t)t * B + row], 1.0f);   // e^mass_t as the pair (mass_t, 1)
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        key = umax64(key, shfl_xor_u64(key, off));
        lse_merge(m, s, __shfl_xor(m, off), __shfl_xor(s, off));
      }
      if (lane == 0) score_group(g, key, m, s);
    }
  } else {
    for (int g = tid; g < n_groups; g += NT) {
      const int t1 = min(n_tiles, (g + 1) * tpg);
      uint64_t key = 0ull;
      float m = -__builtin_inff(), s = 0.f;
      for (int t = g * tpg; t < t1; ++t) {
        key = umax64(key, cand[(int64_t)t * B + row]);
        lse_merge(m, s, mass[(int64_t)t * B + row], 1.0f);
      }
      score_group(g, key, m, s);
    }
  }
  red_t[tid] = best_t;
  red_k[tid] = best_key;
  __syncthreads();
  for (int w = NT / 2; w >= 1; w >>= 1) {
    if (tid < w && red_t[tid + w] > red_t[tid]) {
      red_t[tid] = red_t[tid + w];
      red_k[tid] = red_k[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) out[row] = key_to_token(red_k[0]);
}

// Gumbel-max over materialised logits: workgroup (part, row) scans `part` =
// IT * 2048 consecutive vocab entries of one row, eight per thread per
// chunk: every chunk's 16- or 32-byte load is issued before any arithmetic
// (IT chunks in flight per thread), then two Philox calls per chunk (one per
// four entries), and the workgroup's best key goes to partial[part, row].
// Rows are ld >= V entries apart with ld a multiple of 8, so a chunk that
// starts below V lies inside its row; entries past V are never candidates.
template <bool BF16, int IT>
__global__ __launch_bounds__(kThreads) void sample_logits_kernel(
    const void* __restrict__ logits, int64_t ld, int32_t V, float score_scale, int32_t greedy,
    NoiseKey nk, int32_t part, uint64_t* __restrict__ partial) {
  constexpr int LOADS = BF16 ? 1 : 2;   // 16-byte loads per chunk of 8 entries
  __shared__ uint64_t red[kThreads / 64];
  const int row = blockIdx.y;
  const int v_begin = blockIdx.x * part;
  uint4 raw[IT][LOADS];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int v = v_begin + (it * kThreads + (int)threadIdx.x) * 8;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      raw[it][u] = make_uint4(0u, 0u, 0u, 0u);
      if (v < V) {
        const char* p = static_cast<const char*>(logits) + ((int64_t)row * ld + v) * (BF16 ? 2 : 4);
        raw[it][u] = load_stream16(p + 16 * u);
      }
    }
  }
  uint64_t best = 0ull;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int v = v_begin + (it * kThreads + (int)threadIdx.x) * 8;
    float l[8];
    if (BF16) {
      const uint4 q = raw[it][0];
      l[0] = bf16_lo(q.x); l[1] = bf16_hi(q.x); l[2] = bf16_lo(q.y); l[3] = bf16_hi(q.y);
      l[4] = bf16_lo(q.z); l[5] = bf16_hi(q.z); l[6] = bf16_lo(q.w); l[7] = bf16_hi(q.w);
    } else {
      const uint4 q0 = raw[it][0], q1 = raw[it][LOADS - 1];
      l[0] = __uint_as_float(q0.x); l[1] = __uint_as_float(q0.y); l[2] = __uint_as_float(q0.z);
      l[3] = __uint_as_float(q0.w); l[4] = __uint_as_float(q1.x); l[5] = __uint_as_float(q1.y);
      l[6] = __uint_as_float(q1.z); l[7] = __uint_as_float(q1.w);
    }
    if (v < V) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 words = make_uint4(0u, 0u, 0u, 0u);
        if (!greedy) words = philox_quad(nk, (uint32_t)((v >> 2) + h), (uint32_t)row);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * h + j;
          const float sc = greedy ? l[e] : score2(l[e], score_scale, pick_word(words, j));
          if (v + e < V) best = umax64(best, pack_key(sc, (uint32_t)(v + e)));
        }
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best = umax64(best, shfl_xor_u64(best, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t k = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) k = umax64(k, red[w]);
    partial[(int64_t)blockIdx.x * gridDim.y + row] = k;
  }
}

__global__ __launch_bounds__(kThreads) void test_philox_kernel(NoiseKey nk, uint32_t b, int64_t v0,
                                                               int64_t n, uint32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const int64_t v = v0 + i;
  const uint4 w = philox_quad(nk, (uint32_t)(v >> 2), b);
  out[i] = pick_word(w, (int)(v & 3));
}

__global__ __launch_bounds__(kThreads) void test_gumbel_kernel(const uint32_t* words, int64_t n,
                                                               float* out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  out[i] = gumbel_from_word(words[i]);
}

// Streams `bytes` from src with 16-byte loads and folds them into one word per
// workgroup: the attainable read bandwidth for a W-sized buffer, and a kernel
// of exactly known HBM read traffic for counter calibration. Workgroup g reads
// the contiguous range [g * chunk, (g + 1) * chunk).
template <int U>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                              int64_t chunk16, uint32_t* __restrict__ sink) {
  const int64_t begin = (int64_t)blockIdx.x * chunk16;
  const int64_t end = min(n16, begin + chunk16);
  uint32_t x = 0;
  for (int64_t i = begin + threadIdx.x; i < end; i += (int64_t)kThreads * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * kThreads;
      v[u] = j < end ? load_stream16(src + j) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint64_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    p[i] = 0ull;
}

}  // namespace

hipError_t launch_fill_zero(uint64_t* p, int64_t n, hipStream_t stream) {
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  return launch(fill_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(kThreads), 0, stream, p, n);
}

hipError_t launch_probe_read(const void* src, int64_t bytes, int64_t chunk_bytes, uint32_t* sink,
                             hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t chunk16 = chunk_bytes / 16;
  if ((n16 + chunk16 - 1) / chunk16 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((n16 + chunk16 - 1) / chunk16));
  return launch(probe_read_kernel<8>, grid, dim3(kThreads), 0, stream, static_cast<const uint4*>(src), n16,
                chunk16, sink);
}

hipError_t launch_stage2(const uint64_t* cand, int32_t B, int32_t n_tiles, int32_t* out,
                         hipStream_t stream) {
  if (n_tiles <= 4 * 256)
    return launch(stage2_kernel<256>, dim3(row_grid(B)), dim3(256), 0, stream, cand, n_tiles, B, out);
  return launch(stage2_kernel<1024>, dim3(row_grid(B)), dim3(1024), 0, stream, cand, n_tiles, B, out);
}

hipError_t launch_stage2_grouped(const uint64_t* cand, const float* mass, int32_t B, int32_t n_tiles,
                                 int32_t tiles_per_group, NoiseKey nk, int32_t* out, hipStream_t stream) {
  return launch(stage2_grouped_kernel<256>, dim3(row_grid(B)), dim3(256), 0, stream, cand, mass, n_tiles, B,
                tiles_per_group, nk, out);
}

// Chunks per thread: as many as keep about 1024 workgroups or more over the
// whole call (four per CU), up to eight 16-byte loads per thread in flight.
// Returns the number of parts used (at most ceil(V / 2048)).
hipError_t launch_sample_logits(const void* logits, int64_t ld, int32_t logits_bf16, int32_t B,
                                int32_t V, float score_scale, int32_t greedy, NoiseKey nk,
                                uint64_t* partial, int32_t* n_parts_out, hipStream_t stream) {
  const int64_t chunks2048 = ((int64_t)V + 2047) / 2048 * B;   // 2048-entry pieces over all rows
  int it = 1;
  while (it < 8 && chunks2048 / (2 * it) >= 1024) it *= 2;
  const int32_t part = 2048 * it;
  const int32_t n_parts = (V + part - 1) / part;
  *n_parts_out = n_parts;
  const dim3 grid(n_parts, B);
  auto go = [&](auto bf16_c, auto it_c) {
    constexpr bool kBF16 = decltype(bf16_c)::value;
    constexpr int kIT = decltype(it_c)::value;
    return launch(sample_logits_kernel<kBF16, kIT>, grid, dim3(kThreads), 0, stream, logits, ld, V, score_scale,
                  greedy, nk, part, partial);
  };
  auto by_it = [&](auto bf16_c) {
    switch (it) {
      case 1: return go(bf16_c, std::integral_constant<int, 1>{});
      case 2: return go(bf16_c, std::integral_constant<int, 2>{});
      case 4: return go(bf16_c, std::integral_constant<int, 4>{});
      default: return go(bf16_c, std::integral_constant<int, 8>{});
    }
  };
  return logits_bf16 ? by_it(std::true_type{}) : by_it(std::false_type{});
}

hipError_t launch_test_philox(NoiseKey nk, uint32_t b, int64_t v0, int64_t n, uint32_t* out,
                              hipStream_t stream) {
  if ((n + kThreads - 1) / kThreads > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
  return launch(test_philox_kernel, grid, dim3(kThreads), 0, stream, nk, b, v0, n, out);
}

hipError_t launch_test_gumbel(const uint32_t* words, int64_t n, float* out, hipStream_t stream) {
  if ((n + kThreads - 1) / kThreads > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
  return launch(test_gumbel_kernel, grid, dim3(kThreads), 0, stream, words, n, out);
}

}  // namespace fs
