// Stage 1, small-batch (GEMV) regime: FlashSampling's fused kernel
// (arXiv 2603.15854, Section 3, "Stage 1 (Fused Kernel)") for B up to a few
// rows, where the LM-head product is a matrix-vector stream over W and the
// kernel is bound by reading W from HBM once.
//
// Work decomposition (one workgroup = one vocab tile x one batch tile):
//  * the batch tile's rows of H are staged once in LDS;
//  * each of the 4 waves owns a contiguous quarter of the tile's vocab rows
//    and walks it four rows at a time; every lane reads 16-byte chunks of the
//    four W rows at a fixed stride of 64 chunks, so a wave load covers 1 KiB
//    of one row (fully coalesced) and many loads are in flight per wave;
//  * products use v_dot2 (bf16 pairs, fp32 accumulate) or fp32 FMA;
//  * the 4 x BB partial sums of a row group are reduced across the wave by a
//    transpose-reduce (each exchange step halves the values a lane keeps), so
//    each lane ends holding the full dot product of one (row, batch) pair;
//  * epilogue in registers: l * (1/T) + Gumbel(Philox word) and a running
//    packed-key maximum per batch row; the tile's candidate per batch row is
//    the maximum over the four waves.
// Optional second epilogue: store the logits (the unfused baseline's GEMM
// and the store-logits check of the IO model, Appendix K of the pages).
#include "fs_common.h"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRows = 4;   // vocab rows per group (one Philox call covers them)
constexpr int kJB = 4;     // 16-byte chunks per lane loaded before use (rows longer than 64 chunks)

template <bool BF16>
__device__ __forceinline__ float dot_chunk(const uint4& w, const uint4& h, float acc) {
  if constexpr (BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x),
                                          __builtin_bit_cast(bf16x2, h.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y),
                                          __builtin_bit_cast(bf16x2, h.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z),
                                          __builtin_bit_cast(bf16x2, h.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w),
                                          __builtin_bit_cast(bf16x2, h.w), acc, false);
  } else {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(h.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(h.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(h.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(h.w), acc);
  }
  return acc;
}

template <int N>
struct Log2 {
  static constexpr int value = 1 + Log2<N / 2>::value;
};
template <>
struct Log2<1> {
  static constexpr int value = 0;
};

// Reduce N per-lane partial sums over the 64 lanes of a wave. On return v[0]
// holds the wave-wide sum of value index (lane >> (6 - log2 N)) & (N - 1).
template <int N>
__device__ __forceinline__ float transpose_reduce(float (&v)[N], int lane) {
  constexpr int LOGN = Log2<N>::value;
#pragma unroll
  for (int k = 0; k < LOGN; ++k) {
    const int cnt = N >> k;
    const int half = cnt >> 1;
    const int m = 32 >> k;
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? v[i] : v[i + half];
      const float keep = upper ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, m);
    }
  }
  float x = v[0];
#pragma unroll
  for (int m = 32 >> LOGN; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// JB: 16-byte chunks per lane loaded before use; 1 when a row is at most 64
// chunks (the loop then runs once and a larger JB only costs registers:
// fp32, 8 batch rows, D = 256 went from 1 to 2 waves per SIMD).
template <int BB, int JB, bool BF16, bool SAMPLE, bool STORE>
__global__ __launch_bounds__(kThreads) void stage1_gemv_kernel(Stage1Args a) {
  constexpr int N = kRows * BB;             // partial sums per lane per row group
  constexpr int S = 6 - Log2<N>::value;     // lane bits below the value index
  constexpr int ESZ = BF16 ? 2 : 4;         // element size
  constexpr int EPC = 16 / ESZ;             // elements per 16-byte chunk
  static_assert(N <= 64, "batch tile too large");

  extern __shared__ uint4 lds_h[];          // [BB][D / EPC] chunks of H
  __shared__ uint64_t red[kWaves][BB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile = blockIdx.x;
  const int b0 = blockIdx.y * BB;
  const int nch = a.D / EPC;                // chunks per row
  const int nj = (nch + 63) >> 6;           // chunks per lane per row

  // Stage the batch tile's rows of H (rows past B are zero).
  for (int i = tid; i < BB * nch; i += kThreads) {
    const int b = i / nch;
    const int c = i - b * nch;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (b0 + b < a.B)
      v = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.H) +
                                           ((int64_t)(b0 + b) * a.ldh + (int64_t)c * EPC) * ESZ);
    lds_h[i] = v;
  }
  __syncthreads();

  const int tile_row0 = tile * a.vocab_tile;
  const int tile_end = min(a.V, tile_row0 + a.vocab_tile);
  const int rows_per_wave = a.vocab_tile / kWaves;
  const int wave_row0 = tile_row0 + wave * rows_per_wave;
  const int wave_end = min(tile_end, wave_row0 + rows_per_wave);

  // value index held by this lane after the reduction
  const int vi = (lane >> S) & (N - 1);
  const int my_r = vi & (kRows - 1);
  const int my_b = vi >> 2;
  const int my_batch = b0 + my_b;

  uint64_t best = 0ull;
  const char* Wbase = static_cast<const char*>(a.W);

  for (int row0 = wave_row0; row0 < wave_end; row0 += kRows) {
    const char* wp[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = min(row0 + r, a.V - 1);
      wp[r] = Wbase + (int64_t)row * a.ldw * ESZ;
    }
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;

    // With a power-of-two row stride the rows read at one column offset sit
    // on few memory channels; for power-of-two widths successive row groups
    // therefore take the row's column blocks in rotated order (measured,
    // 4096-wide head: 1.7-2.4% faster at B = 1 and 2; no gain at other
    // widths). Keyed on D, not on the stride, so a padded W sums in the same
    // order as a contiguous one.
    const int nblk = (nj + JB - 1) / JB;
    const int rot = (a.D & (a.D - 1)) == 0 ? (row0 / kRows) % nblk : 0;
    for (int it = 0; it < nblk; ++it) {
      const int j0 = (it + rot < nblk ? it + rot : it + rot - nblk) * JB;
      uint4 w[JB][kRows];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int c = lane + 64 * (j0 + jj);
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          w[jj][r] = make_uint4(0u, 0u, 0u, 0u);
          if (c < nch) w[jj][r] = load_stream16(wp[r] + (int64_t)c * 16);
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int c = lane + 64 * (j0 + jj);
        if (c < nch) {
#pragma unroll
          for (int b = 0; b < BB; ++b) {
            const uint4 h = lds_h[b * nch + c];
#pragma unroll
            for (int r = 0; r < kRows; ++r) acc[b * kRows + r] = dot_chunk<BF16>(w[jj][r], h, acc[b * kRows + r]);
          }
        }
      }
    }

    const float l = transpose_reduce<N>(acc, lane);
    const int row = row0 + my_r;
    const bool valid = row < wave_end && my_batch < a.B;

    if constexpr (STORE) {
      // gather the group's four rows of this batch row into the r == 0 lane
      const float l1 = __shfl_xor(l, 1 << S);
      const float l2 = __shfl_xor(l, 2 << S);
      const float l3 = __shfl_xor(l, 3 << S);
      const bool writer = (lane & ((4 << S) - 1)) == 0 && my_batch < a.B;
      if (writer) {
        static_assert(kRows == 4, "one row group = four consecutive vocab rows");
        const float q[4] = {l, l1, l2, l3};
        store_logits4(a, my_batch, row0, wave_end, q);
      }
    }

    if constexpr (SAMPLE) {
      float s = l;
      if (!a.greedy) {
        const uint4 words = philox_quad(a.nk, (uint32_t)(row0 >> 2), (uint32_t)my_batch);
        s = score2(l, a.score_scale, pick_word(words, my_r));
      }
      const uint64_t key = valid ? pack_key(s, (uint32_t)row) : 0ull;
      best = umax64(best, key);
    }
  }

  if constexpr (SAMPLE) {
    best = umax64(best, shfl_xor_u64(best, 1 << S));
    best = umax64(best, shfl_xor_u64(best, 2 << S));
    if ((lane & ((4 << S) - 1)) == 0) red[wave][lane >> (S + 2)] = best;
    __syncthreads();
    uint64_t k = 0ull;
    if (tid < BB) {
      k = red[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) k = umax64(k, red[w][tid]);
    }
    publish_candidates(a, tile, b0, min(BB, a.B - b0), k, tid, kThreads);
  }
}

template <int BB, int JB, bool BF16>
hipError_t launch_bb_jb(const Stage1Args& a, hipStream_t stream) {
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const dim3 grid(a.n_tiles, (a.B + BB - 1) / BB);
  const size_t lds = (size_t)BB * a.D * (BF16 ? 2 : 4);
  void (*k)(Stage1Args) = nullptr;
  if (sample && store) k = stage1_gemv_kernel<BB, JB, BF16, true, true>;
  else if (sample) k = stage1_gemv_kernel<BB, JB, BF16, true, false>;
  else k = stage1_gemv_kernel<BB, JB, BF16, false, true>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  Stage1Args b = a;
  if ((int64_t)grid.x * grid.y > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // workgroup count is int32
  b.total_wgs = (int32_t)(grid.x * grid.y);
  return launch(k, grid, dim3(kThreads), lds, stream, b);
}

template <int BB, bool BF16>
hipError_t launch_bb(const Stage1Args& a, hipStream_t stream) {
  const int nch = a.D / (BF16 ? 8 : 4);
  return nch <= 64 ? launch_bb_jb<BB, 1, BF16>(a, stream) : launch_bb_jb<BB, kJB, BF16>(a, stream);
}

}  // namespace

// Batch rows per workgroup: the smallest power of two >= B, up to 8 (bf16)
// or 4 (fp32; 2 when a row of H is at most 1 KiB), while the tile of H fits
// 64 KiB of LDS. Larger fp32 tiles hold too many registers: measured on a
// 4096 x 256 fp32 head, B = 64 took 133 us with 8 rows per workgroup, 35
// with 4 and 28 with 2; on 32768 x 1024, 4 rows beat 2 by 16%.
int gemv_batch_tile(int64_t B, int64_t D, fs_dtype_t dtype) {
  const int64_t esz = dtype == FS_DTYPE_BF16 ? 2 : 4;
  const int cap = esz == 2 ? 8 : D * esz <= 1024 ? 2 : 4;
  int bb = 1;
  while (bb < cap && bb < B) bb *= 2;
  while (bb > 1 && bb * D * esz > 65536) bb /= 2;
  return bb;
}

hipError_t launch_stage1_gemv(const Stage1Args& a, fs_dtype_t dtype, hipStream_t stream) {
  const int bb = gemv_batch_tile(a.B, a.D, dtype);
  const bool bf16 = dtype == FS_DTYPE_BF16;
  switch (bb) {
    case 1: return bf16 ? launch_bb<1, true>(a, stream) : launch_bb<1, false>(a, stream);
    case 2: return bf16 ? launch_bb<2, true>(a, stream) : launch_bb<2, false>(a, stream);
    case 4: return bf16 ? launch_bb<4, true>(a, stream) : launch_bb<4, false>(a, stream);
    default: return bf16 ? launch_bb<8, true>(a, stream) : launch_bb<8, false>(a, stream);
  }
}

}  // namespace fs
