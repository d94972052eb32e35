// Stage 1 for fp32 heads on the matrix cores: FlashSampling's fused kernel
// (arXiv 2603.15854, Section 3, "Stage 1 (Fused Kernel)") with fp32 inputs,
// fp32 products and fp32 accumulation (v_mfma_f32_16x16x4_f32), for batches
// past the few rows the GEMV kernel serves well.
//
// Tile: one workgroup = 128 vocab rows (8 waves, one 16-row block each) x
// BN = 16*NB batch rows. Row-major W [V, D] (D a multiple of 4), K blocks of
// 128 columns, K steps of 16:
//  * A operand straight from the rows: lane (r, q) = (lane % 16, lane / 16)
//    loads W[16m + r][128c + 16t + 4q .. +4] (one 16-byte piece; a wave load
//    covers 64 bytes of 16 rows), pieces past D are zero;
//  * the matrix instruction takes one fp32 per lane for each operand, so one
//    16-byte piece feeds four instructions: sub-step j pairs element j of the
//    W piece with element j of the H piece H[n][128c + 16t + 4q .. +4]. The
//    k carried by (lane slot q, sub-step j) is 16t + 4q + j on both sides,
//    so the sum runs over every k of the step exactly once;
//  * H blocks [BN, 128] are staged in LDS, double-buffered, rows padded to
//    544 bytes (an odd multiple of 32: conflict-free 16-byte reads).
// After the product a lane holds four consecutive vocab rows of one batch
// row, as in the bf16 kernels, so the epilogue is theirs: one Philox call per
// lane and batch block, l * (1/T) + Gumbel, running maximum, one key per
// (batch row, vocab tile); or the logits are stored.
#include "fs_common.h"

namespace fs {
namespace {

constexpr int kNW = 8;                  // waves: vocab tile = 128 rows
constexpr int kKB = 128;                // columns per K block
constexpr int kKS = kKB / 16;           // K steps per block (one 16-byte piece per lane each)
constexpr int kRow = kKB + 8;           // padded H row in LDS (floats)

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(const float4& w, const float4& h, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, h.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, h.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, h.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.w, h.w, c, 0, 0, 0);
  return c;
}

template <int NB, bool SAMPLE, bool STORE>
__global__ __launch_bounds__(64 * kNW) void mfma_f32_kernel(Stage1Args a, int32_t n_bt) {
  constexpr int BN = 16 * NB;
  constexpr int NT = 64 * kNW;
  constexpr int HP = BN * (kKB / 4) / NT;   // 16-byte pieces of H per thread per block
  static_assert(HP >= 1 && HP * NT == BN * (kKB / 4), "batch tile vs workgroup size");

  __shared__ float4 lds_h4[2 * BN * kRow / 4];
  __shared__ uint64_t red[kNW][BN];
  float* lds_h = reinterpret_cast<float*>(lds_h4);

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int b0 = bt * BN;
  const int D = a.D;
  const int nC = (D + kKB - 1) / kKB;
  const int m = vt * kNW + wave;
  // rows past V read the last row (their candidates are never valid)
  const float* wrow = static_cast<const float*>(a.W) + (int64_t)min(16 * m + r, a.V - 1) * a.ldw + 4 * q;
  auto wload = [&](int c, int t) {
    const int k = c * kKB + 16 * t + 4 * q;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < D) v = *reinterpret_cast<const float4*>(wrow + c * kKB + 16 * t);
    return v;
  };
  const float* H = static_cast<const float*>(a.H);

  int hn[HP], hk[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = tid + NT * i;
    hn[i] = p / (kKB / 4);
    hk[i] = 4 * (p % (kKB / 4));
  }
  auto load_h = [&](int c, float4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const int k = c * kKB + hk[i];
      h[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (b0 + hn[i] < a.B && k < D) h[i] = *reinterpret_cast<const float4*>(H + (int64_t)(b0 + hn[i]) * a.ldh + k);
    }
  };
  auto store_h = [&](int buf, const float4 (&h)[HP]) {
#pragma unroll
    for (int i = 0; i < HP; ++i)
      *reinterpret_cast<float4*>(lds_h + buf * BN * kRow + hn[i] * kRow + hk[i]) = h[i];
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Rolling prefetch as in the bf16 kernels: the register of K step t is
  // reloaded with step t of the next block once its products are issued.
  float4 w[kKS];
  float4 hreg[HP];
#pragma unroll
  for (int t = 0; t < kKS; ++t) w[t] = wload(0, t);
  load_h(0, hreg);
  store_h(0, hreg);
  __syncthreads();

  for (int c = 0; c < nC; ++c) {
    const bool more = c + 1 < nC;
    if (more) load_h(c + 1, hreg);
    const float* hb = lds_h + (c & 1) * BN * kRow;
#pragma unroll
    for (int t = 0; t < kKS; ++t) {
      const float4 x = w[t];
      if (more) w[t] = wload(c + 1, t);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float4 h = *reinterpret_cast<const float4*>(hb + (nb * 16 + r) * kRow + 16 * t + 4 * q);
        acc[nb] = mfma4(x, h, acc[nb]);
      }
    }
    if (more) {
      store_h((c + 1) & 1, hreg);
      __syncthreads();
    }
  }

  const int v0 = 16 * m + 4 * q;   // this lane's four consecutive vocab rows
  if constexpr (STORE) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = b0 + nb * 16 + r;
      const float l[4] = {acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]};
      if (b < a.B && v0 < a.V) store_logits4(a, b, v0, a.V, l);
    }
  }
  if constexpr (SAMPLE) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = b0 + nb * 16 + r;
      uint4 words = make_uint4(0u, 0u, 0u, 0u);
      if (!a.greedy) words = philox_quad(a.nk, (uint32_t)(v0 >> 2), (uint32_t)b);
      RunMax best = runmax_init();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float l = acc[nb][j];
        const float s = a.greedy ? l : score2(l, a.score_scale, pick_word(words, j));
        if (v0 + j < a.V) runmax_take(best, s, v0 + j);
      }
      uint64_t key = runmax_key(best);
      key = umax64(key, shfl_xor_u64(key, 16));
      key = umax64(key, shfl_xor_u64(key, 32));
      if (q == 0) red[wave][nb * 16 + r] = key;
    }
    __syncthreads();
    uint64_t k = 0ull;
    if (tid < BN) {
      k = red[0][tid];
#pragma unroll
      for (int w2 = 1; w2 < kNW; ++w2) k = umax64(k, red[w2][tid]);
    }
    publish_candidates(a, vt, b0, min(BN, a.B - b0), k, tid, NT);
  }
}

template <int NB>
hipError_t launch_nb(const Stage1Args& a, hipStream_t stream) {
  constexpr int BN = 16 * NB;
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const int n_bt = (a.B + BN - 1) / BN;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  void (*k)(Stage1Args, int32_t) = nullptr;
  if (sample && store) k = mfma_f32_kernel<NB, true, true>;
  else if (sample) k = mfma_f32_kernel<NB, true, false>;
  else k = mfma_f32_kernel<NB, false, true>;
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  return launch(k, dim3((unsigned)grid), dim3(64 * kNW), 0, stream, b, (int32_t)n_bt);
}

}  // namespace

int32_t mfma_f32_tile_rows() { return 16 * kNW; }

// Batch tile 16, 32 or 64 columns: the smallest that holds B, 64 above.
hipError_t launch_stage1_mfma_f32(const Stage1Args& a, hipStream_t stream) {
  const int bn = a.batch_tile ? a.batch_tile : (a.B <= 16 ? 16 : a.B <= 32 ? 32 : 64);
  if (bn == 16) return launch_nb<1>(a, stream);
  if (bn == 32) return launch_nb<2>(a, stream);
  return launch_nb<4>(a, stream);
}

}  // namespace fs
