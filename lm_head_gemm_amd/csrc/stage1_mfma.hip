// Stage 1, matrix-core regime: FlashSampling's fused kernel (arXiv
// 2603.15854, Section 3, "Stage 1 (Fused Kernel)") on CDNA4 bf16 MFMA, for
// batches large enough that the LM-head product is a real contraction.
// Serves row-major W whose D is not a multiple of 256; for the others the
// tiled-layout kernels read the rows directly (stage1_tiled.hip), which keeps
// four times as many waves resident.
//
// Tile: one workgroup = BM vocab rows x BN batch rows; 4 waves, each owning
// 16*MB consecutive vocab rows and all BN batch rows. The product is
// C[v, b] = sum_d W[v, d] H[b, d] with vocab on the MFMA M axis, so after
// v_mfma_f32_16x16x32_bf16 a lane holds four consecutive vocab rows of one
// batch row: exactly the four words of one Philox4x32-10 call.
//
// Data flow per K chunk of 256:
//  * W is read from HBM with coalesced non-temporal loads (one wave load =
//    512 contiguous bytes of each of two rows), one chunk ahead of the math,
//    so each W byte is read exactly once; the wave then transposes its own
//    rows through a private LDS region (16-byte pieces XOR-swizzled by row,
//    conflict-free on both sides) into the MFMA A layout. Reading W directly
//    in the A layout (64 bytes of 16 rows per load) streams measurably
//    slower from HBM than whole 512-byte row pieces;
//  * the H chunk [BN, 256] is staged by the whole workgroup into LDS (rows
//    padded by 16 bytes so the B-operand reads are bank-conflict free),
//    double-buffered, and shared by the four waves.
// Epilogue in registers: l * (1/T) + Gumbel, packed-key maximum per batch
// row over the wave's rows, then over the waves through LDS; one candidate
// per (batch row, vocab tile). Optionally the logits are stored instead of
// or besides sampling (the unfused baseline's GEMM and the IO-model check).
//
// Large batches are split into batch tiles; workgroups that share a vocab
// tile get consecutive slots on the same XCD so the tile of W is fetched
// from HBM once and re-read from that XCD's L2.
#include "fs_common.h"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKS = 8;               // MFMA K steps (of 32) per K chunk
constexpr int kBK = 32 * kKS;        // 256
// padded H row in LDS (elements): a stride of an odd multiple of 32 bytes reads conflict-free
constexpr int kLdsRow = kBK + 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int NB, int MB, bool SAMPLE, bool STORE>
__global__ __launch_bounds__(kThreads, 2) void stage1_mfma_kernel(Stage1Args a, int32_t n_bt) {
  constexpr int BN = 16 * NB;
  constexpr int BM = kWaves * 16 * MB;
  constexpr int WROWS = 16 * MB;                        // vocab rows per wave
  constexpr int WLOADS = WROWS / 2;                     // W loads per lane per chunk
  constexpr int HPIECES = BN * (kBK / 8) / kThreads;   // 16-byte pieces of H per thread per chunk
  static_assert(HPIECES >= 1, "batch tile too small");

  __shared__ uint4 lds_h4[2 * BN * kLdsRow / 8];
  __shared__ uint4 lds_w4[kWaves * WROWS * (kBK / 8)];  // per-wave transpose regions
  __shared__ uint64_t red[kWaves][BN];
  uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_h4);

  int vt, bt;
  if (!tile_of(blockIdx.x, a.n_tiles, n_bt, &vt, &bt)) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int row0 = vt * BM + wave * WROWS;   // first vocab row of this wave
  const int b0 = bt * BN;
  const int D = a.D;
  const int nchunk = (D + kBK - 1) / kBK;

  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  const uint16_t* H = static_cast<const uint16_t*>(a.H);
  uint4* wl = lds_w4 + wave * WROWS * (kBK / 8);

  // load i of a chunk covers rows 2i (lanes 0..31) and 2i+1 (lanes 32..63)
  const int lrow = lane >> 5;
  const int piece = lane & 31;
  const uint16_t* wsrc[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i)
    wsrc[i] = W + (int64_t)min(row0 + 2 * i + lrow, a.V - 1) * a.ldw + 8 * piece;

  auto load_w = [&](int c, uint4 (&w)[WLOADS]) {
    const int k = c * kBK + 8 * piece;
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      w[i] = make_uint4(0u, 0u, 0u, 0u);
      if (k < D) w[i] = load_stream16(wsrc[i] + c * kBK);
    }
  };
  // slot of 16-byte piece p of wave-local row rho: p ^ (rho & 15)
  auto store_w = [&](const uint4 (&w)[WLOADS]) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int rho = 2 * i + lrow;
      wl[rho * (kBK / 8) + (piece ^ (rho & 15))] = w[i];
    }
  };
  auto load_h = [&](int c, uint4 (&h)[HPIECES]) {
#pragma unroll
    for (int i = 0; i < HPIECES; ++i) {
      const int p = tid + kThreads * i;
      const int n = p / (kBK / 8);
      const int k = c * kBK + 8 * (p % (kBK / 8));
      h[i] = make_uint4(0u, 0u, 0u, 0u);
      if (b0 + n < a.B && k < D) h[i] = *reinterpret_cast<const uint4*>(H + (int64_t)(b0 + n) * a.ldh + k);
    }
  };
  auto store_h = [&](int buf, const uint4 (&h)[HPIECES]) {
#pragma unroll
    for (int i = 0; i < HPIECES; ++i) {
      const int p = tid + kThreads * i;
      const int n = p / (kBK / 8);
      const int kk = 8 * (p % (kBK / 8));
      *reinterpret_cast<uint4*>(lds_h + buf * BN * kLdsRow + n * kLdsRow + kk) = h[i];
    }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two register sets for W alternate between "in flight" and "being
  // transposed", so the loads of chunk c+1 stay outstanding during chunk c.
  uint4 wa[WLOADS], wb[WLOADS];
  uint4 hreg[HPIECES];
  load_h(0, hreg);
  store_h(0, hreg);
  load_w(0, wa);
  __syncthreads();

  auto step = [&](int c, uint4 (&wcur)[WLOADS], uint4 (&wnext)[WLOADS]) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunk;
    if (more) {
      // H first: its registers are needed (for the LDS store) before the
      // next chunk of W, and loads complete in issue order
      load_h(c + 1, hreg);
      load_w(c + 1, wnext);
    }
    // the wave's own region: its previous reads were issued before these
    // writes and LDS operations of one wave execute in order
    store_w(wcur);
    const uint16_t* hb = lds_h + buf * BN * kLdsRow;
#pragma unroll
    for (int t = 0; t < kKS; ++t) {
      uint4 afrag[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int rho = 16 * mb + r;
        afrag[mb] = wl[rho * (kBK / 8) + ((4 * t + q) ^ (rho & 15))];
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 bfrag = *reinterpret_cast<const uint4*>(hb + (nb * 16 + r) * kLdsRow + 32 * t + 8 * q);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma16x16x32(afrag[mb], bfrag, acc[mb][nb]);
      }
    }
    if (more) store_h(buf ^ 1, hreg);
    __syncthreads();
  };
  for (int c = 0; c < nchunk; c += 2) {
    step(c, wa, wb);
    if (c + 1 < nchunk) step(c + 1, wb, wa);
  }

  // ---------------------------------------------------------------- epilogue
  const int tile_end = min(a.V, vt * BM + BM);
  if constexpr (STORE) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = b0 + nb * 16 + r;
      if (b >= a.B) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int v0 = row0 + 16 * mb + 4 * q;
        const float l[4] = {acc[mb][nb][0], acc[mb][nb][1], acc[mb][nb][2], acc[mb][nb][3]};
        store_logits4(a, b, v0, tile_end, l);
      }
    }
  }

  if constexpr (SAMPLE) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = b0 + nb * 16 + r;
      uint64_t best = 0ull;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int v0 = row0 + 16 * mb + 4 * q;
        uint4 words = make_uint4(0u, 0u, 0u, 0u);
        if (!a.greedy) words = philox_quad(a.nk, (uint32_t)(v0 >> 2), (uint32_t)b);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float l = acc[mb][nb][j];
          const float s = a.greedy ? l : score2(l, a.score_scale, pick_word(words, j));
          const bool valid = v0 + j < tile_end && b < a.B;
          best = umax64(best, valid ? pack_key(s, (uint32_t)(v0 + j)) : 0ull);
        }
      }
      best = umax64(best, shfl_xor_u64(best, 16));
      best = umax64(best, shfl_xor_u64(best, 32));
      if (q == 0) red[wave][nb * 16 + r] = best;
    }
    __syncthreads();
    uint64_t k = 0ull;
    if (tid < BN) {
      k = red[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) k = umax64(k, red[w][tid]);
    }
    publish_candidates(a, vt, b0, min(BN, a.B - b0), k, tid, kThreads);
  }
}

template <int NB, int MB>
hipError_t launch_nb(const Stage1Args& a, hipStream_t stream) {
  constexpr int BN = 16 * NB;
  const bool sample = a.cand != nullptr;
  const bool store = a.logits != nullptr;
  const int n_bt = (a.B + BN - 1) / BN;
  const int64_t G = (int64_t)a.n_tiles * n_bt;
  const int64_t grid = n_bt == 1 ? G : (G + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;   // launch() checks grid x threads
  void (*k)(Stage1Args, int32_t) = nullptr;
  if (sample && store) k = stage1_mfma_kernel<NB, MB, true, true>;
  else if (sample) k = stage1_mfma_kernel<NB, MB, true, false>;
  else k = stage1_mfma_kernel<NB, MB, false, true>;
  Stage1Args b = a;
  b.total_wgs = (int32_t)G;
  return launch(k, dim3((unsigned)grid), dim3(kThreads), 0, stream, b, (int32_t)n_bt);
}

template <int MB>
hipError_t launch_mb(const Stage1Args& a, hipStream_t stream) {
  const int bn = a.batch_tile ? a.batch_tile : (a.B <= 16 ? 16 : a.B <= 32 ? 32 : 64);
  if (bn == 16) return launch_nb<1, MB>(a, stream);
  if (bn == 32) return launch_nb<2, MB>(a, stream);
  return launch_nb<4, MB>(a, stream);
}

}  // namespace

// Vocab rows per MFMA workgroup for a given number of 16-row blocks per wave.
int mfma_tile_rows(int mb) { return kWaves * 16 * mb; }

hipError_t launch_stage1_mfma(const Stage1Args& a, hipStream_t stream) {
  if (a.vocab_tile == mfma_tile_rows(1)) return launch_mb<1>(a, stream);
  return launch_mb<2>(a, stream);
}

}  // namespace fs
