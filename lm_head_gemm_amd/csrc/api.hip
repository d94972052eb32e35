// C ABI of libflashsample: argument validation, Stage-1 variant and tile
// selection, workspace layout and kernel launches. Nothing here allocates
// device memory; every launch goes on the caller's stream.
#include <cmath>
#include <cstring>
#include <mutex>

#include "fs_common.h"

// Workspace of fs_sample_fused_noalloc: a static device array, one copy per
// GPU at that GPU's own address. Host code never uses this name as an
// address (on the host it is only a stand-in); it takes the device address
// from hipGetSymbolAddress once per device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[FS_NOALLOC_SCRATCH_BYTES];

namespace fs {
namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxB = 65536;
constexpr int64_t kMaxV = 0x7FFFFFFF;       // tokens are int32
constexpr int64_t kMaxD = 1 << 20;
constexpr int32_t kGemvGranule = 16;        // 4 waves x 4-row groups
constexpr int32_t kGemvDefaultTile = 16;
constexpr int32_t kGemvLargeBTile = 64;     // row-major GEMV above kGemvSmallB rows (fp32 heads)
constexpr int64_t kGemvSmallB = 8;
constexpr int32_t kMfmaGranule = 64;
constexpr int32_t kTiledGemvTile = 128;    // tiled layout: 8 waves x 16 rows
constexpr int32_t kTiledMfmaTile = 128;     // tiled layout: 8 waves x 16 rows
constexpr int32_t kTiledWideTile = 256;     // tiled layout: 8 waves x 2 x 16 rows
constexpr int32_t kTiledWideBatch = 128;    // batch tile of the wide kernel
constexpr int32_t kTiledBigBatch = 256;     // opt-in 256 x 256 tile (tiled, sampling only)
constexpr int64_t kTiledWideMinB = 65;      // batches from here on use the wide kernel
constexpr int32_t kMfmaSmallBTile = 64;    // LDS-transposing kernel: one 16-row block per wave
constexpr int32_t kMfmaLargeBTile = 128;    // two blocks per wave above 32 rows
constexpr int32_t kRowsTile = 128;          // row-direct kernel (D a multiple of 256): 8 waves x 16 rows
constexpr int64_t kGemvMaxB = 2;            // batches above this use the MFMA kernels
// Row-major bf16 heads of hidden size kGemvLongRowD and more use 256-row GEMV
// tiles up to kGemvMaxB rows (one workgroup's two H rows fill at most 32 KiB of
// LDS). Measured, fused call per step, 8192 x 128256 head, B <= 2: 310-314 us
// against 344-348 with 16-row tiles.
constexpr int64_t kGemvLongRowD = 8192;
constexpr int32_t kGemvLongTile = 256;
constexpr int32_t kSamplePart = 2048;       // unfused sampler: smallest part of a row per workgroup
constexpr size_t kAlign = 256;
// The GEMV kernels stage whole H rows in LDS (160 KiB per workgroup) next to
// their own reduction arrays (under 1 KiB).
constexpr int64_t kMaxHRowBytes = 159 * 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t dtype_size(fs_dtype_t t) { return t == FS_DTYPE_BF16 ? 2 : 4; }

bool dtype_ok(int t) { return t == FS_DTYPE_BF16 || t == FS_DTYPE_F32; }

bool sizes_ok(int64_t B, int64_t D, int64_t V) {
  return B > 0 && D > 0 && V > 0 && B <= kMaxB && D <= kMaxD && V <= kMaxV;
}

fs_status_t fail_hip(hipError_t e) {
  g_last_hip_error = (int)e;
  return FS_ERR_HIP;
}

struct Plan {
  fs_variant_t variant;
  int32_t tile;
  int64_t n_tiles;
  int32_t batch_tile = 0;
  bool tiled = false;     // W in the tiled layout
  bool single_pass = false;
  int32_t group_size = 0; // > 0: grouped variant
  int64_t half_tiles = 0; // the last half_tiles of the n_tiles vocab tiles hold 64 rows each
};

struct FusedCall {
  Plan plan;
  Stage1Args args;
  size_t ws_bytes = 0;    // workspace bytes the call uses
  bool grouped = false;   // Stage 2 of the grouped variant
};

// Picks the Stage-1 kernel family and vocab tile. Returns false on invalid options.
//   Row-major W: GEMV for batches up to kGemvMaxB rows (vocab tile: multiple
//     of 16 rows; 256 on bf16 heads at least kGemvLongRowD wide), MFMA above:
//     bf16 with D a multiple of 256 the row-direct kernel (128 rows) up to 64
//     rows and the wide kernel (256 rows) from 65 on; other D the
//     LDS-transposing kernel (64 or 128 rows); fp32 the fp32 matrix-core
//     kernel (128 rows).
//   Tiled W (bf16): MFMA at every B (GEMV when asked for); vocab tile 64 or
//     128 rows (4 or 8 waves of one 16-row block each), and from 65 rows on
//     the 256-row wide tile (8 waves of two blocks, batch tile 128 or 256).
//   group_size > 0 (grouped variant): the MFMA kernels with the log-mass
//     epilogue; groups must be unions of vocab tiles.
bool make_plan(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype, const fs_options_t* o, Plan* p,
               fs_status_t* why) {
  *why = FS_ERR_INVALID_ARGUMENT;
  const int layout = o ? o->weights_layout : FS_LAYOUT_ROWS;
  if (layout != FS_LAYOUT_ROWS && layout != FS_LAYOUT_TILED) return false;
  if (o && o->reserved != 0) return false;
  const int32_t group_size = o ? o->group_size : 0;
  if (group_size < 0) return false;
  int variant = o ? o->variant : FS_VARIANT_AUTO;
  if (variant != FS_VARIANT_AUTO && variant != FS_VARIANT_GEMV && variant != FS_VARIANT_MFMA) return false;
  if (group_size > 0) {
    // the grouped variant: bf16, tiled weights or row-major ones with D a
    // multiple of 256 (the kernels with the log-mass epilogue), MFMA, two-stage
    const bool direct_ok = layout == FS_LAYOUT_TILED || rows_direct_ok(D);   // kernels with the log-mass epilogue
    if (!direct_ok || dtype != FS_DTYPE_BF16 || variant == FS_VARIANT_GEMV || (o && o->single_pass)) {
      *why = FS_ERR_UNSUPPORTED;
      return false;
    }
    variant = FS_VARIANT_MFMA;
  }
  int32_t tile = o ? o->vocab_tile : 0;
  const int32_t bt = o ? o->batch_tile : 0;
  if (bt != 0 && bt != 16 && bt != 32 && bt != 64 && bt != kTiledWideBatch && bt != kTiledBigBatch) return false;
  if (bt == kTiledBigBatch) {
    // the 256 x 256 tile: tiled bf16 W, D a multiple of 32, plain sampling
    const bool ok = layout == FS_LAYOUT_TILED && dtype == FS_DTYPE_BF16 && D % 32 == 0 && group_size == 0 &&
                    !(o && o->logits) && variant != FS_VARIANT_GEMV &&
                    (o->vocab_tile == 0 || o->vocab_tile == kTiledWideTile);
    if (!ok) {
      *why = FS_ERR_UNSUPPORTED;
      return false;
    }
    p->variant = FS_VARIANT_MFMA;
    p->tile = kTiledWideTile;
    p->n_tiles = (V + kTiledWideTile - 1) / kTiledWideTile;
    p->batch_tile = kTiledBigBatch;
    p->tiled = true;
    p->single_pass = o->single_pass;
    p->group_size = 0;
    return true;
  }
  const bool long_rows = layout == FS_LAYOUT_ROWS && dtype == FS_DTYPE_BF16 && D >= kGemvLongRowD;
  // tiled W: the matrix-core kernels at every B (measured 0-2.3% faster than
  // GEMV at B <= 2: the 128-row tiles stream the layout's 64 KiB runs)
  if (variant == FS_VARIANT_AUTO)
    variant = (B > kGemvMaxB || layout == FS_LAYOUT_TILED) ? FS_VARIANT_MFMA : FS_VARIANT_GEMV;
  if (variant == FS_VARIANT_MFMA && dtype == FS_DTYPE_F32 && layout == FS_LAYOUT_ROWS) {
    // fp32 matrix-core kernel: 128-row vocab tiles, batch tiles of 16, 32 or 64
    if (tile == 0) tile = mfma_f32_tile_rows();
    if (tile != mfma_f32_tile_rows() || bt == kTiledWideBatch) return false;
    p->variant = FS_VARIANT_MFMA;
    p->tile = tile;
    p->n_tiles = (V + tile - 1) / tile;
    p->batch_tile = bt;
    p->tiled = false;
    p->single_pass = o && o->single_pass;
    p->group_size = 0;
    return true;
  }
  if (layout == FS_LAYOUT_TILED) {
    if (dtype != FS_DTYPE_BF16) {
      *why = FS_ERR_UNSUPPORTED;
      return false;
    }
    if (tile == 0)
      tile = variant != FS_VARIANT_MFMA ? kTiledGemvTile : B >= kTiledWideMinB ? kTiledWideTile : kTiledMfmaTile;
    const bool wide = variant == FS_VARIANT_MFMA && tile == kTiledWideTile;
    if (tile != 64 && tile != 128 && !wide) return false;
    if (wide != (bt == kTiledWideBatch) && bt != 0) return false;  // 128-column batch tiles only with the wide tile
  } else if (variant == FS_VARIANT_MFMA) {
    if (dtype != FS_DTYPE_BF16) {
      *why = FS_ERR_UNSUPPORTED;
      return false;
    }
    // D a multiple of 256: the tiled-layout kernels read the rows directly,
    // the 256-row wide tile included; other D: the transposing kernel
    const bool direct = rows_direct_ok(D);
    if (tile == 0)
      tile = direct ? (B >= kTiledWideMinB ? kTiledWideTile : kRowsTile) : B > 32 ? kMfmaLargeBTile : kMfmaSmallBTile;
    const bool wide = direct && tile == kTiledWideTile;
    if (tile != mfma_tile_rows(1) && tile != mfma_tile_rows(2) && !wide) return false;
    if (wide != (bt == kTiledWideBatch) && bt != 0) return false;
  } else {
    // more rows per workgroup once the batch tile is large: fewer, longer
    // workgroups amortise staging H and the cross-wave reduction (fp32,
    // 4096 x 256 head, B = 256: 97 -> 80 us)
    if (tile == 0) {
      if (long_rows && B <= kGemvMaxB) tile = kGemvLongTile;
      else tile = B > kGemvSmallB ? kGemvLargeBTile : kGemvDefaultTile;
    }
    if (tile < 0 || tile % kGemvGranule != 0) return false;
  }
  p->variant = (fs_variant_t)variant;
  p->tile = tile;
  p->n_tiles = (V + tile - 1) / tile;
  p->batch_tile = variant == FS_VARIANT_MFMA ? bt : 0;
  p->tiled = layout == FS_LAYOUT_TILED;
  p->single_pass = o && o->single_pass;
  p->group_size = group_size;
  if (p->n_tiles > 0x7FFFFFFF) return false;
  if (group_size > 0 && group_size % tile != 0) return false;   // groups are unions of vocab tiles
  return true;
}

// The fused call's plan: make_plan's, with the 128-row tiles of a ragged last
// round of workgroups split into 64-row tiles where the sampling-only tiled
// kernel runs (one batch tile, no logits store, no log-masses). The count
// depends on the current device (resident workgroups), so the sizing queries
// and the call agree on one device.
bool make_fused_plan(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype, const fs_options_t* o, Plan* p,
                     fs_status_t* why) {
  if (!make_plan(B, D, V, dtype, o, p, why)) return false;
  if (p->tiled && p->variant == FS_VARIANT_MFMA && p->tile == kTiledMfmaTile && p->group_size == 0 &&
      !(o && o->logits)) {
    p->half_tiles = tiled_half_tiles(p->n_tiles, B, p->batch_tile);
    p->n_tiles += p->half_tiles / 2;
    if (p->n_tiles > 0x7FFFFFFF) return false;
  }
  return true;
}

hipError_t launch_stage1(const Plan& p, const Stage1Args& a, fs_dtype_t dtype, hipStream_t stream) {
  if (p.tiled) return launch_stage1_tiled(a, p.variant == FS_VARIANT_MFMA, stream);
  if (p.variant != FS_VARIANT_MFMA) return launch_stage1_gemv(a, dtype, stream);
  if (dtype == FS_DTYPE_F32) return launch_stage1_mfma_f32(a, stream);
  // row-major MFMA: the A operand straight from the rows when D is a multiple
  // of the K block, else the kernel that transposes W through LDS
  return rows_direct_ok(a.D) ? launch_stage1_rows_direct(a, stream) : launch_stage1_mfma(a, stream);
}

size_t cand_bytes(int64_t B, const Plan& p) {
  return align_up((size_t)B * (size_t)p.n_tiles * sizeof(uint64_t), kAlign);
}

size_t fused_ws_bytes(int64_t B, const Plan& p) {
  if (p.single_pass)   // keys + the counters, one 256-byte slot each
    return align_up((size_t)B * sizeof(uint64_t), kAlign) + (size_t)(kSpGroups + 1) * kSpSlot * sizeof(uint32_t);
  if (p.group_size > 0) return cand_bytes(B, p) + align_up((size_t)B * (size_t)p.n_tiles * sizeof(float), kAlign);
  return cand_bytes(B, p);
}

int64_t unfused_ld(int64_t V) { return (V + 7) / 8 * 8; }
int64_t unfused_parts(int64_t V) { return (V + kSamplePart - 1) / kSamplePart; }

size_t unfused_ws_bytes(int64_t B, int64_t V, fs_dtype_t logits_dtype) {
  const size_t logits = align_up((size_t)B * unfused_ld(V) * dtype_size(logits_dtype), kAlign);
  return logits + align_up((size_t)B * unfused_parts(V) * sizeof(uint64_t), kAlign);
}

NoiseKey noise_key(uint64_t seed, uint64_t step) {
  return NoiseKey{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)step, (uint32_t)(step >> 32)};
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared validation of the sampling entry points.
fs_status_t check_common(const void* H, int64_t ldh, const void* W, int64_t ldw, int dtype,
                         int64_t B, int64_t D, int64_t V, float T, const void* ws,
                         const int32_t* out, const fs_options_t* o) {
  if (!H || !W || !ws || !out) return FS_ERR_INVALID_ARGUMENT;
  if (!sizes_ok(B, D, V)) return FS_ERR_INVALID_ARGUMENT;
  const bool tiled = o && o->weights_layout == FS_LAYOUT_TILED;
  if (tiled) ldw = D;  // ignored
  if (ldh < D || ldw < D) return FS_ERR_INVALID_ARGUMENT;
  if (!(T >= 0.f) || !std::isfinite(T)) return FS_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(dtype)) return FS_ERR_UNSUPPORTED;
  const int64_t esz = (int64_t)dtype_size((fs_dtype_t)dtype);
  if (!aligned16(H) || !aligned16(W) || !aligned16(ws)) return FS_ERR_UNSUPPORTED;
  if ((D * esz) % 16 || (ldh * esz) % 16 || (ldw * esz) % 16) return FS_ERR_UNSUPPORTED;
  if (D * esz > kMaxHRowBytes) return FS_ERR_UNSUPPORTED;  // one H row must fit LDS
  return FS_OK;
}

Stage1Args stage1_args(const void* H, int64_t ldh, const void* W, int64_t ldw, int64_t B,
                       int64_t D, int64_t V, float T, uint64_t seed, uint64_t step,
                       const Plan& p) {
  Stage1Args a{};
  a.H = H;
  a.ldh = ldh;
  a.W = W;
  a.ldw = ldw;
  a.B = (int32_t)B;
  a.D = (int32_t)D;
  a.V = (int32_t)V;
  a.greedy = T == 0.f;
  a.inv_t = T == 0.f ? 0.f : 1.0f / T;
  a.score_scale = T == 0.f ? 0.f : (float)(1.0 / ((double)T * 0.693147180559945309417));
  a.nk = noise_key(seed, step);
  a.vocab_tile = p.tile;
  a.n_tiles = (int32_t)p.n_tiles;
  a.batch_tile = p.batch_tile;
  a.half_tiles = (int32_t)p.half_tiles;
  return a;
}

// A validated fused call: its plan and the Stage-1 arguments with the
// workspace carved up (candidates, log-masses or single-pass keys).
fs_status_t prepare_fused(const void* H, int64_t ldh, const void* W, int64_t ldw, fs_dtype_t dtype, int64_t B,
                          int64_t D, int64_t V, float temperature, uint64_t seed, uint64_t step, void* workspace,
                          size_t workspace_bytes, int32_t* out_tokens, const fs_options_t* opts, FusedCall* call) {
  fs_status_t st = check_common(H, ldh, W, ldw, dtype, B, D, V, temperature, workspace, out_tokens, opts);
  if (st != FS_OK) return st;
  Plan& p = call->plan;
  if (!make_fused_plan(B, D, V, dtype, opts, &p, &st)) return st;
  if (opts && opts->logits) {
    if (!dtype_ok(opts->logits_dtype)) return FS_ERR_UNSUPPORTED;
    if (opts->ld_logits < V) return FS_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)opts->logits & 15u) != 0) return FS_ERR_UNSUPPORTED;
  }
  call->ws_bytes = fused_ws_bytes(B, p);
  if (workspace_bytes < call->ws_bytes) return FS_ERR_WORKSPACE_TOO_SMALL;

  Stage1Args& a = call->args;
  a = stage1_args(H, ldh, W, ldw, B, D, V, temperature, seed, step, p);
  a.cand = static_cast<uint64_t*>(workspace);
  call->grouped = p.group_size > 0 && !a.greedy;   // greedy: the plain maximiser
  if (call->grouped) a.mass = reinterpret_cast<float*>(static_cast<char*>(workspace) + cand_bytes(B, p));
  if (p.single_pass) {
    a.single_pass = 1;
    a.keys = static_cast<uint64_t*>(workspace);
    a.counter = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                            align_up((size_t)B * sizeof(uint64_t), kAlign));
    a.out = out_tokens;
  }
  if (opts && opts->logits) {
    a.logits = opts->logits;
    a.ld_logits = opts->ld_logits;
    a.logits_bf16 = opts->logits_dtype == FS_DTYPE_BF16;
  }
  return FS_OK;
}

// Enqueues a prepared fused call: Stage 1 (with the optional timing events
// around it), then Stage 2 unless it is folded into Stage 1.
fs_status_t enqueue_fused(const FusedCall& call, fs_dtype_t dtype, int32_t* out_tokens, hipStream_t stream,
                          const fs_options_t* opts) {
  const Plan& p = call.plan;
  const Stage1Args& a = call.args;
  hipError_t e;
  if (opts && opts->stage1_start && (e = hipEventRecord(opts->stage1_start, stream)) != hipSuccess)
    return fail_hip(e);
  e = launch_stage1(p, a, dtype, stream);
  if (e != hipSuccess) return fail_hip(e);
  if (opts && opts->stage1_stop && (e = hipEventRecord(opts->stage1_stop, stream)) != hipSuccess)
    return fail_hip(e);
  if (call.grouped) {
    e = launch_stage2_grouped(a.cand, a.mass, a.B, a.n_tiles, p.group_size / p.tile, a.nk, out_tokens, stream);
    if (e != hipSuccess) return fail_hip(e);
  } else if (!p.single_pass) {
    e = launch_stage2(a.cand, a.B, a.n_tiles, out_tokens, stream);
    if (e != hipSuccess) return fail_hip(e);
  }
  return FS_OK;
}

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (hipGetSymbolAddress) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // guarded by g_scratch_mutex

fs_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return FS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e);
    if (!p) return fail_hip(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FS_OK;
}

}  // namespace
}  // namespace fs

using namespace fs;

extern "C" {

const char* fs_status_string(fs_status_t s) {
  switch (s) {
    case FS_OK: return "FS_OK";
    case FS_ERR_INVALID_ARGUMENT: return "FS_ERR_INVALID_ARGUMENT";
    case FS_ERR_UNSUPPORTED: return "FS_ERR_UNSUPPORTED";
    case FS_ERR_WORKSPACE_TOO_SMALL: return "FS_ERR_WORKSPACE_TOO_SMALL";
    case FS_ERR_HIP: return "FS_ERR_HIP";
  }
  return "FS_ERR_UNKNOWN";
}

int fs_last_hip_error(void) { return g_last_hip_error; }

int32_t fs_vocab_tile_granule(fs_variant_t variant) {
  switch (variant) {
    case FS_VARIANT_AUTO:
    case FS_VARIANT_GEMV: return kGemvGranule;
    case FS_VARIANT_MFMA: return kMfmaGranule;
    default: return -1;
  }
}

int64_t fs_num_vocab_tiles(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype, const fs_options_t* opts) {
  if (!sizes_ok(B, D, V) || !dtype_ok(dtype)) return -1;
  Plan p;
  fs_status_t why;
  if (!make_fused_plan(B, D, V, dtype, opts, &p, &why)) return -1;
  return p.n_tiles;
}

size_t fs_workspace_bytes_ex(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype, const fs_options_t* opts) {
  if (!sizes_ok(B, D, V) || !dtype_ok(dtype)) return 0;
  Plan p;
  fs_status_t why;
  if (!make_fused_plan(B, D, V, dtype, opts, &p, &why)) return 0;
  return fused_ws_bytes(B, p);
}

size_t fs_workspace_bytes(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype) {
  return fs_workspace_bytes_ex(B, D, V, dtype, nullptr);
}

fs_status_t fs_sample_fused_ex(const void* H, int64_t ldh, const void* W, int64_t ldw, fs_dtype_t dtype,
                               int64_t B, int64_t D, int64_t V, float temperature, uint64_t seed,
                               uint64_t step, void* workspace, size_t workspace_bytes,
                               int32_t* out_tokens, hipStream_t stream, const fs_options_t* opts) {
  FusedCall call;
  const fs_status_t st = prepare_fused(H, ldh, W, ldw, dtype, B, D, V, temperature, seed, step, workspace,
                                       workspace_bytes, out_tokens, opts, &call);
  if (st != FS_OK) return st;
  return enqueue_fused(call, dtype, out_tokens, stream, opts);
}

fs_status_t fs_sample_fused_noalloc(const void* H, int64_t ldh, const void* W, int64_t ldw, fs_dtype_t dtype,
                                    int64_t B, int64_t D, int64_t V, float temperature, uint64_t seed,
                                    uint64_t step, int32_t* out_tokens, hipStream_t stream,
                                    const fs_options_t* opts) {
  constexpr size_t kScratchBytes = FS_NOALLOC_SCRATCH_BYTES;
  FusedCall call;
  // validate first (no device call), with a stand-in for the scratch address
  fs_status_t st = prepare_fused(H, ldh, W, ldw, dtype, B, D, V, temperature, seed, step,
                                 reinterpret_cast<void*>(kAlign), kScratchBytes, out_tokens, opts, &call);
  if (st != FS_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != FS_OK) return st;
  st = prepare_fused(H, ldh, W, ldw, dtype, B, D, V, temperature, seed, step, ws, kScratchBytes, out_tokens,
                     opts, &call);
  if (st != FS_OK) return st;
  if (call.plan.single_pass) {
    // the single-pass keys and counter start at zero; the array holds
    // whatever the previous call on this GPU left (a fill kernel, not a
    // memset, so the call stays capturable)
    const hipError_t e = launch_fill_zero(static_cast<uint64_t*>(ws), (int64_t)(call.ws_bytes / 8), stream);
    if (e != hipSuccess) return fail_hip(e);
  }
  return enqueue_fused(call, dtype, out_tokens, stream, opts);
}

fs_status_t fs_sample_fused(const void* H, int64_t ldh, const void* W, int64_t ldw, fs_dtype_t dtype,
                            int64_t B, int64_t D, int64_t V, float temperature, uint64_t seed,
                            uint64_t step, void* workspace, size_t workspace_bytes, int32_t* out_tokens,
                            hipStream_t stream) {
  return fs_sample_fused_ex(H, ldh, W, ldw, dtype, B, D, V, temperature, seed, step, workspace,
                            workspace_bytes, out_tokens, stream, nullptr);
}

size_t fs_unfused_workspace_bytes(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype,
                                  fs_dtype_t logits_dtype) {
  if (!sizes_ok(B, D, V) || !dtype_ok(dtype) || !dtype_ok(logits_dtype)) return 0;
  return unfused_ws_bytes(B, V, logits_dtype);
}

fs_status_t fs_sample_unfused_ex(const void* H, int64_t ldh, const void* W, int64_t ldw, fs_dtype_t dtype,
                                 int64_t B, int64_t D, int64_t V, float temperature, uint64_t seed,
                                 uint64_t step, fs_dtype_t logits_dtype, void* workspace,
                                 size_t workspace_bytes, int32_t* out_tokens, hipStream_t stream,
                                 const fs_options_t* opts) {
  fs_status_t st = check_common(H, ldh, W, ldw, dtype, B, D, V, temperature, workspace, out_tokens, opts);
  if (st != FS_OK) return st;
  if (!dtype_ok(logits_dtype)) return FS_ERR_UNSUPPORTED;
  if (opts && opts->group_size != 0) return FS_ERR_UNSUPPORTED;   // the baseline is plain sampling
  if (opts && opts->batch_tile == kTiledBigBatch) return FS_ERR_UNSUPPORTED;   // that tile only samples
  Plan p;
  if (!make_plan(B, D, V, dtype, opts, &p, &st)) return st;
  if (workspace_bytes < unfused_ws_bytes(B, V, logits_dtype)) return FS_ERR_WORKSPACE_TOO_SMALL;

  const int64_t ld = unfused_ld(V);
  const size_t logits_bytes = align_up((size_t)B * ld * dtype_size(logits_dtype), kAlign);
  char* ws = static_cast<char*>(workspace);
  uint64_t* partial = reinterpret_cast<uint64_t*>(ws + logits_bytes);   // room for unfused_parts(V) per row

  // step 1: GEMM that writes the logits (same Stage-1 main loop, store epilogue)
  Stage1Args a = stage1_args(H, ldh, W, ldw, B, D, V, temperature, seed, step, p);
  a.cand = nullptr;
  a.logits = ws;
  a.ld_logits = ld;
  a.logits_bf16 = logits_dtype == FS_DTYPE_BF16;
  hipError_t e = launch_stage1(p, a, dtype, stream);
  if (e != hipSuccess) return fail_hip(e);
  // step 2: sampler that reads them back
  int32_t n_parts = 0;
  e = launch_sample_logits(ws, ld, a.logits_bf16, a.B, a.V, a.score_scale, a.greedy, a.nk, partial, &n_parts,
                           stream);
  if (e != hipSuccess) return fail_hip(e);
  e = launch_stage2(partial, a.B, n_parts, out_tokens, stream);
  if (e != hipSuccess) return fail_hip(e);
  return FS_OK;
}

fs_status_t fs_sample_unfused(const void* H, int64_t ldh, const void* W, int64_t ldw, fs_dtype_t dtype,
                              int64_t B, int64_t D, int64_t V, float temperature, uint64_t seed,
                              uint64_t step, fs_dtype_t logits_dtype, void* workspace,
                              size_t workspace_bytes, int32_t* out_tokens, hipStream_t stream) {
  return fs_sample_unfused_ex(H, ldh, W, ldw, dtype, B, D, V, temperature, seed, step, logits_dtype,
                              workspace, workspace_bytes, out_tokens, stream, nullptr);
}

size_t fs_tiled_weights_bytes(int64_t V, int64_t D, fs_dtype_t dtype) {
  if (dtype != FS_DTYPE_BF16 || !sizes_ok(1, D, V)) return 0;
  return (size_t)tiled_weights_bytes(V, D);
}

fs_status_t fs_pack_weights_tiled(const void* W, int64_t ldw, int64_t V, int64_t D, fs_dtype_t dtype,
                                  void* tiled, size_t tiled_bytes, hipStream_t stream) {
  if (!W || !tiled || !sizes_ok(1, D, V) || ldw < D) return FS_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(dtype) || dtype != FS_DTYPE_BF16) return FS_ERR_UNSUPPORTED;
  if (!aligned16(W) || !aligned16(tiled) || (D * 2) % 16 || (ldw * 2) % 16) return FS_ERR_UNSUPPORTED;
  if (tiled_bytes < (size_t)tiled_weights_bytes(V, D)) return FS_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = launch_pack_tiled(W, ldw, (int32_t)V, (int32_t)D, tiled, stream);
  return e == hipSuccess ? FS_OK : fail_hip(e);
}

fs_status_t fs_test_philox(uint64_t seed, uint64_t step, int64_t b, int64_t v0, int64_t n,
                           uint32_t* words_out, hipStream_t stream) {
  if (!words_out || n <= 0 || v0 < 0 || b < 0 || b > 0xFFFFFFFFll || v0 + n > (int64_t)1 << 34)
    return FS_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_test_philox(noise_key(seed, step), (uint32_t)b, v0, n, words_out, stream);
  return e == hipSuccess ? FS_OK : fail_hip(e);
}

fs_status_t fs_test_gumbel(const uint32_t* words, int64_t n, float* g_out, hipStream_t stream) {
  if (!words || !g_out || n <= 0 || n > ((int64_t)1 << 32)) return FS_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_test_gumbel(words, n, g_out, stream);
  return e == hipSuccess ? FS_OK : fail_hip(e);
}

fs_status_t fs_workspace_reset(void* workspace, size_t bytes, hipStream_t stream) {
  if (!workspace || bytes == 0 || bytes % 8) return FS_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace)) return FS_ERR_UNSUPPORTED;
  hipError_t e = launch_fill_zero(static_cast<uint64_t*>(workspace), (int64_t)(bytes / 8), stream);
  return e == hipSuccess ? FS_OK : fail_hip(e);
}

int64_t fs_probe_read_blocks(int64_t bytes, int64_t chunk_bytes) {
  if (bytes <= 0 || chunk_bytes <= 0 || bytes % 16 || chunk_bytes % 16) return -1;
  const int64_t n = (bytes + chunk_bytes - 1) / chunk_bytes;
  return n > 0x7FFFFFFF ? -1 : n;
}

fs_status_t fs_probe_read(const void* src, int64_t bytes, int64_t chunk_bytes, uint32_t* sink,
                          hipStream_t stream) {
  if (!src || !sink || fs_probe_read_blocks(bytes, chunk_bytes) < 0) return FS_ERR_INVALID_ARGUMENT;
  if (!aligned16(src)) return FS_ERR_UNSUPPORTED;
  hipError_t e = launch_probe_read(src, bytes, chunk_bytes, sink, stream);
  return e == hipSuccess ? FS_OK : fail_hip(e);
}

}  // extern "C"
