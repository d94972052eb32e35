/*
 * flashsample.h - C ABI of the MI355X (gfx950) fused LM-head sampler.
 *
 * Operation (FlashSampling: Fast and Memory-Efficient Exact Sampling,
 * arXiv 2603.15854, Section 3): given hidden states H [B, D] and LM-head
 * weights W [V, D], draw one token per batch row from softmax(H W^T / T)
 * by the Gumbel-max trick,
 *
 *     token[b] = argmax_v ( l[b, v] / T + g(seed, step, b, v) ),  l = H W^T,
 *
 * where g is standard Gumbel noise that depends only on (seed, step, row b,
 * vocab index v). The fused entry point computes l tile by tile on chip,
 * keeps one candidate per (row, vocab tile) (Stage 1 of the method section)
 * and reduces the candidates to one token per row (Stage 2), so the [B, V]
 * logits never reach device memory. The unfused entry point is the
 * two-step baseline of the same section's IO model: a GEMM that writes the
 * logits, then a sampler that reads them.
 *
 * Noise (the pages ask for i.i.d. Gumbels; the generator is this library's
 * choice): Philox4x32-10 (Salmon et al., SC'11) with key
 * (seed mod 2^32, seed >> 32) and counter (v >> 2, b, step mod 2^32,
 * step >> 32); word v & 3 of the output is x, u = (x + 1/2) 2^-32 and
 * g = -ln(-ln u). Ties go to the lowest vocab index; NaN scores never win;
 * a row whose scores are all NaN yields -1. T == 0 is greedy argmax of l.
 *
 * Conventions for every entry point below:
 *  - H, W, workspace and outputs are DEVICE pointers owned by the caller;
 *    the library allocates nothing and keeps no mutable global state (the
 *    one exception: fs_sample_fused_noalloc's static per-GPU scratch array).
 *  - H is row-major [B, D] with row stride ldh elements, W row-major [V, D]
 *    with row stride ldw elements (ld >= D). Both have the same dtype.
 *    Base pointers must be 16-byte aligned and ld * sizeof(dtype) and
 *    D * sizeof(dtype) multiples of 16 (else FS_ERR_UNSUPPORTED). One H row
 *    must fit the on-chip LDS beside the kernels' own reduction arrays:
 *    D * sizeof(dtype) <= 159 KiB (D <= 81408 bf16, 40704 fp32; else
 *    FS_ERR_UNSUPPORTED).
 *  - Calls are asynchronous on `stream`: they validate, enqueue and return.
 *    Only the workspace and the outputs are written. Distinct calls may run
 *    concurrently if they use distinct workspaces and outputs.
 *  - A call enqueues kernel launches only (plus the two timing event records
 *    when fs_options asks for them): no allocation, copy or memset, so it can
 *    be captured in a HIP graph and replayed; the kernel arguments (sizes,
 *    temperature, seed, step, pointers) are fixed at capture.
 *  - Validation is synchronous; on any error nothing is enqueued. A shape
 *    whose first launch would count more work-items in one grid dimension
 *    than a dispatch holds (2^32) is refused at that launch with FS_ERR_HIP
 *    and fs_last_hip_error() == hipErrorInvalidConfiguration, still before
 *    anything is enqueued.
 *  - No C++ exception crosses this interface.
 */
#ifndef FLASHSAMPLE_H
#define FLASHSAMPLE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fs_status {
  FS_OK = 0,
  FS_ERR_INVALID_ARGUMENT = 1,   /* null pointer, size <= 0 or too large, ld < D, bad T */
  FS_ERR_UNSUPPORTED = 2,        /* dtype, alignment or option not supported */
  FS_ERR_WORKSPACE_TOO_SMALL = 3,
  FS_ERR_HIP = 4                 /* a HIP launch failed; see fs_last_hip_error() */
} fs_status_t;

typedef enum fs_dtype { FS_DTYPE_BF16 = 0, FS_DTYPE_F32 = 1 } fs_dtype_t;

/* Stage-1 kernel family. AUTO: GEMV (wavefront dot products) up to 2 batch
 * rows (up to 4 on row-major bf16 W with 4096 <= D <= 8192), matrix cores
 * above (bf16: v_mfma_f32_16x16x32_bf16; fp32, row-major W only:
 * v_mfma_f32_16x16x4_f32, fp32 products and sums). */
typedef enum fs_variant { FS_VARIANT_AUTO = 0, FS_VARIANT_GEMV = 1, FS_VARIANT_MFMA = 2 } fs_variant_t;

/* Layout of the W argument.
 *  ROWS:  row-major [V, D] with row stride ldw (the default).
 *  TILED: the one-time repacked copy made by fs_pack_weights_tiled (bf16
 *         only): blocks of 16 vocab rows x 256 columns, each 8 KiB
 *         contiguous in matrix-core operand order; block (m, c) at index
 *         ((m / 8) * ceil(D / 256) + c) * 8 + m % 8; ldw is ignored. */
typedef enum fs_layout { FS_LAYOUT_ROWS = 0, FS_LAYOUT_TILED = 1 } fs_layout_t;

/* Options for the _ex entry points; a zero-initialised struct means defaults.
 * Results never depend on variant or vocab_tile (the argmax decomposes over
 * any vocab partition), only speed does. */
typedef struct fs_options {
  int32_t variant;         /* fs_variant_t */
  int32_t vocab_tile;      /* rows per Stage-1 vocab tile; 0 = variant default.
                              Row-major W: a multiple of the variant's granule
                              (fs_vocab_tile_granule); MFMA: 64 or 128, or 256
                              when D is a multiple of 256 (fp32: 128 only,
                              the fp32 matrix-core kernel). Tiled W: 64 or 128,
                              or 256 for MFMA. 256 is the wide kernel (8 waves
                              of two 16-row blocks, 128-column batch tiles; the
                              default from B = 65 on where allowed). */
  void* logits;            /* non-null: the fused call also stores l = H W^T
                              (device [B, V] row-major, stride ld_logits) */
  int64_t ld_logits;
  int32_t logits_dtype;    /* fs_dtype_t of the stored logits */
  int32_t batch_tile;      /* MFMA only: batch rows per workgroup (16, 32 or
                              64; 128 with the 256-row tiled tile, and only
                              there); 0 = chosen from B. Larger batches are
                              split into tiles that re-read W from L2.
                              256: the 256 x 256 tile with both operands
                              copied straight into LDS (tiled bf16 W, D a
                              multiple of 32, fused sampling without stored
                              logits or groups; else FS_ERR_UNSUPPORTED);
                              never chosen by itself. */
  hipEvent_t stage1_start; /* non-null: recorded on `stream` right before and */
  hipEvent_t stage1_stop;  /* right after the Stage-1 launch (for timing) */
  int32_t weights_layout;  /* fs_layout_t of W */
  int32_t single_pass;     /* nonzero: fold Stage 2 into Stage 1 (one launch).
                              Each Stage-1 workgroup takes an atomic maximum
                              of its keys into a [B] key array in the
                              workspace and counts itself finished (two
                              levels of counters); the last workgroup to
                              finish writes the tokens and returns the
                              workspace to zero.
                              The workspace (fs_workspace_bytes_ex with this
                              option) must be zero before its first use
                              (fs_workspace_reset), and calls sharing it must
                              not overlap. Results equal the two-stage ones. */
  int32_t group_size;      /* > 0: the grouped variant (FlashSampling, arXiv
                              2603.15854, Section 3, tensor-parallel
                              paragraphs: a local sample and a local log-mass
                              per vocabulary group, exact by hierarchical
                              factorisation). Groups are the contiguous vocab
                              ranges [k G, (k+1) G); each group's local sample
                              is its Gumbel-max with the token noise, its
                              log-mass log sum exp(l/T) over its non-NaN
                              entries, and the group is drawn by Gumbel-max over
                              the log-masses with a second Philox stream (counter
                              word 0 = 0xC0000000 | k >> 2, row, step; word
                              k & 3). The sample then follows softmax(l/T) but
                              differs from the plain call's for the same seed.
                              G must be a multiple of the Stage-1 vocab tile
                              (any multiple of 256 always is). Bf16, tiled
                              weights or row-major ones with D a multiple of
                              256; not with single_pass. T == 0 gives the plain
                              greedy result. 0 = plain sampling. */
  int32_t reserved;        /* must be 0 */
} fs_options_t;

/* Human-readable name of a status code (static storage). */
const char* fs_status_string(fs_status_t status);

/* hipError_t of the most recent FS_ERR_HIP returned on the calling thread
 * (0 if none). */
int fs_last_hip_error(void);

/* Number of Stage-1 vocab tiles the fused call uses for these sizes (the
 * candidate buffer is [n_tiles, B] 64-bit keys at the start of the
 * workspace, tile-major so each Stage-1 workgroup writes one contiguous
 * run). On tiled W with 17-64 rows and 128-row tiles, the tiles of a last
 * round of resident workgroups at most a quarter full count twice (each runs
 * as two 64-row tiles); that depends on the current device's compute units
 * and occupancy, so this query, fs_workspace_bytes_ex and the call agree when
 * made with the same device current (no device: no such split counted).
 * Returns -1 for invalid sizes or options. */
int64_t fs_num_vocab_tiles(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype,
                           const fs_options_t* opts);

/* Row granule a vocab_tile option must be a multiple of, for a variant. */
int32_t fs_vocab_tile_granule(fs_variant_t variant);

/* Workspace bytes fs_sample_fused needs (candidate buffer of the Stage-1
 * tiles: one 64-bit key per (row, vocab tile); with group_size, also one fp32
 * log-mass per (row, vocab tile); with single_pass, B keys and the
 * finished-workgroup counters, 8448 bytes).
 * The size arguments come in the order of the sampling calls' own: B, D, V
 * (batch rows, hidden size, vocabulary rows). Device-dependent like
 * fs_num_vocab_tiles (query with the call's device current; a too small
 * workspace is refused with FS_ERR_WORKSPACE_TOO_SMALL before any launch).
 * 0 on invalid sizes or options. */
size_t fs_workspace_bytes(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype);
size_t fs_workspace_bytes_ex(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype,
                             const fs_options_t* opts);

/* Zeroes a workspace on `stream` with a fill kernel (no memset node, so it
 * may be captured in a graph). Needed once before the first single-pass
 * call on a workspace. bytes must be a multiple of 8; ws 16-byte aligned. */
fs_status_t fs_workspace_reset(void* workspace, size_t bytes, hipStream_t stream);

/* Fused sampler (FlashSampling Stage 1 + Stage 2; Section 3, the two-stage
 * list and the exactness paragraph).
 *   H, ldh, W, ldw, dtype, B, D, V: as in the conventions above.
 *   temperature: T >= 0 and finite (T == 0: greedy).
 *   seed, step: noise key and decode step (see the noise paragraph above).
 *   workspace: device, >= fs_workspace_bytes(...) bytes, 16-byte aligned.
 *   out_tokens: device int32 [B].
 * Errors: FS_ERR_INVALID_ARGUMENT, FS_ERR_UNSUPPORTED,
 *         FS_ERR_WORKSPACE_TOO_SMALL, FS_ERR_HIP. */
fs_status_t fs_sample_fused(const void* H, int64_t ldh, const void* W, int64_t ldw,
                            fs_dtype_t dtype, int64_t B, int64_t D, int64_t V,
                            float temperature, uint64_t seed, uint64_t step,
                            void* workspace, size_t workspace_bytes,
                            int32_t* out_tokens, hipStream_t stream);

/* Same, with options (forced variant or vocab tile, optional logits store
 * as in the pages' IO-model check, Appendix K, and Stage-1 timing events). */
fs_status_t fs_sample_fused_ex(const void* H, int64_t ldh, const void* W, int64_t ldw,
                               fs_dtype_t dtype, int64_t B, int64_t D, int64_t V,
                               float temperature, uint64_t seed, uint64_t step,
                               void* workspace, size_t workspace_bytes,
                               int32_t* out_tokens, hipStream_t stream,
                               const fs_options_t* opts);

/* Allocation-free fused sampler, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, results and errors as fs_sample_fused_ex
 * without the workspace: the candidate buffer (or the single-pass keys, or
 * the grouped variant's log-masses) lives in a static device array of
 * FS_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held until
 * the process ends. Its device address is looked up once per device on the
 * first call with that device current (the stream must belong to the current
 * device). The call allocates nothing and enqueues kernels only (single_pass
 * adds a fill kernel that zeroes the keys first).
 *  - Sizes whose workspace (fs_workspace_bytes_ex) exceeds
 *    FS_NOALLOC_SCRATCH_BYTES: FS_ERR_WORKSPACE_TOO_SMALL, nothing enqueued
 *    (e.g. V = 128256: two-stage up to B = 1024 and beyond fits).
 *  - Every call on one GPU shares that GPU's array: calls that overlap in
 *    time on one GPU (other streams, other threads) race and give undefined
 *    tokens; serialise them. */
#define FS_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
fs_status_t fs_sample_fused_noalloc(const void* H, int64_t ldh, const void* W, int64_t ldw,
                                    fs_dtype_t dtype, int64_t B, int64_t D, int64_t V,
                                    float temperature, uint64_t seed, uint64_t step,
                                    int32_t* out_tokens, hipStream_t stream,
                                    const fs_options_t* opts);

/* Bytes of the tiled copy of a [V, D] bf16 LM head (V rounded up to a
 * group of 8 blocks of 16 rows, D to 256 columns, zero padded). 0 for
 * invalid sizes or fp32. */
size_t fs_tiled_weights_bytes(int64_t V, int64_t D, fs_dtype_t dtype);

/* Repacks a row-major bf16 W [V, D] (stride ldw) into the tiled layout
 * (device buffer `tiled` of at least fs_tiled_weights_bytes bytes, 16-byte
 * aligned). Weights are static, so this runs once when the head is loaded;
 * the sampling entry points then take the tiled copy with
 * weights_layout = FS_LAYOUT_TILED and read it with one contiguous 1 KiB
 * load per wave per matrix-core step. Errors as fs_sample_fused. */
fs_status_t fs_pack_weights_tiled(const void* W, int64_t ldw, int64_t V, int64_t D, fs_dtype_t dtype,
                                  void* tiled, size_t tiled_bytes, hipStream_t stream);

/* Workspace of the unfused baseline: the [B, V] logits in logits_dtype plus
 * the sampler's partial candidates. Size arguments B, D, V as in the sampling
 * calls; dtype is the H and W dtype. 0 on invalid sizes. */
size_t fs_unfused_workspace_bytes(int64_t B, int64_t D, int64_t V, fs_dtype_t dtype,
                                  fs_dtype_t logits_dtype);

/* Unfused baseline of the IO model (Section 3, "the baseline runs two
 * steps"): GEMM kernel writes l = H W^T to the workspace in logits_dtype,
 * then a Gumbel-max sampler kernel reads it back. Same noise, tie and NaN
 * rules as the fused call; with FS_DTYPE_F32 logits the tokens equal the
 * fused ones, with FS_DTYPE_BF16 the logits are rounded before noise.
 * Arguments and errors as fs_sample_fused. */
fs_status_t fs_sample_unfused(const void* H, int64_t ldh, const void* W, int64_t ldw,
                              fs_dtype_t dtype, int64_t B, int64_t D, int64_t V,
                              float temperature, uint64_t seed, uint64_t step,
                              fs_dtype_t logits_dtype,
                              void* workspace, size_t workspace_bytes,
                              int32_t* out_tokens, hipStream_t stream);

/* Same, with options (weights_layout, forced variant and tiles; the logits
 * and event fields are ignored). */
fs_status_t fs_sample_unfused_ex(const void* H, int64_t ldh, const void* W, int64_t ldw,
                                 fs_dtype_t dtype, int64_t B, int64_t D, int64_t V,
                                 float temperature, uint64_t seed, uint64_t step,
                                 fs_dtype_t logits_dtype,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t* out_tokens, hipStream_t stream,
                                 const fs_options_t* opts);

/* Test hooks (device buffers): the Philox words the kernels use for
 * vocab indices v0 .. v0+n-1 of row b, and the fp32 Gumbel map the kernels
 * apply to arbitrary words. */
fs_status_t fs_test_philox(uint64_t seed, uint64_t step, int64_t b, int64_t v0, int64_t n,
                           uint32_t* words_out, hipStream_t stream);
fs_status_t fs_test_gumbel(const uint32_t* words, int64_t n, float* g_out, hipStream_t stream);

/* Measurement hook: reads `bytes` (multiple of 16) from the device buffer
 * src with 16-byte loads, workgroup g covering [g*chunk_bytes,
 * (g+1)*chunk_bytes), and writes one folded word per workgroup to sink
 * (device, fs_probe_read_blocks(bytes, chunk_bytes) words). It moves exactly
 * the bytes of a W-sized read and nothing else, which gives the attainable
 * streaming bandwidth and a reference for hardware traffic counters. */
int64_t fs_probe_read_blocks(int64_t bytes, int64_t chunk_bytes);
fs_status_t fs_probe_read(const void* src, int64_t bytes, int64_t chunk_bytes, uint32_t* sink,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHSAMPLE_H */
