/* Exercises the host side of the C ABI without a device: argument
 * validation of every sampling entry point, kernel and tile planning and
 * workspace arithmetic over a grid of shapes and options. Meant to run with
 * the library's host code built under AddressSanitizer, so an out-of-bounds
 * or use-after-free in that code aborts the run. Every pointer below is an
 * aligned stand-in that is never dereferenced: each call either fails
 * validation (the expected status is checked) or is a sizing query.
 *
 * usage: abi_validation          exit status 0 when every check held */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "flashsample.h"

#define FAKE ((void*)(uintptr_t)0x100000)

static int failures = 0;

static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s: got %d, want %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(got, want) expect((int)(got), (int)(want), #got, __LINE__)

static fs_status_t fused(const void* H, int64_t ldh, const void* W, int64_t ldw, int dtype, int64_t B, int64_t D,
                         int64_t V, float T, void* ws, size_t wsb, int32_t* out, const fs_options_t* o) {
  return fs_sample_fused_ex(H, ldh, W, ldw, (fs_dtype_t)dtype, B, D, V, T, 1, 2, ws, wsb, out, NULL, o);
}

int main(void) {
  fs_options_t o;
  int32_t* out = (int32_t*)FAKE;

  /* status strings, including out-of-range codes */
  for (int s = -2; s < 8; ++s)
    if (!fs_status_string((fs_status_t)s)) ++failures;

  /* argument validation of the fused call */
  memset(&o, 0, sizeof o);
  EXPECT(fused(NULL, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_INVALID_ARGUMENT);
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 0, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_INVALID_ARGUMENT);
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, (int64_t)1 << 31, 1.f, FAKE, 1 << 20, out, &o),
         FS_ERR_INVALID_ARGUMENT);
  EXPECT(fused(FAKE, 32, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_INVALID_ARGUMENT);
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, -1.f, FAKE, 1 << 20, out, &o),
         FS_ERR_INVALID_ARGUMENT);
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, NAN, FAKE, 1 << 20, out, &o), FS_ERR_INVALID_ARGUMENT);
  EXPECT(fused(FAKE, 64, FAKE, 64, 9, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_UNSUPPORTED);
  EXPECT(fused((char*)FAKE + 2, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o),
         FS_ERR_UNSUPPORTED);
  EXPECT(fused(FAKE, 68, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_UNSUPPORTED);
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 8, out, &o), FS_ERR_WORKSPACE_TOO_SMALL);
  o.variant = 7;
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_INVALID_ARGUMENT);
  memset(&o, 0, sizeof o);
  o.logits = FAKE;
  o.ld_logits = 999;
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_INVALID_ARGUMENT);
  memset(&o, 0, sizeof o);
  o.reserved = 3;
  EXPECT(fused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, FAKE, 1 << 20, out, &o), FS_ERR_INVALID_ARGUMENT);

  /* the allocation-free entry point validates before touching the device */
  memset(&o, 0, sizeof o);
  EXPECT(fs_sample_fused_noalloc(NULL, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, 0, 0, out, NULL, &o),
         FS_ERR_INVALID_ARGUMENT);
  EXPECT(fs_sample_fused_noalloc(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 4096, 64, 128256, 1.f, 0, 0, out, NULL, &o),
         FS_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(fs_sample_fused_noalloc(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, -2.f, 0, 0, out, NULL, NULL),
         FS_ERR_INVALID_ARGUMENT);

  /* unfused baseline validation */
  EXPECT(fs_sample_unfused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, 0, 0, (fs_dtype_t)5, FAKE, 1 << 20,
                           out, NULL),
         FS_ERR_UNSUPPORTED);
  EXPECT(fs_sample_unfused(FAKE, 64, FAKE, 64, FS_DTYPE_BF16, 2, 64, 1000, 1.f, 0, 0, FS_DTYPE_F32, FAKE, 16, out,
                           NULL),
         FS_ERR_WORKSPACE_TOO_SMALL);

  /* planning and workspace arithmetic over a grid of shapes and options:
   * every answer must be consistent (a workspace at least one key per tile
   * and row, or 0 together with an invalid tile count) */
  static const int64_t Bs[] = {1, 2, 3, 4, 5, 8, 16, 33, 64, 65, 128, 256, 257, 1024, 65536};
  static const int64_t Ds[] = {8, 64, 256, 264, 3584, 4096, 7168, 8192, 81408};
  static const int64_t Vs[] = {1, 5, 1000, 4099, 128256, 152064, 2000003};
  static const int32_t tiles[] = {0, 16, 48, 64, 128, 256, 1008};
  static const int32_t bts[] = {0, 16, 32, 64, 128, 256};
  long checked = 0;
  for (size_t ib = 0; ib < sizeof Bs / sizeof Bs[0]; ++ib)
    for (size_t id = 0; id < sizeof Ds / sizeof Ds[0]; ++id)
      for (size_t iv = 0; iv < sizeof Vs / sizeof Vs[0]; ++iv)
        for (int dt = 0; dt < 2; ++dt)
          for (int layout = 0; layout < 2; ++layout)
            for (int variant = 0; variant < 3; ++variant)
              for (size_t it = 0; it < sizeof tiles / sizeof tiles[0]; ++it)
                for (size_t ibt = 0; ibt < sizeof bts / sizeof bts[0]; ++ibt)
                  for (int flags = 0; flags < 4; ++flags) {
                    memset(&o, 0, sizeof o);
                    o.weights_layout = layout;
                    o.variant = variant;
                    o.vocab_tile = tiles[it];
                    o.batch_tile = bts[ibt];
                    o.single_pass = flags & 1;
                    o.group_size = (flags & 2) ? 4096 : 0;
                    const int64_t B = Bs[ib], D = Ds[id], V = Vs[iv];
                    const int64_t nt = fs_num_vocab_tiles(B, D, V, (fs_dtype_t)dt, &o);
                    const size_t ws = fs_workspace_bytes_ex(B, D, V, (fs_dtype_t)dt, &o);
                    if ((nt < 0) != (ws == 0)) {
                      fprintf(stderr, "inconsistent plan B=%lld D=%lld V=%lld: tiles %lld, workspace %zu\n",
                              (long long)B, (long long)D, (long long)V, (long long)nt, ws);
                      ++failures;
                    } else if (nt > 0 && !o.single_pass && ws < (size_t)B * (size_t)nt * 8u) {
                      fprintf(stderr, "workspace too small for its own plan\n");
                      ++failures;
                    }
                    /* a workspace one byte short is refused before any launch */
                    if (ws > 0 && D * (dt ? 4 : 2) <= 159 * 1024)
                      EXPECT(fused(FAKE, D, FAKE, D, dt, B, D, V, 1.f, FAKE, ws - 1, out, &o),
                             FS_ERR_WORKSPACE_TOO_SMALL);
                    ++checked;
                  }
  EXPECT(fs_tiled_weights_bytes(4099, 1032, FS_DTYPE_BF16), 264 * 5 * 8192);
  EXPECT(fs_pack_weights_tiled(FAKE, 64, 10, 64, FS_DTYPE_BF16, FAKE, 100, NULL), FS_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(fs_workspace_reset(FAKE, 12, NULL), FS_ERR_INVALID_ARGUMENT);
  EXPECT(fs_probe_read_blocks(100, 16), -1);
  printf("checked %ld plans, %d failures\n", checked, failures);
  return failures == 0 ? 0 : 1;
}
