/* Drives the library through its C ABI alone (no Python): row-major and tiled
 * weights, the fused and the unfused entry points, and one validation error.
 * Inputs are bf16 values from a fixed LCG; the program writes them to
 * <outdir>/H.bin and <outdir>/W.bin (raw bf16 bits, row-major) so a test can
 * check the printed tokens against the oracle.
 *
 * usage: sample_from_c OUTDIR B D V T SEED STEP
 * prints: "rows <tokens...>", "tiled <tokens...>", "unfused <tokens...>" and
 * "error <status name>"; exit status 0 when every call behaved. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flashsample.h"

#define CHECK_HIP(x)                                                       \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));              \
      return 2;                                                            \
    }                                                                      \
  } while (0)
#define CHECK_FS(x)                                                        \
  do {                                                                     \
    fs_status_t s_ = (x);                                                  \
    if (s_ != FS_OK) {                                                     \
      fprintf(stderr, "%s: %s\n", #x, fs_status_string(s_));               \
      return 3;                                                            \
    }                                                                      \
  } while (0)

static uint32_t lcg_state = 12345u;
static float next_uniform(void) { /* in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

static uint16_t to_bf16(float f) { /* round to nearest even (finite inputs) */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static int write_file(const char* dir, const char* name, const void* p, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, n, f) != n) return 1;
  fclose(f);
  return 0;
}

static void print_tokens(const char* tag, const int32_t* t, int64_t B) {
  printf("%s", tag);
  for (int64_t b = 0; b < B; ++b) printf(" %d", t[b]);
  printf("\n");
}

int main(int argc, char** argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s OUTDIR B D V T SEED STEP\n", argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  const int64_t B = atoll(argv[2]), D = atoll(argv[3]), V = atoll(argv[4]);
  const float T = (float)atof(argv[5]);
  const uint64_t seed = strtoull(argv[6], NULL, 10), step = strtoull(argv[7], NULL, 10);

  uint16_t* h = malloc((size_t)(B * D) * 2);
  uint16_t* w = malloc((size_t)(V * D) * 2);
  int32_t* tok = malloc((size_t)B * 4);
  if (!h || !w || !tok) return 2;
  for (int64_t i = 0; i < B * D; ++i) h[i] = to_bf16(next_uniform());
  for (int64_t i = 0; i < V * D; ++i) w[i] = to_bf16(next_uniform() * 0.1f);
  if (write_file(dir, "H.bin", h, (size_t)(B * D) * 2) || write_file(dir, "W.bin", w, (size_t)(V * D) * 2)) return 2;

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  void *dh, *dw, *dtiled, *dws, *duws;
  int32_t* dout;
  CHECK_HIP(hipMalloc(&dh, (size_t)(B * D) * 2));
  CHECK_HIP(hipMalloc(&dw, (size_t)(V * D) * 2));
  CHECK_HIP(hipMalloc((void**)&dout, (size_t)B * 4));
  CHECK_HIP(hipMemcpy(dh, h, (size_t)(B * D) * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dw, w, (size_t)(V * D) * 2, hipMemcpyHostToDevice));

  /* row-major weights, plain fused call */
  const size_t ws = fs_workspace_bytes(B, D, V, FS_DTYPE_BF16);
  if (ws == 0) return 3;
  CHECK_HIP(hipMalloc(&dws, ws));
  CHECK_FS(fs_sample_fused(dh, D, dw, D, FS_DTYPE_BF16, B, D, V, T, seed, step, dws, ws, dout, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(tok, dout, (size_t)B * 4, hipMemcpyDeviceToHost));
  print_tokens("rows", tok, B);

  /* the same head repacked once into the tiled layout */
  const size_t tb = fs_tiled_weights_bytes(V, D, FS_DTYPE_BF16);
  if (tb == 0) return 3;
  CHECK_HIP(hipMalloc(&dtiled, tb));
  CHECK_FS(fs_pack_weights_tiled(dw, D, V, D, FS_DTYPE_BF16, dtiled, tb, stream));
  fs_options_t o;
  memset(&o, 0, sizeof o);
  o.weights_layout = FS_LAYOUT_TILED;
  const size_t ws2 = fs_workspace_bytes_ex(B, D, V, FS_DTYPE_BF16, &o);
  void* dws2;
  CHECK_HIP(hipMalloc(&dws2, ws2));
  CHECK_FS(fs_sample_fused_ex(dh, D, dtiled, 0, FS_DTYPE_BF16, B, D, V, T, seed, step, dws2, ws2, dout, stream, &o));
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(tok, dout, (size_t)B * 4, hipMemcpyDeviceToHost));
  print_tokens("tiled", tok, B);

  /* the unfused baseline: fp32 logits in the workspace, then a sampler */
  const size_t uws = fs_unfused_workspace_bytes(B, D, V, FS_DTYPE_BF16, FS_DTYPE_F32);
  CHECK_HIP(hipMalloc(&duws, uws));
  CHECK_FS(fs_sample_unfused(dh, D, dw, D, FS_DTYPE_BF16, B, D, V, T, seed, step, FS_DTYPE_F32, duws, uws, dout,
                             stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(tok, dout, (size_t)B * 4, hipMemcpyDeviceToHost));
  print_tokens("unfused", tok, B);

  /* validation: a null output pointer is refused before anything runs */
  const fs_status_t bad = fs_sample_fused(dh, D, dw, D, FS_DTYPE_BF16, B, D, V, T, seed, step, dws, ws, NULL, stream);
  printf("error %s\n", fs_status_string(bad));

  hipFree(duws);
  hipFree(dws2);
  hipFree(dtiled);
  hipFree(dws);
  hipFree(dout);
  hipFree(dw);
  hipFree(dh);
  hipStreamDestroy(stream);
  free(tok);
  free(w);
  free(h);
  return bad == FS_ERR_INVALID_ARGUMENT ? 0 : 4;
}
