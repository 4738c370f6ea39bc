/*
 * A stream driven through the C ABI from plain C (no Python, no torch): device buffers from
 * hipMalloc, one hipStream, the step protocol of sdv2.h.
 *
 *   c_abi_driver <inputs> <outputs>
 *
 * <inputs>:  the sdv2_config struct as laid out in sdv2.h, int64 num_chunks, float scale, then
 *            for every step with a non-empty stream batch (schedule from sdv2_plan_step): for
 *            every layer q, k, v, each [nbatch][T'N][H][d] in the activation dtype, and, when
 *            the step commits a chunk and embed_dim > 0, that chunk's fp32 embedding.
 * <outputs>: for the same steps and layers, the attention output [nbatch][T'N][H][d], and
 *            after each commit with an embedding the sink decision: int64 slot (j* if
 *            replaced, else -1, also when no decision was taken), double alpha_j* (1 when no
 *            decision was taken).
 * Exit status 0 on success; any failing call prints its sdv2_last_error() text and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "sdv2.h"

#define CHECK_HIP(x)                                                           \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

#define CHECK_SDV2(x)                                                          \
  do {                                                                         \
    int rc_ = (x);                                                             \
    if (rc_ != SDV2_OK) {                                                      \
      fprintf(stderr, "%s: %d %s\n", #x, rc_, sdv2_last_error());              \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

static void read_exact(FILE* f, void* p, size_t n) {
  if (fread(p, 1, n, f) != n) {
    fprintf(stderr, "short input file\n");
    exit(1);
  }
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <inputs> <outputs>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  FILE* out = fopen(argv[2], "wb");
  if (!in || !out) {
    fprintf(stderr, "cannot open the files\n");
    return 1;
  }
  sdv2_config cfg;
  int64_t num_chunks;
  float scale;
  read_exact(in, &cfg, sizeof cfg);
  read_exact(in, &num_chunks, sizeof num_chunks);
  read_exact(in, &scale, sizeof scale);
  CHECK_SDV2(sdv2_config_validate(&cfg));

  size_t kv_bytes = 0, meta_bytes = 0, ws_bytes = 0;
  CHECK_SDV2(sdv2_cache_size(&cfg, &kv_bytes, &meta_bytes, &ws_bytes));
  void *d_kv = NULL, *d_meta = NULL, *d_ws = NULL;
  CHECK_HIP(hipMalloc(&d_kv, kv_bytes));
  CHECK_HIP(hipMalloc(&d_meta, meta_bytes));
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes > 0 ? ws_bytes : 256));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  sdv2_cache* cache = NULL;
  CHECK_SDV2(sdv2_cache_create(&cfg, d_kv, kv_bytes, d_meta, meta_bytes, d_ws, ws_bytes, stream, &cache));

  const size_t eb = cfg.dtype == SDV2_F32 ? 4 : 2;   /* activation bytes */
  const size_t rows = (size_t)cfg.chunk_frames * cfg.grid_h * cfg.grid_w;
  const size_t elem_bytes = rows * cfg.num_heads * cfg.head_dim * eb;   /* one element's q (k, v, out) */
  const size_t max_bytes = elem_bytes * cfg.stream_batch;
  void *d_q = NULL, *d_k = NULL, *d_v = NULL, *d_o = NULL;
  CHECK_HIP(hipMalloc(&d_q, max_bytes));
  CHECK_HIP(hipMalloc(&d_k, max_bytes));
  CHECK_HIP(hipMalloc(&d_v, max_bytes));
  CHECK_HIP(hipMalloc(&d_o, max_bytes));
  char* h = (char*)malloc(max_bytes);
  if (!h) return 1;
  float* d_embed = NULL;
  float* h_embed = NULL;
  if (cfg.embed_dim > 0) {
    CHECK_HIP(hipMalloc((void**)&d_embed, sizeof(float) * cfg.embed_dim));
    h_embed = (float*)malloc(sizeof(float) * cfg.embed_dim);
    if (!h_embed) return 1;
  }

  const int64_t num_steps = num_chunks + cfg.stream_batch - 1;
  int steps_run = 0;
  for (int64_t s = 0; s < num_steps; ++s) {
    int64_t first = 0, commit = -1, newest = -1;
    int32_t nb = 0;
    CHECK_SDV2(sdv2_plan_step(&cfg, num_chunks, s, &first, &nb, &commit, &newest));
    if (nb == 0) continue;
    int32_t applied = 0;
    CHECK_SDV2(sdv2_rope_refresh(cache, newest, &applied, stream));
    const size_t bytes = elem_bytes * (size_t)nb;
    for (int32_t layer = 0; layer < cfg.num_layers; ++layer) {
      void* dst[3] = {d_q, d_k, d_v};
      for (int j = 0; j < 3; ++j) {
        read_exact(in, h, bytes);
        CHECK_HIP(hipMemcpyAsync(dst[j], h, bytes, hipMemcpyHostToDevice, stream));
        CHECK_HIP(hipStreamSynchronize(stream));   /* h is reused for the next tensor */
      }
      CHECK_SDV2(sdv2_cache_append(cache, layer, first, nb, d_q, d_k, d_v, stream));
      CHECK_SDV2(sdv2_chunk_attention(cache, layer, nb, d_q, d_o, scale, stream));
      CHECK_HIP(hipMemcpyAsync(h, d_o, bytes, hipMemcpyDeviceToHost, stream));
      CHECK_HIP(hipStreamSynchronize(stream));
      if (fwrite(h, 1, bytes, out) != bytes) return 1;
    }
    if (commit >= 0) {
      CHECK_SDV2(sdv2_cache_commit(cache, commit, stream));
      if (cfg.embed_dim > 0) {
        read_exact(in, h_embed, sizeof(float) * cfg.embed_dim);
        CHECK_HIP(hipMemcpyAsync(d_embed, h_embed, sizeof(float) * cfg.embed_dim, hipMemcpyHostToDevice, stream));
        int32_t slot = -3;                    /* the call always writes it */
        double alpha = 0.0;
        const int64_t last_frame = (commit + 1) * cfg.chunk_frames - 1;
        CHECK_SDV2(sdv2_sink_replace(cache, last_frame, d_embed, NULL, NULL, 0, NULL, &slot, &alpha, stream));
        const int64_t slot64 = slot;
        if (fwrite(&slot64, sizeof slot64, 1, out) != 1 || fwrite(&alpha, sizeof alpha, 1, out) != 1) return 1;
      }
    }
    ++steps_run;
  }
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_SDV2(sdv2_cache_destroy(cache));
  free(h);
  free(h_embed);
  if (d_embed) hipFree(d_embed);
  hipFree(d_q);
  hipFree(d_k);
  hipFree(d_v);
  hipFree(d_o);
  hipFree(d_kv);
  hipFree(d_meta);
  hipFree(d_ws);
  hipStreamDestroy(stream);
  fclose(in);
  fclose(out);
  printf("c_abi_driver: %d steps\n", steps_run);
  return 0;
}
