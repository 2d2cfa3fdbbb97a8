/* A plain C caller that runs the all-reduce through libddpsim.so with
 * nothing but the HIP runtime (no PyTorch): p rank buffers from hipMalloc,
 * ring_allreduce_sim (fused, averaged by p) on a stream, then the inputs and
 * the results are written to <dir>/inputs.bin and <dir>/outputs.bin for the
 * Python test to check against the oracle. Inputs are a fixed integer
 * hash of (rank, index) scaled to [-1, 1). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ddpsim.h"

#define CHECK(x)                                                            \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      return 2;                                                             \
    }                                                                       \
  } while (0)

static float input_value(uint32_t r, uint32_t i) {
  uint32_t h = r * 0x9E3779B1u ^ (i + 0x7F4A7C15u) * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 13;
  return (float)(int32_t)(h >> 8) / (float)(1 << 23) - 1.0f;
}

int main(int argc, char **argv) {
  if (argc != 2) return 1;
  const int p = 4;
  const int64_t n = 1000003;
  float *host = (float *)malloc(sizeof(float) * (size_t)(p * n));
  void *bufs[4];
  for (int r = 0; r < p; ++r) {
    for (int64_t i = 0; i < n; ++i) host[r * n + i] = input_value((uint32_t)r, (uint32_t)i);
    CHECK(hipMalloc(&bufs[r], sizeof(float) * (size_t)n));
    CHECK(hipMemcpy(bufs[r], host + r * n, sizeof(float) * (size_t)n, hipMemcpyHostToDevice));
  }
  char path[4096];
  snprintf(path, sizeof path, "%s/inputs.bin", argv[1]);
  FILE *f = fopen(path, "wb");
  fwrite(host, sizeof(float), (size_t)(p * n), f);
  fclose(f);
  hipStream_t stream;
  CHECK(hipStreamCreate(&stream));
  ddp_comm_stats st;
  ddp_status s = ring_allreduce_sim(bufs, p, n, DDP_F32, DDP_AVG_WORLD, NULL, DDP_ALGO_FUSED,
                                    NULL, 0, stream, &st);
  if (s != DDP_OK) {
    fprintf(stderr, "ring_allreduce_sim: %s\n", ddp_last_error());
    return 3;
  }
  CHECK(hipStreamSynchronize(stream));
  for (int r = 0; r < p; ++r) {
    CHECK(hipMemcpy(host + r * n, bufs[r], sizeof(float) * (size_t)n, hipMemcpyDeviceToHost));
    CHECK(hipFree(bufs[r]));
  }
  CHECK(hipStreamDestroy(stream));
  snprintf(path, sizeof path, "%s/outputs.bin", argv[1]);
  f = fopen(path, "wb");
  fwrite(host, sizeof(float), (size_t)(p * n), f);
  fclose(f);
  printf("steps %lld messages %lld bytes_sent_per_rank %lld\n", (long long)st.steps,
         (long long)st.messages, (long long)st.bytes_sent_per_rank);
  free(host);
  return 0;
}
