/* A plain C caller that runs the all-reduce through libddpsim.so with
 * nothing but the HIP runtime (no PyTorch): p rank buffers from hipMalloc,
 * ring_allreduce_sim (fused, averaged by p) on a stream, then the inputs and
 * the results are written to <dir>/inputs.bin and <dir>/outputs.bin for the
 * Python test to check against the oracle. Inputs are a fixed integer
 * hash of (rank, index) scaled to [-1, 1).
 *
 * Then the caller that cannot allocate: bf16 buffers all-reduced with the
 * step-by-step ring through ring_allreduce_sim_noalloc, once eagerly and
 * once captured in a HIP graph that is replayed twice (the second replay
 * on the first one's results); inputs and the three results go to
 * <dir>/bf16_*.bin. */
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

static uint16_t to_bf16(float f) {
  union {
    float f;
    uint32_t u;
  } v = {f};
  return (uint16_t)((v.u + 0x7FFFu + ((v.u >> 16) & 1u)) >> 16);
}

static int dump(const char *dir, const char *name, const void *data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (f == NULL) return 1;
  fwrite(data, 1, bytes, f);
  fclose(f);
  return 0;
}

/* bf16 ring through the no-allocation entry point: eager, then a captured
 * graph replayed twice. */
static int bf16_noalloc(const char *dir, hipStream_t stream) {
  enum { P = 4 };
  const int64_t n = 100003;
  const size_t bytes = sizeof(uint16_t) * (size_t)n;
  uint16_t *host = (uint16_t *)malloc(bytes * P);
  void *bufs[P];
  for (int r = 0; r < P; ++r) {
    for (int64_t i = 0; i < n; ++i) {
      host[r * n + i] = to_bf16(input_value((uint32_t)(r + 7), (uint32_t)i));
    }
    CHECK(hipMalloc(&bufs[r], bytes));
  }
  if (dump(dir, "bf16_inputs.bin", host, bytes * P)) return 4;
  const char *names[3] = {"bf16_eager.bin", "bf16_graph1.bin", "bf16_graph2.bin"};
  hipGraph_t graph = NULL;
  hipGraphExec_t exec = NULL;
  for (int run = 0; run < 3; ++run) {
    if (run < 2) {
      for (int r = 0; r < P; ++r) {
        CHECK(hipMemcpy(bufs[r], host + r * n, bytes, hipMemcpyHostToDevice));
      }
    }
    if (run == 0) {
      if (ring_allreduce_sim_noalloc(bufs, P, n, DDP_BF16, DDP_AVG_WORLD, NULL, DDP_ALGO_RING,
                                     stream, NULL) != DDP_OK) {
        fprintf(stderr, "ring_allreduce_sim_noalloc: %s\n", ddp_last_error());
        return 3;
      }
    } else {
      if (run == 1) {
        CHECK(hipStreamBeginCapture(stream, hipStreamCaptureModeRelaxed));
        if (ring_allreduce_sim_noalloc(bufs, P, n, DDP_BF16, DDP_AVG_WORLD, NULL, DDP_ALGO_RING,
                                       stream, NULL) != DDP_OK) {
          fprintf(stderr, "captured ring_allreduce_sim_noalloc: %s\n", ddp_last_error());
          return 3;
        }
        CHECK(hipStreamEndCapture(stream, &graph));
        CHECK(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
      }
      CHECK(hipGraphLaunch(exec, stream));
    }
    CHECK(hipStreamSynchronize(stream));
    uint16_t *out = (uint16_t *)malloc(bytes * P);
    for (int r = 0; r < P; ++r) {
      CHECK(hipMemcpy(out + r * n, bufs[r], bytes, hipMemcpyDeviceToHost));
    }
    if (dump(dir, names[run], out, bytes * P)) return 4;
    free(out);
  }
  CHECK(hipGraphExecDestroy(exec));
  CHECK(hipGraphDestroy(graph));
  for (int r = 0; r < P; ++r) CHECK(hipFree(bufs[r]));
  free(host);
  return 0;
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
  const int rc = bf16_noalloc(argv[1], stream);
  if (rc != 0) return rc;
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
