/* pa_cache_write + pa_decode driven from C through the HIP runtime's C API
 * (no Python, no torch in this program). Reads a batch from a folder of raw
 * files written by the test (meta.txt: S Hq Hkv D B num_blocks max_blocks T scale;
 * k.bin, v.bin: bf16 [T][Hkv][D]; slots.bin: int64 [T]; q.bin: bf16
 * [S][Hq][D]; tables.bin: int32 [S][max_blocks]; lens.bin: int32 [S]),
 * writes the new tokens into a bf16 pool, decodes, and writes out.bin (bf16
 * [S][Hq][D]); the test compares it with the fp64 oracle. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pagedkv.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 2;                                                             \
    }                                                                       \
  } while (0)
#define CHECK_PA(x)                                                         \
  do {                                                                      \
    pa_status s_ = (x);                                                     \
    if (s_ != PA_OK) {                                                      \
      fprintf(stderr, "%s: %s (%s)\n", #x, pa_status_string(s_), pa_last_error()); \
      return 3;                                                             \
    }                                                                       \
  } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  const size_t got = fread(p, 1, bytes, f);
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int upload(void** dev, const void* host, size_t bytes) {
  if (hipMalloc(dev, bytes ? bytes : 16) != hipSuccess) return 1;
  if (bytes && hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return 1;
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: gpu_decode <folder>\n");
    return 1;
  }
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", dir);
  FILE* mf = fopen(path, "r");
  int S, Hq, Hkv, D, B, nb, maxb, T;
  float scale;
  if (!mf || fscanf(mf, "%d %d %d %d %d %d %d %d %f", &S, &Hq, &Hkv, &D, &B, &nb, &maxb, &T,
                    &scale) != 9) {
    fprintf(stderr, "bad meta.txt\n");
    return 1;
  }
  fclose(mf);
  const size_t row = (size_t)Hkv * D * 2, qrow = (size_t)Hq * D * 2;
  void* k = read_file(dir, "k.bin", (size_t)T * row);
  void* v = read_file(dir, "v.bin", (size_t)T * row);
  void* slots = read_file(dir, "slots.bin", (size_t)T * 8);
  void* q = read_file(dir, "q.bin", (size_t)S * qrow);
  void* tables = read_file(dir, "tables.bin", (size_t)S * maxb * 4);
  void* lens = read_file(dir, "lens.bin", (size_t)S * 4);
  if (!k || !v || !slots || !q || !tables || !lens) {
    fprintf(stderr, "missing input file\n");
    return 1;
  }

  const size_t pool_bytes = (size_t)nb * Hkv * B * D * 2;
  pa_pool pool;
  memset(&pool, 0, sizeof pool);
  CHECK_HIP(hipMalloc(&pool.k_pool, pool_bytes));
  CHECK_HIP(hipMalloc(&pool.v_pool, pool_bytes));
  pool.num_blocks = nb;
  pool.num_kv_heads = Hkv;
  pool.block_size = B;
  pool.head_dim = D;
  pool.dtype = PA_BF16;
  pool.k_scale = pool.v_scale = 1.0f;

  void *dk, *dv, *dslots, *dq, *dtables, *dlens, *dout, *ws;
  if (upload(&dk, k, (size_t)T * row) || upload(&dv, v, (size_t)T * row) ||
      upload(&dslots, slots, (size_t)T * 8) || upload(&dq, q, (size_t)S * qrow) ||
      upload(&dtables, tables, (size_t)S * maxb * 4) || upload(&dlens, lens, (size_t)S * 4)) {
    fprintf(stderr, "upload failed\n");
    return 2;
  }
  CHECK_HIP(hipMalloc(&dout, (size_t)S * qrow));
  const size_t ws_bytes = pa_decode_workspace_bytes(S, Hq, Hkv, D, 0);
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  hipStream_t st;
  CHECK_HIP(hipStreamCreate(&st));

  /* host checks of the arrays, then the two device calls on one stream */
  CHECK_PA(pa_check_slots(&pool, (const int64_t*)slots, T));
  CHECK_PA(pa_check_batch(&pool, (const int32_t*)tables, maxb, (const int32_t*)lens, S));
  CHECK_PA(pa_cache_write(&pool, dk, dv, (const int64_t*)dslots, T, (void*)st));
  CHECK_PA(pa_decode(dout, dq, &pool, (const int32_t*)dtables, maxb, (const int32_t*)dlens, S, Hq,
                     scale, 0, ws, ws_bytes, (void*)st));
  CHECK_HIP(hipStreamSynchronize(st));

  void* out = malloc((size_t)S * qrow);
  CHECK_HIP(hipMemcpy(out, dout, (size_t)S * qrow, hipMemcpyDeviceToHost));
  snprintf(path, sizeof path, "%s/out.bin", dir);
  FILE* of = fopen(path, "wb");
  if (!of || fwrite(out, 1, (size_t)S * qrow, of) != (size_t)S * qrow) {
    fprintf(stderr, "cannot write out.bin\n");
    return 1;
  }
  fclose(of);
  printf("decoded %d sequences\n", S);
  return 0;
}
