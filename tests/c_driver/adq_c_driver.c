/*
 * A plain C caller of the library, used by tests/test_c_abi_gpu.py: runs
 * AddRmsNormDynamicQuantV2 through the two-phase C calls of include/adq.h on
 * its own HIP stream, with device memory from hipMalloc, and checks the
 * error reporting of phase 1.
 *
 * usage: adq_c_driver DIR
 *   DIR/shape.txt: "m n dtype [mode]" (dtype 1 = F16, 2 = BF16; mode 0 =
 *     the planner's path, 1 = the split-row path's one-launch form set with
 *     adq_executor_set_split, then the same executor run again through the
 *     entry point that allocates nothing, whose outputs must be the same
 *     bytes)
 *   DIR/{x1,x2,gamma,beta,s1,s2}.bin: 16-bit values, row-major
 * writes DIR/{xout,y1,y2,scale1,scale2}.bin (y1 INT8, y2 INT4X2) and prints
 * the executor description, then "ok".
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "adq.h"

#define CHECK_HIP(call)                                                          \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));          \
      exit(2);                                                                   \
    }                                                                            \
  } while (0)

#define CHECK_ADQ(call)                                                          \
  do {                                                                           \
    adq_status s_ = (call);                                                      \
    if (s_ != ADQ_OK) {                                                          \
      fprintf(stderr, "%s returned %d: %s\n", #call, (int)s_, adq_last_error()); \
      exit(3);                                                                   \
    }                                                                            \
  } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(4); }
  void* buf = malloc(bytes);
  if (!buf || fread(buf, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(4); }
  fclose(f);
  return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(4); }
  fclose(f);
}

/* device copy of a host file of `bytes` bytes */
static void* upload(const char* dir, const char* name, size_t bytes) {
  void* host = read_file(dir, name, bytes);
  void* dev = NULL;
  CHECK_HIP(hipMalloc(&dev, bytes));
  CHECK_HIP(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
  free(host);
  return dev;
}

static void download(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes);
  if (!host) exit(4);
  CHECK_HIP(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  write_file(dir, name, host, bytes);
  free(host);
}

static adq_tensor tensor(void* data, int dtype, int ndim, int64_t d0, int64_t d1) {
  adq_tensor t;
  memset(&t, 0, sizeof t);
  t.data = data;
  t.dtype = dtype;
  t.ndim = ndim;
  t.shape[0] = d0;
  t.shape[1] = d1;
  return t;
}

int main(int argc, char** argv) {
  if (argc != 2) { fprintf(stderr, "usage: %s DIR\n", argv[0]); return 1; }
  const char* dir = argv[1];
  long long m = 0, n = 0;
  int dtype = 0, mode = 0;
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/shape.txt", dir);
    FILE* f = fopen(path, "r");
    if (!f || fscanf(f, "%lld %lld %d", &m, &n, &dtype) != 3) { fprintf(stderr, "bad shape.txt\n"); return 4; }
    if (fscanf(f, "%d", &mode) != 1) mode = 0;
    fclose(f);
  }
  const size_t elems = (size_t)m * (size_t)n, row = (size_t)n * 2;
  void* x1 = upload(dir, "x1.bin", elems * 2);
  void* x2 = upload(dir, "x2.bin", elems * 2);
  void* gamma = upload(dir, "gamma.bin", row);
  void* beta = upload(dir, "beta.bin", row);
  void* s1 = upload(dir, "s1.bin", row);
  void* s2 = upload(dir, "s2.bin", row);
  void *xout, *y1, *y2, *sc1, *sc2;
  CHECK_HIP(hipMalloc(&xout, elems * 2));
  CHECK_HIP(hipMalloc(&y1, elems));
  CHECK_HIP(hipMalloc(&y2, elems / 2));
  CHECK_HIP(hipMalloc(&sc1, (size_t)m * 4));
  CHECK_HIP(hipMalloc(&sc2, (size_t)m * 4));

  const adq_tensor tx1 = tensor(x1, dtype, 2, m, n), tx2 = tensor(x2, dtype, 2, m, n);
  const adq_tensor tg = tensor(gamma, dtype, 1, n, 0), tb = tensor(beta, dtype, 1, n, 0);
  const adq_tensor ts1 = tensor(s1, dtype, 1, n, 0), ts2 = tensor(s2, dtype, 1, n, 0);
  const adq_tensor ty1 = tensor(y1, ADQ_INT8, 2, m, n), ty2 = tensor(y2, ADQ_INT4X2, 2, m, n / 2);
  const adq_tensor tsc1 = tensor(sc1, ADQ_F32, 1, m, 0), tsc2 = tensor(sc2, ADQ_F32, 1, m, 0);
  const adq_tensor txo = tensor(xout, dtype, 2, m, n);
  const bool mask[2] = {true, true};

  /* phase 1 rejects a missing input and says why */
  uint64_t ws_size = 0;
  adq_executor* ex = NULL;
  adq_status st = adq_add_rms_norm_dynamic_quant_v2_get_workspace_size(
      NULL, &tx2, &tg, &tb, &ts1, &ts2, 1e-6, mask, &ty1, &ty2, &tsc1, &tsc2, &txo, &ws_size, &ex);
  if (st != ADQ_ERR_NULLPTR || ex != NULL || strlen(adq_last_error()) == 0) {
    fprintf(stderr, "missing x1: status %d, executor %p\n", (int)st, (void*)ex);
    return 5;
  }

  CHECK_ADQ(adq_add_rms_norm_dynamic_quant_v2_get_workspace_size(
      &tx1, &tx2, &tg, &tb, &ts1, &ts2, 1e-6, mask, &ty1, &ty2, &tsc1, &tsc2, &txo, &ws_size, &ex));
  if (mode == 1) {
    const adq_split_config cfg = {0, 1, -1, 0};
    CHECK_ADQ(adq_executor_set_split(ex, &cfg, &ws_size));
  }
  void* ws = NULL;
  if (ws_size) CHECK_HIP(hipMalloc(&ws, ws_size));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  CHECK_ADQ(adq_add_rms_norm_dynamic_quant_v2(ws, ws_size, ex, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  if (mode == 1) {
    /* the same plan through the entry point that allocates nothing: the
       outputs must come out the same, byte for byte */
    const size_t sizes[5] = {elems * 2, elems, elems / 2, (size_t)m * 4, (size_t)m * 4};
    void* outs[5] = {xout, y1, y2, sc1, sc2};
    void* first[5];
    for (int i = 0; i < 5; ++i) {
      first[i] = malloc(sizes[i]);
      if (!first[i]) exit(4);
      CHECK_HIP(hipMemcpy(first[i], outs[i], sizes[i], hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemset(outs[i], 0x5A, sizes[i]));
    }
    CHECK_ADQ(adq_add_rms_norm_dynamic_quant_v2_no_alloc(ex, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    for (int i = 0; i < 5; ++i) {
      void* again = malloc(sizes[i]);
      if (!again) exit(4);
      CHECK_HIP(hipMemcpy(again, outs[i], sizes[i], hipMemcpyDeviceToHost));
      if (memcmp(again, first[i], sizes[i]) != 0) {
        fprintf(stderr, "output %d differs between the two entry points\n", i);
        return 6;
      }
      free(again);
      free(first[i]);
    }
  }
  char desc[512];
  adq_executor_describe(ex, desc, sizeof desc);
  adq_executor_destroy(ex);

  download(dir, "xout.bin", xout, elems * 2);
  download(dir, "y1.bin", y1, elems);
  download(dir, "y2.bin", y2, elems / 2);
  download(dir, "scale1.bin", sc1, (size_t)m * 4);
  download(dir, "scale2.bin", sc2, (size_t)m * 4);
  CHECK_HIP(hipStreamDestroy(stream));
  void* bufs[] = {x1, x2, gamma, beta, s1, s2, xout, y1, y2, sc1, sc2, ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) CHECK_HIP(hipFree(bufs[i]));
  printf("%s\nok\n", desc);
  return 0;
}
