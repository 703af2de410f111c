/* c_client.c -- a plain C11 program that drives the epilog through the C ABI
 * only (include/kvepi.h and the HIP runtime's C API; no C++, no torch).
 *
 * usage: c_client DIR
 * DIR holds one case, written by tests/test_gpu_c_client.py:
 *   case.txt      "key value" lines: T d x_stride mode group eps_bits x_fp16
 *                 index_mode seq_len rope_dim, and c_num c_size c_head
 *                 c_stride of the cache (a_... of the aux cache when
 *                 aux.bin is there), sizes in elements, eps as its IEEE bits
 *   x.bin slots.bin gamma.bin cos.bin sin.bin cache.bin aux.bin
 * and receives
 *   run.bin / run_aux.bin    the caches after kvepi_run_ex
 *   prep.bin / prep_aux.bin  the caches, reset to their initial bytes, after
 *                            kvepi_prepare_ex and two kvepi_run_prepared
 * It prints one line per step and exits non-zero on any failed call. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvepi.h"

static char dir[4096];

static int64_t get(const char *key) {
  char path[4200], k[64];
  long long v;
  snprintf(path, sizeof path, "%s/case.txt", dir);
  FILE *f = fopen(path, "r");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  while (fscanf(f, "%63s %lld", k, &v) == 2) {
    if (strcmp(k, key) == 0) {
      fclose(f);
      return (int64_t)v;
    }
  }
  fclose(f);
  fprintf(stderr, "case.txt has no %s\n", key);
  exit(2);
}

/* the file's bytes in host memory (*n set to its size); NULL if it is absent */
static void *slurp(const char *name, size_t *n) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  fseek(f, 0, SEEK_END);
  *n = (size_t)ftell(f);
  fseek(f, 0, SEEK_SET);
  void *p = malloc(*n ? *n : 1);
  if (*n && fread(p, 1, *n, f) != *n) {
    fprintf(stderr, "short read of %s\n", path);
    exit(2);
  }
  fclose(f);
  return p;
}

static void spill(const char *name, const void *p, size_t n) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(p, 1, n, f) != n) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

#define HIP(call)                                                        \
  do {                                                                   \
    hipError_t e_ = (call);                                              \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));         \
      exit(3);                                                           \
    }                                                                    \
  } while (0)

#define KV(call)                                                         \
  do {                                                                   \
    kvepi_status s_ = (call);                                            \
    printf("%s -> %s\n", #call, kvepi_status_str(s_));                   \
    if (s_ != KVEPI_OK) exit(4);                                         \
  } while (0)

/* a device copy of file `name` (NULL, size 0 if absent) */
static void *upload(const char *name, size_t *n) {
  size_t sz = 0;
  void *h = slurp(name, &sz);
  if (!h) {
    *n = 0;
    return NULL;
  }
  void *d = NULL;
  HIP(hipMalloc(&d, sz ? sz : 1));
  HIP(hipMemcpy(d, h, sz, hipMemcpyHostToDevice));
  free(h);
  *n = sz;
  return d;
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  snprintf(dir, sizeof dir, "%s", argv[1]);
  const int64_t T = get("T"), d = get("d"), xs = get("x_stride");
  const int32_t mode = (int32_t)get("mode"), group = (int32_t)get("group");
  const uint32_t eps_bits = (uint32_t)get("eps_bits");
  float eps;
  memcpy(&eps, &eps_bits, 4);

  size_t nx, ns, ng, nc, nsn, ncache, naux;
  void *x = upload("x.bin", &nx), *slots = upload("slots.bin", &ns);
  void *gamma = upload("gamma.bin", &ng), *cs = upload("cos.bin", &nc);
  void *sn = upload("sin.bin", &nsn);
  void *cache = upload("cache.bin", &ncache), *aux = upload("aux.bin", &naux);
  size_t n0, a0;
  void *cache_init = slurp("cache.bin", &n0);
  void *aux_init = aux ? slurp("aux.bin", &a0) : NULL;

  kvepi_cache c = {cache, get("c_num"), get("c_size"), get("c_head"), get("c_stride")};
  kvepi_cache a = {aux, 0, 0, 0, 0};
  if (aux) {
    a.block_num = get("a_num");
    a.block_size = get("a_size");
    a.head_dim = get("a_head");
    a.block_stride = get("a_stride");
  }
  kvepi_options opt = {(int32_t)get("x_fp16"), (int32_t)get("index_mode"), get("seq_len"),
                       (int32_t)get("rope_dim"), 0};

  uint64_t ws = 1;
  KV(kvepi_get_workspace_ex(x, T, d, xs, gamma, cs, sn, (const int32_t *)slots, &c,
                            aux ? &a : NULL, mode, group, eps, &opt, &ws));
  if (ws != 0) {
    fprintf(stderr, "workspace %llu, expected 0\n", (unsigned long long)ws);
    return 5;
  }
  hipStream_t stream;
  HIP(hipStreamCreate(&stream));
  KV(kvepi_run_ex(x, T, d, xs, gamma, cs, sn, (const int32_t *)slots, &c, aux ? &a : NULL,
                  mode, group, eps, &opt, NULL, 0, stream));
  HIP(hipStreamSynchronize(stream));
  void *out = malloc(ncache), *aout = aux ? malloc(naux) : NULL;
  HIP(hipMemcpy(out, cache, ncache, hipMemcpyDeviceToHost));
  spill("run.bin", out, ncache);
  if (aux) {
    HIP(hipMemcpy(aout, aux, naux, hipMemcpyDeviceToHost));
    spill("run_aux.bin", aout, naux);
  }

  /* the prepared call, run twice on the caches reset to their initial bytes */
  HIP(hipMemcpy(cache, cache_init, ncache, hipMemcpyHostToDevice));
  if (aux) HIP(hipMemcpy(aux, aux_init, naux, hipMemcpyHostToDevice));
  kvepi_prepared prep;
  KV(kvepi_prepare_ex(x, T, d, xs, gamma, cs, sn, (const int32_t *)slots, &c, aux ? &a : NULL,
                      mode, group, eps, &opt, &prep));
  kvepi_prepared copy;
  memcpy(&copy, &prep, sizeof copy); /* a bytewise copy runs as well */
  KV(kvepi_run_prepared(&prep, stream));
  KV(kvepi_run_prepared(&copy, stream));
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(out, cache, ncache, hipMemcpyDeviceToHost));
  spill("prep.bin", out, ncache);
  if (aux) {
    HIP(hipMemcpy(aout, aux, naux, hipMemcpyDeviceToHost));
    spill("prep_aux.bin", aout, naux);
  }

  /* a struct that no preparation filled is refused, and launches nothing */
  kvepi_prepared zero;
  memset(&zero, 0, sizeof zero);
  const kvepi_status st = kvepi_run_prepared(&zero, stream);
  printf("kvepi_run_prepared(unprepared) -> %s\n", kvepi_status_str(st));
  if (st != KVEPI_ERR_PARAM) return 6;

  HIP(hipStreamDestroy(stream));
  void *bufs[] = {x, slots, gamma, cs, sn, cache, aux};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) HIP(hipFree(bufs[i]));
  free(out);
  free(aout);
  free(cache_init);
  free(aux_init);
  printf("c_client ok\n");
  return 0;
}
