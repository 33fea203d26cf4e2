/*
 * A plain C consumer of libpagedattn: include/pagedattn.h compiled as C, the
 * library linked directly, device memory from the HIP runtime, no Python.
 *
 *   decode_step check      host-side checks only (never touches a GPU):
 *                          version, status strings, an argument error.
 *   decode_step run DIR    one decode step from raw little-endian files in
 *                          DIR: the slots of one new token per sequence
 *                          (pa_slot_mapping), their cache write
 *                          (pa_reshape_and_cache), then
 *                          pa_paged_attention_decode; writes DIR/out.bin,
 *                          DIR/k_out.bin, DIR/v_out.bin and DIR/slots.bin.
 *
 * DIR/meta.txt holds "S H D B N M max_ctx scale" (fp16 elements); the inputs
 * are q.bin [S][H][D], k.bin / v.bin [N][H][B][D], tables.bin int32 [S][M],
 * ctx.bin int32 [S], new_k.bin / new_v.bin [S][H][D], seq.bin / pos.bin int32 [S]
 * (sequence and position of each new token).
 * Exit status 0 on success; on failure the status and pa_last_error() are
 * printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pagedattn.h"

static int fail(const char *what, pa_status st) {
  fprintf(stderr, "%s: %s (%s)\n", what, pa_status_string(st), pa_last_error());
  return 1;
}

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *p = malloc(bytes ? bytes : 1);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char *dir, const char *name, const void *p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return 1;
  size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put != bytes;
}

/* Device copy of a host buffer (NULL on failure). */
static void *to_device(const void *h, size_t bytes) {
  void *d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) return NULL;
  if (bytes && hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

static int check(void) {
  if (pa_abi_version() < 1) return fail("pa_abi_version", PA_ERR_INVALID_ARG);
  if (strcmp(pa_status_string(PA_OK), "") == 0) return fail("pa_status_string", PA_ERR_INVALID_ARG);
  /* A null key pointer is refused on the host, before any device call. */
  pa_status st = pa_reshape_and_cache(NULL, NULL, 64, 64, NULL, NULL, NULL, 1, 1, 64, 16, 4, PA_F16, NULL);
  if (st != PA_ERR_INVALID_ARG || pa_last_error()[0] == '\0') {
    fprintf(stderr, "expected PA_ERR_INVALID_ARG with a message, got %d\n", (int)st);
    return 1;
  }
  printf("check ok: abi %d, refused: %s\n", pa_abi_version(), pa_last_error());
  return 0;
}

static int run(const char *dir) {
  int S, H, D, B, M, max_ctx;
  long long N;
  float scale;
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", dir);
  FILE *mf = fopen(path, "r");
  if (!mf) return fail("meta.txt", PA_ERR_INVALID_ARG);
  int got = fscanf(mf, "%d %d %d %d %lld %d %d %f", &S, &H, &D, &B, &N, &M, &max_ctx, &scale);
  fclose(mf);
  if (got != 8 || S <= 0 || H <= 0 || D <= 0 || B <= 0 || N <= 0 || M <= 0) return fail("meta.txt", PA_ERR_INVALID_ARG);

  const size_t e = 2; /* fp16 */
  const size_t qb = (size_t)S * H * D * e, cb = (size_t)N * H * B * D * e;
  void *hq = read_file(dir, "q.bin", qb), *hk = read_file(dir, "k.bin", cb), *hv = read_file(dir, "v.bin", cb);
  void *ht = read_file(dir, "tables.bin", (size_t)S * M * 4), *hc = read_file(dir, "ctx.bin", (size_t)S * 4);
  void *hnk = read_file(dir, "new_k.bin", qb), *hnv = read_file(dir, "new_v.bin", qb);
  void *hseq = read_file(dir, "seq.bin", (size_t)S * 4), *hpos = read_file(dir, "pos.bin", (size_t)S * 4);
  if (!hq || !hk || !hv || !ht || !hc || !hnk || !hnv || !hseq || !hpos)
    return fail("reading inputs", PA_ERR_INVALID_ARG);

  void *q = to_device(hq, qb), *k = to_device(hk, cb), *v = to_device(hv, cb);
  void *tables = to_device(ht, (size_t)S * M * 4), *ctx = to_device(hc, (size_t)S * 4);
  void *nk = to_device(hnk, qb), *nv = to_device(hnv, qb);
  void *seq = to_device(hseq, (size_t)S * 4), *pos = to_device(hpos, (size_t)S * 4);
  void *out = NULL, *slots = NULL;
  if (!q || !k || !v || !tables || !ctx || !nk || !nv || !seq || !pos || hipMalloc(&out, qb) != hipSuccess ||
      hipMalloc(&slots, (size_t)S * 8) != hipSuccess)
    return fail("device buffers", PA_ERR_HIP);

  /* The step: translate the new tokens' positions to slots, write them,
     then attend (the null stream). */
  pa_status st = pa_slot_mapping((const int32_t *)tables, M, S, (const int32_t *)seq, (const int32_t *)pos, S, B, N,
                                 (int64_t *)slots, NULL);
  if (st != PA_OK) return fail("pa_slot_mapping", st);
  st = pa_reshape_and_cache(nk, nv, (int64_t)H * D, (int64_t)H * D, k, v, (const int64_t *)slots, S, H, D,
                                      B, N, PA_F16, NULL);
  if (st != PA_OK) return fail("pa_reshape_and_cache", st);
  const size_t wsb = pa_decode_workspace_bytes(S, H, D, max_ctx, B, 0);
  void *ws = NULL;
  if (wsb == 0 || hipMalloc(&ws, wsb) != hipSuccess) return fail("workspace", PA_ERR_WORKSPACE);
  st = pa_paged_attention_decode(out, q, k, v, (const int32_t *)tables, M, (const int32_t *)ctx, max_ctx, S, H, D, B,
                                 N, scale, PA_F16, 0, ws, wsb, NULL);
  if (st != PA_OK) return fail("pa_paged_attention_decode", st);
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", PA_ERR_HIP);

  void *hout = malloc(qb), *hslots = malloc((size_t)S * 8);
  if (!hout || hipMemcpy(hout, out, qb, hipMemcpyDeviceToHost) != hipSuccess) return fail("copy out", PA_ERR_HIP);
  if (!hslots || hipMemcpy(hslots, slots, (size_t)S * 8, hipMemcpyDeviceToHost) != hipSuccess)
    return fail("copy slots", PA_ERR_HIP);
  if (hipMemcpy(hk, k, cb, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hv, v, cb, hipMemcpyDeviceToHost) != hipSuccess)
    return fail("copy caches", PA_ERR_HIP);
  if (write_file(dir, "out.bin", hout, qb) || write_file(dir, "k_out.bin", hk, cb) ||
      write_file(dir, "v_out.bin", hv, cb) || write_file(dir, "slots.bin", hslots, (size_t)S * 8))
    return fail("writing outputs", PA_ERR_INVALID_ARG);
  printf("run ok: %d sequences, %d heads\n", S, H);
  return 0;
}

int main(int argc, char **argv) {
  if (argc == 2 && strcmp(argv[1], "check") == 0) return check();
  if (argc == 3 && strcmp(argv[1], "run") == 0) return run(argv[2]);
  fprintf(stderr, "usage: %s check | run DIR\n", argv[0]);
  return 2;
}
