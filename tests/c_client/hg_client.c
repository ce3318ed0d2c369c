/*
 * A plain C client of libhg.so: no Python, no torch, only the C ABI in
 * include/hg.h and the HIP runtime for device memory and a stream. The gather
 * tests drive it with seeded inputs and check what it writes against the CPU
 * oracle.
 *
 * usage: hg_client IN OUT
 * IN:  int32 tp, shard, cap, m, calls, variant (0: hg_gather, 1: hg_push +
 *      hg_collect, 2: hg_gather_static, which leaves the context untouched),
 *      then `calls` input sets of tp x m x shard BF16 (uint16).
 * OUT: per call m x tp*shard BF16 outputs; then int32 parity; then both
 *      mailbox parities, cap x tp*shard BF16 each.
 * Exit status 0 on success; otherwise the failing step goes to stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "hg.h"

static int fail(const char *what, int code) {
  fprintf(stderr, "hg_client: %s failed (%d: %s; %s)\n", what, code, hg_strerror(code),
          hg_last_error_detail());
  return 1;
}

#define HIP_OK(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "hg_client: %s: %s\n", #expr, hipGetErrorString(e_));       \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

static int read_all(FILE *f, void *p, size_t n) { return fread(p, 1, n, f) == n; }
static int write_all(FILE *f, const void *p, size_t n) { return fwrite(p, 1, n, f) == n; }

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: hg_client IN OUT\n");
    return 2;
  }
  FILE *in = fopen(argv[1], "rb");
  FILE *out = fopen(argv[2], "wb");
  if (!in || !out) {
    fprintf(stderr, "hg_client: cannot open the input or the output file\n");
    return 1;
  }
  int32_t hdr[6];
  if (!read_all(in, hdr, sizeof hdr)) return fail("reading the header", HG_EINVAL);
  const int tp = hdr[0], shard = hdr[1], cap = hdr[2], m = hdr[3], calls = hdr[4], variant = hdr[5];
  if (tp < 1 || tp > HG_MAX_TP || shard < 1 || m < 1 || m > cap || calls < 1) {
    fprintf(stderr, "hg_client: bad header\n");
    return 1;
  }
  const size_t shard_bytes = (size_t)m * shard * 2;
  const size_t row_bytes = (size_t)tp * shard * 2;

  HIP_OK(hipSetDevice(0));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  hg_ctx *h = NULL;
  int rc = hg_create(tp, shard, cap, &h);
  if (rc != HG_OK) return fail("hg_create", rc);

  void *dev_shards[HG_MAX_TP];
  void *dev_out = NULL, *dev_box = NULL;
  for (int r = 0; r < tp; ++r) HIP_OK(hipMalloc(&dev_shards[r], shard_bytes));
  HIP_OK(hipMalloc(&dev_out, (size_t)m * row_bytes));
  HIP_OK(hipMalloc(&dev_box, (size_t)cap * row_bytes));
  unsigned char *host = malloc(shard_bytes > (size_t)cap * row_bytes ? shard_bytes : (size_t)cap * row_bytes);
  if (!host) return fail("malloc", HG_ENOMEM);

  for (int c = 0; c < calls; ++c) {
    for (int r = 0; r < tp; ++r) {
      if (!read_all(in, host, shard_bytes)) return fail("reading an input set", HG_EINVAL);
      HIP_OK(hipMemcpy(dev_shards[r], host, shard_bytes, hipMemcpyHostToDevice));
    }
    if (variant == 0) {
      rc = hg_gather(h, (const void *const *)dev_shards, m, dev_out, s);
      if (rc != HG_OK) return fail("hg_gather", rc);
    } else if (variant == 2) {
      rc = hg_gather_static(tp, shard, (const void *const *)dev_shards, m, dev_out, s);
      if (rc != HG_OK) return fail("hg_gather_static", rc);
    } else {
      rc = hg_push(h, (const void *const *)dev_shards, m, s);
      if (rc != HG_OK) return fail("hg_push", rc);
      rc = hg_collect(h, m, dev_out, s);
      if (rc != HG_OK) return fail("hg_collect", rc);
    }
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(host, dev_out, (size_t)m * row_bytes, hipMemcpyDeviceToHost));
    if (!write_all(out, host, (size_t)m * row_bytes)) return fail("writing an output", HG_EINVAL);
  }
  rc = hg_poll_status(h, s);
  if (rc != HG_OK) return fail("hg_poll_status", rc);
  const int32_t parity = hg_parity(h);
  if (!write_all(out, &parity, sizeof parity)) return fail("writing the parity", HG_EINVAL);
  for (int p = 0; p < 2; ++p) {
    rc = hg_copy_mailbox(h, p, dev_box, s);
    if (rc != HG_OK) return fail("hg_copy_mailbox", rc);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(host, dev_box, (size_t)cap * row_bytes, hipMemcpyDeviceToHost));
    if (!write_all(out, host, (size_t)cap * row_bytes)) return fail("writing a mailbox", HG_EINVAL);
  }
  rc = hg_destroy(h);
  if (rc != HG_OK) return fail("hg_destroy", rc);
  for (int r = 0; r < tp; ++r) HIP_OK(hipFree(dev_shards[r]));
  HIP_OK(hipFree(dev_out));
  HIP_OK(hipFree(dev_box));
  HIP_OK(hipStreamDestroy(s));
  free(host);
  if (fclose(out) != 0) return fail("closing the output", HG_EINVAL);
  fclose(in);
  return 0;
}
