/* A plain C caller of the library: no Python, no torch.  It allocates the
 * buffers with the HIP runtime, moves 3 MiB + 5 bytes through a SIMPLE
 * connection (4 channels x 8 slots x 64 KiB in HBM) twice on one stream,
 * and checks the destination, the counters and an error path; then it
 * moves the same bytes with the entry point that allocates nothing, as LL,
 * and checks the destination and the reported status.  Exit code 0 means
 * every check passed; the first failing check prints its reason. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "xfer.h"

#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      fprintf(stderr, "FAIL: ");         \
      fprintf(stderr, __VA_ARGS__);      \
      fprintf(stderr, "\n");             \
      return 1;                          \
    }                                    \
  } while (0)

int main(void) {
  const size_t n = (3u << 20) + 5;
  const int nch = 4, nslots = 8;
  const size_t slot = 64u << 10;
  uint8_t* host = (uint8_t*)malloc(n);
  uint8_t* back = (uint8_t*)malloc(n);
  CHECK(host && back, "host allocation");
  uint64_t x = 0x9E3779B97F4A7C15ull;
  for (size_t i = 0; i < n; ++i) {  /* xorshift bytes */
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    host[i] = (uint8_t)x;
  }
  void *src = NULL, *dst = NULL;
  CHECK(hipMalloc(&src, n) == hipSuccess && hipMalloc(&dst, n) == hipSuccess, "hipMalloc");
  CHECK(hipMemcpy(src, host, n, hipMemcpyHostToDevice) == hipSuccess, "upload");
  CHECK(hipMemset(dst, 0, n) == hipSuccess, "clear");
  hipStream_t stream;
  CHECK(hipStreamCreate(&stream) == hipSuccess, "stream");

  xfer_conn* c = NULL;
  xfer_attr attr;
  memset(&attr, 0, sizeof(attr));
  attr.wgs_per_channel = 2;
  attr.block_threads = 256;
  int rc = xfer_conn_create_ex(XFER_PROTO_SIMPLE, nch, nslots, slot, XFER_FIFO_DEVICE, &attr, &c);
  CHECK(rc == XFER_OK, "create: %s (%s)", xfer_status_string(rc), xfer_last_error());
  for (int r = 0; r < 2; ++r) {
    rc = xfer_run(c, src, dst, n, (void*)stream);
    CHECK(rc == XFER_OK, "run: %s (%s)", xfer_status_string(rc), xfer_last_error());
  }
  CHECK(hipStreamSynchronize(stream) == hipSuccess, "sync");
  CHECK(hipMemcpy(back, dst, n, hipMemcpyDeviceToHost) == hipSuccess, "download");
  CHECK(memcmp(host, back, n) == 0, "destination differs from source");

  /* each channel moved ceil(n/nch) rounded up to 16 bytes (the last one the
     rest), in 64 KiB steps, twice */
  const uint64_t per = ((n + nch - 1) / nch + 15) & ~(uint64_t)15;
  for (int ch = 0; ch < nch; ++ch) {
    xfer_chan_state st;
    rc = xfer_conn_query(c, ch, &st);
    CHECK(rc == XFER_OK, "query: %s", xfer_last_error());
    uint64_t beg = per * (uint64_t)ch, len = 0;
    if (beg < n) len = (beg + per < n ? beg + per : n) - beg;
    const uint64_t steps = 2 * ((len + slot - 1) / slot);
    CHECK(st.error == XFER_OK && st.lanes_agree, "channel %d state", ch);
    CHECK(st.head == steps && st.tail == steps && st.steps == steps,
          "channel %d: head %llu tail %llu steps %llu, expected %llu", ch,
          (unsigned long long)st.head, (unsigned long long)st.tail,
          (unsigned long long)st.steps, (unsigned long long)steps);
  }
  /* overlapping buffers are refused with a message, before any launch */
  rc = xfer_run(c, src, (uint8_t*)src + 1, 64, (void*)stream);
  CHECK(rc == XFER_ERR_INVALID_ARG && strlen(xfer_last_error()) > 0, "overlap not refused");

  CHECK(xfer_conn_destroy(c) == XFER_OK, "destroy");

  /* no connection, nothing allocated by the library: LL through its fixed
     array, the failure code written to a device word after the transfer */
  uint32_t* status = NULL;
  uint32_t status_host = 0x7777;
  CHECK(hipMalloc((void**)&status, sizeof(*status)) == hipSuccess, "hipMalloc(status)");
  CHECK(hipMemset(dst, 0, n) == hipSuccess, "clear");
  memset(&attr, 0, sizeof(attr));
  attr.wgs_per_channel = 4;
  attr.block_threads = 512;
  rc = xfer_run_noalloc(XFER_PROTO_LL, nch, nslots, 32u << 10, &attr, src, dst, n, status,
                        (void*)stream);
  CHECK(rc == XFER_OK, "noalloc: %s (%s)", xfer_status_string(rc), xfer_last_error());
  CHECK(hipStreamSynchronize(stream) == hipSuccess, "sync");
  CHECK(hipMemcpy(back, dst, n, hipMemcpyDeviceToHost) == hipSuccess, "download");
  CHECK(hipMemcpy(&status_host, status, sizeof(status_host), hipMemcpyDeviceToHost) == hipSuccess,
        "status download");
  CHECK(status_host == 0, "noalloc status %u", status_host);
  CHECK(memcmp(host, back, n) == 0, "noalloc destination differs from source");
  (void)hipFree(status);
  (void)hipStreamDestroy(stream);
  (void)hipFree(src);
  (void)hipFree(dst);
  free(host);
  free(back);
  printf("abi_example: ok\n");
  return 0;
}
