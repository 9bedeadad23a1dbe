/* A plain C client of libdust.so: no Python, no torch.  It reads a problem
 * from a binary file, runs dust_estimate on the default HIP stream with
 * buffers it allocates itself, and writes G_W back, so the tests can check
 * the C ABI end to end (sizing, validation, the estimate, error statuses).
 *
 *   abi_client <in.bin> <out.bin>
 *
 * in.bin:  int64 T, d_in, d_out, seq_len, dtype, K, antithetic; float sigma,
 *          gamma; uint64 seed; then X [T][d_in], W [d_out][d_in] and
 *          target [T][d_out] as raw elements of the dtype (bf16: 2 bytes).
 * out.bin: int32 status of the estimate, int32 status of an odd-K call with
 *          antithetic pairs, int32 status of a call with one byte too little
 *          workspace, then G_W [d_out][d_in] float.
 * Prints one line "ok <status>" and exits 0 when every call behaved as
 * documented; exits 1 otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dust.h"

static int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && bytes && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 1;
  int64_t hdr[7];
  float sg[2];
  uint64_t seed;
  if (fread(hdr, sizeof hdr, 1, in) != 1 || fread(sg, sizeof sg, 1, in) != 1 ||
      fread(&seed, sizeof seed, 1, in) != 1) {
    fclose(in);
    return 1;
  }
  const int64_t T = hdr[0], d_in = hdr[1], d_out = hdr[2], seq_len = hdr[3];
  const int32_t dtype = (int32_t)hdr[4], K = (int32_t)hdr[5], anti = (int32_t)hdr[6];
  const size_t es = dtype == DUST_BF16 ? 2 : 4;
  const size_t bx = (size_t)(T * d_in) * es, bw = (size_t)(d_out * d_in) * es,
               bt = (size_t)(T * d_out) * es, bg = (size_t)(d_out * d_in) * sizeof(float);
  void* hx = read_block(in, bx);
  void* hw = read_block(in, bw);
  void* ht = read_block(in, bt);
  fclose(in);
  float* hg = (float*)malloc(bg);
  if (!hx || !hw || !ht || !hg) return 1;

  const size_t ws_bytes = dust_workspace_bytes(T, d_in, d_out, K, anti, dtype);
  if (ws_bytes == 0) return 1;
  void *dx, *dw, *dt, *dg, *dws;
  if (check_hip(hipMalloc(&dx, bx), "hipMalloc") || check_hip(hipMalloc(&dw, bw), "hipMalloc") ||
      check_hip(hipMalloc(&dt, bt), "hipMalloc") || check_hip(hipMalloc(&dg, bg), "hipMalloc") ||
      check_hip(hipMalloc(&dws, ws_bytes), "hipMalloc"))
    return 1;
  if (check_hip(hipMemcpy(dx, hx, bx, hipMemcpyHostToDevice), "copy X") ||
      check_hip(hipMemcpy(dw, hw, bw, hipMemcpyHostToDevice), "copy W") ||
      check_hip(hipMemcpy(dt, ht, bt, hipMemcpyHostToDevice), "copy target"))
    return 1;

  const dust_status_t st = dust_estimate(dx, dw, dt, T, d_in, d_out, seq_len, dtype, K, sg[0],
                                         sg[1], seed, anti, (float*)dg, NULL, NULL, NULL, NULL,
                                         dws, ws_bytes, NULL);
  if (st != DUST_OK) fprintf(stderr, "dust_estimate: %s\n", dust_last_error());
  if (check_hip(hipDeviceSynchronize(), "synchronize") ||
      check_hip(hipMemcpy(hg, dg, bg, hipMemcpyDeviceToHost), "copy G_W"))
    return 1;
  /* documented failures: checked on the host, before any launch */
  const dust_status_t odd = dust_estimate(dx, dw, dt, T, d_in, d_out, seq_len, dtype, 3, sg[0],
                                          sg[1], seed, 1, (float*)dg, NULL, NULL, NULL, NULL, dws,
                                          ws_bytes, NULL);
  const int odd_msg = dust_last_error()[0] != '\0';
  const dust_status_t small = dust_estimate(dx, dw, dt, T, d_in, d_out, seq_len, dtype, K, sg[0],
                                            sg[1], seed, anti, (float*)dg, NULL, NULL, NULL, NULL,
                                            dws, ws_bytes - 1, NULL);

  FILE* out = fopen(argv[2], "wb");
  if (!out) return 1;
  const int32_t codes[3] = {(int32_t)st, (int32_t)odd, (int32_t)small};
  fwrite(codes, sizeof codes, 1, out);
  fwrite(hg, 1, bg, out);
  fclose(out);
  hipFree(dx);
  hipFree(dw);
  hipFree(dt);
  hipFree(dg);
  hipFree(dws);
  free(hx);
  free(hw);
  free(ht);
  free(hg);
  const int good = st == DUST_OK && odd == DUST_ERR_INVALID_ARG && odd_msg &&
                   small == DUST_ERR_WORKSPACE;
  printf("%s %d\n", good ? "ok" : "bad", (int)st);
  return good ? 0 : 1;
}
