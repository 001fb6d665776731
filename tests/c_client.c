/* A plain C caller of libnarrowcast: current per-tensor E4M3 scaling of one
 * fp32 vector through the C ABI alone (no Python), the sequence a training
 * step runs -- amax, scale update, cast.
 *
 *   c_client IN OUT_CODES OUT_COUNTS OUT_STATE
 *
 * IN holds n little-endian fp32 values.  Writes the n codes, the cast's
 * nc_counts and the tensor's nc_scale_state as raw bytes.  Exit status 0 on
 * success; a failing call prints its status string. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>
#include "narrowcast.h"

#define HIP_OK(e) do { hipError_t r_ = (e); if (r_ != hipSuccess) { \
  fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(r_)); return 2; } } while (0)
#define NC_OK_(e) do { nc_status r_ = (e); if (r_ != NC_OK) { \
  fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, nc_status_string(r_)); return 3; } } while (0)

static int write_file(const char *path, const void *p, size_t bytes) {
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); return 1; }
  fclose(f);
  return 0;
}

int main(int argc, char **argv) {
  if (argc != 5) { fprintf(stderr, "usage: c_client IN OUT_CODES OUT_COUNTS OUT_STATE\n"); return 1; }
  FILE *f = fopen(argv[1], "rb");
  if (!f) { fprintf(stderr, "cannot read %s\n", argv[1]); return 1; }
  fseek(f, 0, SEEK_END);
  const long bytes = ftell(f);
  fseek(f, 0, SEEK_SET);
  const int64_t n = bytes / 4;
  float *x = (float *)malloc((size_t)n * 4 + 4);
  uint8_t *codes = (uint8_t *)malloc((size_t)n + 1);
  if (!x || !codes || fread(x, 4, (size_t)n, f) != (size_t)n) { fprintf(stderr, "short read\n"); return 1; }
  fclose(f);

  void *dx, *dcodes, *ws;
  nc_counts *dam, *dout, out;
  nc_scale_state *dst, st;
  HIP_OK(hipMalloc(&dx, (size_t)n * 4 + 16));
  HIP_OK(hipMalloc(&dcodes, (size_t)n + 16));
  HIP_OK(hipMalloc((void **)&dam, sizeof(nc_counts)));
  HIP_OK(hipMalloc((void **)&dout, sizeof(nc_counts)));
  HIP_OK(hipMalloc((void **)&dst, sizeof(nc_scale_state)));
  HIP_OK(hipMemcpy(dx, x, (size_t)n * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(dam, 0, sizeof(nc_counts)));
  HIP_OK(hipMemset(dout, 0, sizeof(nc_counts)));
  HIP_OK(hipMemset(dst, 0, sizeof(nc_scale_state)));   /* all-zero: a fresh state */

  nc_tensor t;
  memset(&t, 0, sizeof(t));
  t.x = dx;
  t.codes = (uint8_t *)dcodes;
  t.n = n;
  const size_t ws_bytes = nc_workspace_bytes(&t, 1);
  HIP_OK(hipMalloc(&ws, ws_bytes > 16 ? ws_bytes : 16));

  nc_policy pol;
  memset(&pol, 0, sizeof(pol));
  pol.fmt = NC_E4M3;
  pol.est = NC_EST_CURRENT;
  pol.window = 1;
  pol.interval = 1;
  pol.ls_growth_interval = 1;
  pol.ema_alpha = 0.0625f;

  NC_OK_(nc_amax(&t, 1, NC_F32, NULL, dam, ws, ws_bytes, NULL));
  NC_OK_(nc_scale_update(&pol, 1, dst, NULL, dam, NULL, NULL));
  NC_OK_(nc_cast_tensor(&t, 1, NC_F32, NC_E4M3, dst, NULL, dout, NULL, ws, ws_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(codes, dcodes, (size_t)n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&out, dout, sizeof(out), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&st, dst, sizeof(st), hipMemcpyDeviceToHost));
  if (write_file(argv[2], codes, (size_t)n) || write_file(argv[3], &out, sizeof(out)) ||
      write_file(argv[4], &st, sizeof(st)))
    return 1;
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dcodes));
  HIP_OK(hipFree(dam));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dst));
  HIP_OK(hipFree(ws));
  free(x);
  free(codes);
  printf("c_client: %lld elements, k = %d, clips %llu\n", (long long)n, st.k, (unsigned long long)out.n_clip);
  return 0;
}
