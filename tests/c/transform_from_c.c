/* Unpack, pack and E4M3 block quant of one group through the C ABI from C,
 * with device memory from the HIP runtime (hipMalloc / hipMemcpy) and no torch.
 * Usage: transform_from_c <dir>. Reads <dir>/plan.txt ("n V S R_mat", then n
 * lines "rows cols kind p0 p1 start"), gathered.f32 (R_mat*S fp32),
 * grads.f32 (every tensor's gradient, one after another) and prev.f32
 * (R_mat*S fp32). Writes unpacked.f32 (the tensors one after another),
 * packed.f32 (accumulating pack with sigma = fl32(1/V)), codes.u8 and
 * scales.f32. Prints "ok" or the failing call and rs_last_error(); outputs
 * start as 0xA5 garbage on the device. Used by tests/test_gpu_c_client.py. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rs.h"

static char dir_[4096];

static const char* path(const char* name) {
  static char buf[4200];
  snprintf(buf, sizeof buf, "%s/%s", dir_, name);
  return buf;
}

static int read_file(const char* name, void* dst, size_t bytes) {
  FILE* f = fopen(path(name), "rb");
  if (!f) return -1;
  const size_t got = fread(dst, 1, bytes, f);
  fclose(f);
  return got == bytes ? 0 : -1;
}

static int write_file(const char* name, const void* src, size_t bytes) {
  FILE* f = fopen(path(name), "wb");
  if (!f) return -1;
  const size_t put = fwrite(src, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : -1;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) {                                            \
      printf("hip %s: %s\n", #call, hipGetErrorString(e_));            \
      return 1;                                                        \
    }                                                                  \
  } while (0)

#define RS_OK_(call)                                                   \
  do {                                                                 \
    int st_ = (call);                                                  \
    if (st_ != RS_OK) {                                                \
      printf("rs %s: %d %s\n", #call, st_, rs_last_error());           \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static void* dev_garbage(size_t bytes) {
  void* p = NULL;
  if (hipMalloc(&p, bytes ? bytes : 16) != hipSuccess) return NULL;
  if (hipMemset(p, 0xA5, bytes ? bytes : 16) != hipSuccess) return NULL;
  return p;
}

int main(int argc, char** argv) {
  if (argc != 2 || strlen(argv[1]) >= sizeof dir_) return 2;
  strcpy(dir_, argv[1]);
  FILE* f = fopen(path("plan.txt"), "r");
  if (!f) return 2;
  long long n, V, S, R;
  if (fscanf(f, "%lld %lld %lld %lld", &n, &V, &S, &R) != 4 || n < 1) return 2;
  rs_tensor_spec* specs = calloc((size_t)n, sizeof *specs);
  int64_t* starts = calloc((size_t)n, sizeof *starts);
  size_t* numel = calloc((size_t)n, sizeof *numel);
  void** dst = calloc((size_t)n, sizeof *dst);
  const void** src = calloc((size_t)n, sizeof *src);
  if (!specs || !starts || !numel || !dst || !src) return 2;
  size_t total_elems = 0;
  for (long long i = 0; i < n; ++i) {
    long long r, c, k, p0, p1, s;
    if (fscanf(f, "%lld %lld %lld %lld %lld %lld", &r, &c, &k, &p0, &p1, &s) != 6) return 2;
    specs[i].rows = r;
    specs[i].cols = c;
    specs[i].kind = (int32_t)k;
    specs[i].reserved = 0;
    specs[i].p0 = p0;
    specs[i].p1 = p1;
    starts[i] = s;
    numel[i] = (size_t)(r * c);
    total_elems += numel[i];
  }
  fclose(f);
  const size_t flat = (size_t)(R * S);

  float* h_gathered = malloc(flat * 4);
  float* h_grads = malloc(total_elems * 4);
  float* h_prev = malloc(flat * 4);
  float* h_unpacked = malloc(total_elems * 4);
  float* h_packed = malloc(flat * 4);
  uint8_t* h_codes = malloc(flat);
  if (!h_gathered || !h_grads || !h_prev || !h_unpacked || !h_packed || !h_codes) return 2;
  if (read_file("gathered.f32", h_gathered, flat * 4) || read_file("grads.f32", h_grads, total_elems * 4) ||
      read_file("prev.f32", h_prev, flat * 4))
    return 2;

  HIP_OK(hipSetDevice(0));
  rs_plan* plan = NULL;
  RS_OK_(rs_plan_load(specs, n, V, S, starts, R, 0, &plan));
  int64_t nq = 0;
  RS_OK_(rs_plan_info(plan, NULL, &nq, NULL));

  void* d_gathered = dev_garbage(flat * 4);
  void* d_prev = dev_garbage(flat * 4);
  float* d_packed = dev_garbage(flat * 4);
  void* d_codes = dev_garbage(flat);
  float* d_scales = dev_garbage((size_t)nq * 4);
  if (!d_gathered || !d_prev || !d_packed || !d_codes || !d_scales) return 3;
  HIP_OK(hipMemcpy(d_gathered, h_gathered, flat * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_prev, h_prev, flat * 4, hipMemcpyHostToDevice));
  size_t off = 0;
  for (long long i = 0; i < n; ++i) {
    dst[i] = dev_garbage(numel[i] * 4);
    void* g = dev_garbage(numel[i] * 4);
    if (!dst[i] || !g) return 3;
    HIP_OK(hipMemcpy(g, h_grads + off, numel[i] * 4, hipMemcpyHostToDevice));
    src[i] = g;
    off += numel[i];
  }

  /* the null stream: every call is ordered on it */
  RS_OK_(rs_unpack_gathered(plan, d_gathered, RS_F32, dst, NULL));
  RS_OK_(rs_pack_scatter(plan, src, RS_F32, d_prev, d_packed, RS_F32, RS_SCALE_INV_V, 0.0f, NULL));
  RS_OK_(rs_block_quant(plan, d_gathered, RS_F32, d_codes, RS_E4M3, d_scales, NULL));
  HIP_OK(hipDeviceSynchronize());

  off = 0;
  for (long long i = 0; i < n; ++i) {
    HIP_OK(hipMemcpy(h_unpacked + off, dst[i], numel[i] * 4, hipMemcpyDeviceToHost));
    off += numel[i];
  }
  float* h_scales = malloc((size_t)nq * 4 + 4);
  if (!h_scales) return 2;
  HIP_OK(hipMemcpy(h_packed, d_packed, flat * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_codes, d_codes, flat, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_scales, d_scales, (size_t)nq * 4, hipMemcpyDeviceToHost));
  if (write_file("unpacked.f32", h_unpacked, total_elems * 4) || write_file("packed.f32", h_packed, flat * 4) ||
      write_file("codes.u8", h_codes, flat) || write_file("scales.f32", h_scales, (size_t)nq * 4))
    return 2;

  rs_plan_free(plan);
  for (long long i = 0; i < n; ++i) {
    HIP_OK(hipFree(dst[i]));
    HIP_OK(hipFree((void*)src[i]));
  }
  HIP_OK(hipFree(d_gathered));
  HIP_OK(hipFree(d_prev));
  HIP_OK(hipFree(d_packed));
  HIP_OK(hipFree(d_codes));
  HIP_OK(hipFree(d_scales));
  free(specs);
  free(starts);
  free(numel);
  free(dst);
  free(src);
  free(h_gathered);
  free(h_grads);
  free(h_prev);
  free(h_unpacked);
  free(h_packed);
  free(h_codes);
  free(h_scales);
  printf("ok\n");
  return 0;
}
