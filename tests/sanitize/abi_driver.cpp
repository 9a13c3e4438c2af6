// Calls every C-ABI entry point of include/ssm66.h on arguments the library
// must refuse -- NULL and misaligned pointers, negative, zero, huge and
// overflowing sizes, unknown flags and kernels -- and the host-only queries
// on shapes up to the int64 limits, so that an AddressSanitizer /
// UndefinedBehaviorSanitizer build of the library's host code reports any
// out-of-bounds access or undefined arithmetic (signed overflow, shifts) in
// the validation layer.  Every call here returns before any HIP call (the
// status is checked), so the driver needs no GPU.  Compiled and run by
// tests/test_sanitizers.py; exits 0 when every status is as expected and the
// sanitizers stay silent.
#include <stdint.h>
#include <stdio.h>

#include "../../include/ssm66.h"

static int failures = 0;
static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d, %s: status %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

int main() {
  void* P = (void*)0x10000;   // aligned, never dereferenced
  void* M = (void*)0x10001;   // misaligned for every element type
  float* F = (float*)P;
  const int64_t big = INT64_MAX, huge = (int64_t)1 << 40;
  const int64_t shapes[][4] = {{1, 1, 1, 1},     {0, 5, 8, 16},          {2, 0, 8, 16},
                               {2, 5, 0, 16},    {-1, 5, 8, 16},         {2, -5, 8, 16},
                               {2, 5, -8, 16},   {2, 5, 8, 0},           {2, 5, 8, 17},
                               {big, 2, 2, 16},  {2, big, 2, 16},        {2, 2, big, 16},
                               {1, 1, big / 4, 1}, {1, 1, huge, 1},      {huge, huge, 1, 1},
                               {1, 2, (int64_t)1 << 55, 1}, {(int64_t)1 << 31, 2, 1 << 12, 16}};
  // host-only queries over every shape: no status, only defined arithmetic
  for (const auto& s : shapes) {
    (void)ssm_scan_kernel_name(s[0], s[1], s[2], s[3]);
    (void)ssm_scan_ckpt_size(s[0], s[1], s[2], s[3]);
    (void)ssm_scan_bwd_workspace_size(s[0], s[1], s[2], s[3]);
  }
  for (int k = -3; k < 300; k += 7) (void)ssm_status_string(k);
  (void)ssm_abi_version();

  // the scan: each argument refused in turn
  auto scan = [&](const void* u, const float* A, void* y, int64_t b, int64_t L, int64_t d,
                  int64_t n, int io, int sp, int dm) {
    return ssm_scan_fwd(u, u, A, u, u, nullptr, nullptr, nullptr, sp, dm, y, nullptr, b, L, d,
                        n, io, nullptr);
  };
  EXPECT(scan(P, F, P, 2, 5, 8, 17, SSM_BF16, 1, 0), SSM_ERR_SHAPE);
  EXPECT(scan(P, F, P, -2, 5, 8, 16, SSM_BF16, 1, 0), SSM_ERR_SHAPE);
  EXPECT(scan(P, F, P, big, big, 8, 16, SSM_BF16, 1, 0), SSM_ERR_SHAPE);
  EXPECT(scan(P, F, P, 1, 1, big, 16, SSM_BF16, 1, 0), SSM_ERR_SHAPE);
  EXPECT(scan(P, F, P, 2, 5, 8, 16, 7, 1, 0), SSM_ERR_DTYPE);
  EXPECT(scan(P, F, P, 2, 5, 8, 16, SSM_BF16, 2, 0), SSM_ERR_FLAG);
  EXPECT(scan(P, F, P, 2, 5, 8, 16, SSM_BF16, 1, 5), SSM_ERR_FLAG);
  EXPECT(scan(nullptr, F, P, 2, 5, 8, 16, SSM_BF16, 1, 0), SSM_ERR_NULL);
  EXPECT(scan(P, nullptr, P, 2, 5, 8, 16, SSM_BF16, 1, 0), SSM_ERR_NULL);
  EXPECT(scan(P, F, nullptr, 2, 5, 8, 16, SSM_BF16, 1, 0), SSM_ERR_NULL);
  EXPECT(scan(M, F, P, 2, 5, 8, 16, SSM_BF16, 1, 0), SSM_ERR_ALIGN);
  EXPECT(scan(P, (float*)M, P, 2, 5, 8, 16, SSM_BF16, 1, 0), SSM_ERR_ALIGN);
  EXPECT(scan(P, F, P, 0, 5, 8, 16, SSM_BF16, 1, 0), SSM_OK);
  EXPECT(scan(P, F, P, 2, 5, 0, 16, SSM_BF16, 1, 0), SSM_OK);
  // layers too wide for the kernels' 32-bit offsets, grids past the launch limit
  EXPECT(scan(P, F, P, 1, 1, (int64_t)1 << 55, 1, SSM_BF16, 1, 0), SSM_ERR_UNSUPPORTED);
  EXPECT(scan(P, F, P, 1, 2, (int64_t)1 << 40, 1, SSM_F32, 1, 0), SSM_ERR_UNSUPPORTED);
  EXPECT(scan(P, F, P, (int64_t)1 << 36, 1, 1 << 10, 16, SSM_BF16, 1, 0), SSM_ERR_UNSUPPORTED);
  // forced kernels
  for (int k : {-1, SSM_SCAN_KERNEL_WAVE4 + 1, 1000})
    EXPECT(ssm_scan_fwd_kernel(k, P, P, F, P, P, nullptr, nullptr, nullptr, 1, 0, nullptr,
                               nullptr, nullptr, P, nullptr, nullptr, 2, 5, 8, 16, SSM_BF16,
                               nullptr),
           SSM_ERR_FLAG);
  for (int k = SSM_SCAN_KERNEL_AUTO; k <= SSM_SCAN_KERNEL_WAVE4; ++k)
    EXPECT(ssm_scan_fwd_kernel(k, P, P, F, P, P, nullptr, nullptr, nullptr, 1, 0, nullptr,
                               nullptr, nullptr, P, nullptr, nullptr, 1, 2, (int64_t)1 << 50, 1,
                               SSM_BF16, nullptr),
           SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_scan_fwd_ex(P, P, F, P, P, nullptr, nullptr, nullptr, 1, 0, F, (const int32_t*)M,
                         nullptr, P, F, 2, 5, 8, 16, SSM_BF16, nullptr),
         SSM_ERR_ALIGN);
  EXPECT(ssm_scan_fwd_ckpt(P, P, F, P, P, nullptr, nullptr, nullptr, 1, 0, nullptr, P, nullptr,
                           nullptr, 2, 5, 8, 16, SSM_BF16, nullptr),
         SSM_ERR_NULL);

  // the decode step
  auto step = [&](float* st, const void* u, int64_t b, int64_t d, int64_t n, int io) {
    return ssm_step(st, u, u, F, u, u, nullptr, nullptr, nullptr, 1, 0, P, b, d, n, io, nullptr);
  };
  EXPECT(step(F, P, 2, 8, 0, SSM_F32), SSM_ERR_SHAPE);
  EXPECT(step(F, P, big, big, 16, SSM_F32), SSM_ERR_SHAPE);
  EXPECT(step(nullptr, P, 2, 8, 16, SSM_F32), SSM_ERR_NULL);
  EXPECT(step((float*)M, P, 2, 8, 16, SSM_F32), SSM_ERR_ALIGN);
  EXPECT(step(F, M, 2, 8, 16, SSM_BF16), SSM_ERR_ALIGN);
  EXPECT(step(F, P, (int64_t)1 << 40, (int64_t)1 << 20, 1, SSM_F32), SSM_ERR_UNSUPPORTED);
  EXPECT(step(F, P, 0, 8, 16, SSM_F32), SSM_OK);

  // the backward pass, with a workspace and on the static scratch
  auto bwd = [&](void* ws, size_t wsb, int64_t b, int64_t L, int64_t d, int64_t n) {
    return ssm_scan_bwd(P, P, F, P, P, nullptr, nullptr, nullptr, 1, 0, nullptr, P, nullptr, P,
                        P, F, P, P, nullptr, nullptr, nullptr, nullptr, ws, wsb, b, L, d, n,
                        SSM_BF16, nullptr);
  };
  EXPECT(bwd(nullptr, 0, 2, 5, 8, 16), SSM_ERR_NULL);
  EXPECT(bwd(P, 1, 2, 5, 8, 16), SSM_ERR_SHAPE);
  EXPECT(bwd(M, (size_t)1 << 40, 2, 5, 8, 16), SSM_ERR_ALIGN);
  EXPECT(bwd(P, (size_t)1 << 40, big, 5, 8, 16), SSM_ERR_SHAPE);
  EXPECT(ssm_scan_bwd_noalloc(P, P, F, P, P, nullptr, nullptr, nullptr, 1, 0, nullptr, nullptr,
                              nullptr, P, nullptr, P, P, F, P, P, nullptr, nullptr, nullptr,
                              nullptr, nullptr, 8, 2048, 1536, 16, SSM_BF16, nullptr),
         SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_scan_bwd_noalloc(P, P, F, P, P, nullptr, P, nullptr, 1, 0, nullptr, nullptr,
                              nullptr, P, nullptr, P, P, F, P, P, nullptr, nullptr, nullptr,
                              nullptr, nullptr, 1, 64, 64, 16, SSM_BF16, nullptr),
         SSM_ERR_NULL);  // a gate without its gradient
  {  // lengths and resets: seq_lens must be 4-byte aligned
    const int32_t* lens_m = (const int32_t*)((const char*)F + 2);
    EXPECT(ssm_scan_bwd_ex(P, P, F, P, P, nullptr, nullptr, nullptr, 1, 0, nullptr, lens_m,
                           nullptr, P, nullptr, P, P, F, P, P, nullptr, nullptr, nullptr,
                           nullptr, nullptr, P, (size_t)1 << 40, 2, 5, 8, 16, SSM_BF16, nullptr),
           SSM_ERR_ALIGN);
  }

  // Mamba-2 / SSD
  auto ssd = [&](const void* x, int64_t b, int64_t L, int64_t h, int64_t pd, int64_t n, int io) {
    return ssm_ssd_fwd(x, F, F, P, P, nullptr, nullptr, nullptr, 1, 1, nullptr, P, nullptr, b, L,
                       h, pd, n, io, nullptr);
  };
  EXPECT(ssd(P, 2, 8, 4, 64, 128, 3), SSM_ERR_DTYPE);
  EXPECT(ssd(P, -2, 8, 4, 64, 128, SSM_BF16), SSM_ERR_SHAPE);
  EXPECT(ssd(P, 2, 8, big, 64, 128, SSM_BF16), SSM_ERR_SHAPE);
  EXPECT(ssd(P, 2, 8, big / 32, 64, 128, SSM_BF16), SSM_ERR_SHAPE);
  EXPECT(ssd(P, 2, 8, 4, 24, 128, SSM_BF16), SSM_ERR_UNSUPPORTED);
  EXPECT(ssd(M, 2, 8, 4, 64, 128, SSM_BF16), SSM_ERR_ALIGN);
  EXPECT(ssd(P, (int64_t)1 << 30, 1, 1 << 10, 64, 64, SSM_BF16), SSM_ERR_UNSUPPORTED);

  // the convolution
  auto conv = [&](const void* x, int64_t b, int64_t L, int64_t d, int64_t w, int io) {
    return ssm_conv1d_fwd(x, F, nullptr, 1, nullptr, nullptr, nullptr, P, nullptr, b, L, d, w,
                          io, nullptr);
  };
  EXPECT(conv(P, 2, 8, 16, 5, SSM_BF16), SSM_ERR_SHAPE);
  EXPECT(conv(P, 2, 8, 16, 0, SSM_BF16), SSM_ERR_SHAPE);
  EXPECT(conv(P, big, big, 16, 4, SSM_BF16), SSM_ERR_SHAPE);
  EXPECT(conv(M, 2, 8, 16, 4, SSM_BF16), SSM_ERR_ALIGN);
  EXPECT(conv(P, 2, (int64_t)1 << 30, 16, 4, SSM_BF16), SSM_ERR_UNSUPPORTED);
  EXPECT(ssm_conv1d_step(nullptr, P, F, nullptr, 1, P, 2, 16, 4, SSM_BF16, nullptr),
         SSM_ERR_NULL);
  EXPECT(ssm_conv1d_step(P, P, F, nullptr, 1, P, big, big, 4, SSM_BF16, nullptr), SSM_ERR_SHAPE);
  EXPECT(ssm_conv1d_step(P, P, F, nullptr, 1, P, (int64_t)1 << 40, (int64_t)1 << 20, 1, SSM_F32,
                         nullptr),
         SSM_ERR_UNSUPPORTED);

  // the issue-rate probe
  EXPECT(ssm_alu_probe(3, F, 1, 1, nullptr), SSM_ERR_FLAG);
  EXPECT(ssm_alu_probe(0, F, 0, 1, nullptr), SSM_ERR_SHAPE);
  EXPECT(ssm_alu_probe(0, F, 1, -1, nullptr), SSM_ERR_SHAPE);
  EXPECT(ssm_alu_probe(0, nullptr, 1, 1, nullptr), SSM_ERR_NULL);
  EXPECT(ssm_alu_probe(0, (float*)M, 1, 1, nullptr), SSM_ERR_ALIGN);

  if (failures) {
    fprintf(stderr, "abi driver: %d unexpected statuses\n", failures);
    return 1;
  }
  printf("abi driver: done\n");
  return 0;
}
