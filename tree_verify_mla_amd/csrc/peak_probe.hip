// Roofline probes: a loop of nothing but bf16 matrix-core instructions, and
// the device's compute-unit count and peak clock.  They let a measurement be
// stated beside the published peaks it is divided by (what the matrix cores
// sustain on this device under load, at the clock it actually runs).
#include "common.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int CHAINS = 8;  // independent accumulators per wave: the pipe never waits on a result

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16_t acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;  // the sums keep the loop alive
}

}  // namespace

extern "C" int ddtree_probe_mfma_loop(int grid, int iters, float* out, void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(grid >= 1 && iters >= 1 && out, DDTREE_EINVAL,
                 "probe_mfma_loop: need grid >= 1, iters >= 1 and an output buffer");
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0, ddtree::as_stream(stream), iters,
                     out);
  return ddtree::check_launch("probe_mfma_loop");
}

extern "C" int ddtree_device_info(int* compute_units, int* peak_clock_khz) {
  ddtree::clear_error();
  DDTREE_REQUIRE(compute_units && peak_clock_khz, DDTREE_EINVAL, "device_info: null pointer");
  int dev = 0;
  DDTREE_REQUIRE(hipGetDevice(&dev) == hipSuccess, DDTREE_EHIP, "device_info: no current device");
  DDTREE_REQUIRE(hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, dev) ==
                         hipSuccess &&
                     hipDeviceGetAttribute(peak_clock_khz, hipDeviceAttributeClockRate, dev) ==
                         hipSuccess,
                 DDTREE_EHIP, "device_info: attribute query failed");
  return DDTREE_OK;
}
