// Achievable-peak probes of the two units the hot path is bound by: the bf16
// matrix cores (the dense contraction of every kept block) and HBM (the
// gathered decode).  The benchmark times them beside the kernels so that each
// kernel's rate is reported against the spec peak and against what this
// chip, at its clock of the moment, actually sustains.
#include <hip/hip_runtime.h>

#include "common.h"
#include "sa_peaks.h"

namespace sa {
namespace {

constexpr int kPeakThreads = 256;

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave:
// one chain per 32-cycle MFMA slot keeps the matrix core busy without any
// memory traffic.  The result is written only under a condition that the
// data never meets, so the loop cannot be removed.
__global__ __launch_bounds__(kPeakThreads) void k_peak_mfma(float* sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(threadIdx.x + e));
    b[e] = (__bf16)(2e-3f * (float)e);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32x32x16(a, b, c0);
    c1 = mfma32x32x16(a, b, c1);
    c2 = mfma32x32x16(a, b, c2);
    c3 = mfma32x32x16(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 1234.5f) sink[threadIdx.x] = s;
}

// Streaming read: every thread reads 16-byte elements with four loads in
// flight, striding over the whole buffer, `reps` times.
__global__ __launch_bounds__(kPeakThreads) void k_peak_read(const u32x4* __restrict__ buf, int64_t n16, int reps,
                                                           u32x4* sink) {
  const int64_t nt = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int r = 0; r < reps; ++r) {
    int64_t i = t0;
    for (; i + 3 * nt < n16; i += 4 * nt) {
      const u32x4 x0 = buf[i], x1 = buf[i + nt], x2 = buf[i + 2 * nt], x3 = buf[i + 3 * nt];
      acc ^= x0 ^ x1 ^ x2 ^ x3;
    }
    for (; i < n16; i += nt) acc ^= buf[i];
  }
  if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[t0 & 255] = acc;
}

}  // namespace
}  // namespace sa

extern "C" {

int sa_peak_mfma_bf16(float* sink, int iters, int waves_per_cu, double* flop, void* stream) {
  if (!sink || !flop || iters <= 0 || waves_per_cu <= 0 || waves_per_cu % 4) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 7;
  const int blocks = cus * waves_per_cu / 4;  // 4 waves per workgroup
  hipLaunchKernelGGL(sa::k_peak_mfma, dim3(blocks), dim3(sa::kPeakThreads), 0, (hipStream_t)stream, sink, iters);
  *flop = (double)blocks * 4 * (double)iters * 4 * (32.0 * 32.0 * 16.0 * 2.0);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int sa_peak_read(const void* buf, size_t bytes, int reps, void* sink, double* bytes_read, void* stream) {
  if (!buf || !sink || !bytes_read || reps <= 0 || bytes < 16 || ((uintptr_t)buf & 15)) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 7;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(sa::k_peak_read, dim3(cus * 8), dim3(sa::kPeakThreads), 0, (hipStream_t)stream,
                     (const sa::u32x4*)buf, n16, reps, (sa::u32x4*)sink);
  *bytes_read = (double)n16 * 16.0 * reps;
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
