// Measurement helper: the sustained rate of the bf16 matrix instruction the
// attention kernels are built on (v_mfma_f32_32x32x16_bf16), fed with the
// caller's operand values, and the shader clock while it runs.
//
// The datasheet peak assumes the top clock; under a full matrix load the chip
// lowers its clock by an amount that depends on the data (power), so the rate
// with realistic operand values is the ceiling a real kernel can reach.  Each
// wave keeps four independent accumulators busy (the instruction's latency is
// covered by the other three) and cycles through two A and two B fragments.
// Wave 0 of every workgroup reads the shader cycle counter and the constant-
// rate wall counter at its start and end, so ticks / wall ticks x wall rate
// is the average shader clock over the workgroup's lifetime.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mf.h"
#include "mf_device.h"

namespace mf {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeVectors = 4096;  // bf16x8 operand vectors the caller supplies (64 KiB)

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(const bf16x8* __restrict__ src,
                                                                   float* __restrict__ sink,
                                                                   unsigned long long* __restrict__ clocks,
                                                                   int iters) {
  const int t = blockIdx.x * kProbeThreads + threadIdx.x;
  const bf16x8 a0 = src[t % kProbeVectors];
  const bf16x8 a1 = src[(t + 1) % kProbeVectors];
  const bf16x8 b0 = src[(t + 2) % kProbeVectors];
  const bf16x8 b1 = src[(t + 3) % kProbeVectors];
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long m0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a0, b0, c0);
    c1 = mfma32(a1, b0, c1);
    c2 = mfma32(a0, b1, c2);
    c3 = mfma32(a1, b1, c3);
  }
  const unsigned long long m1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[t] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = m1 - m0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

}  // namespace mf

extern "C" mf_status mf_mfma_probe(const void* operands, int32_t n_blocks, int32_t iters, float* sink,
                                   uint64_t* clocks, int32_t* wall_clock_khz, void* stream) {
  if (operands == nullptr || sink == nullptr || clocks == nullptr || n_blocks <= 0 || iters <= 0 ||
      n_blocks > (1 << 20) || (reinterpret_cast<uintptr_t>(operands) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(clocks) & 7) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return MF_ERR_INVALID_ARG;
  if (wall_clock_khz != nullptr) {
    int dev = 0;
    int khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return MF_ERR_HIP;
    *wall_clock_khz = khz;
  }
  hipLaunchKernelGGL(mf::mfma_probe_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(mf::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const mf::bf16x8*>(operands), sink,
                     reinterpret_cast<unsigned long long*>(clocks), iters);
  return hipGetLastError() == hipSuccess ? MF_OK : MF_ERR_HIP;
}
