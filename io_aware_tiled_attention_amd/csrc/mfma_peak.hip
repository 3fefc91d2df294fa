// mfma_peak.hip -- measurement kernel (not part of the attention path): the
// rate at which this GPU's matrix cores run v_mfma_f32_32x32x16_bf16 with
// every operand in registers, no memory traffic and no other work.  It is
// the attainable ceiling against which the attention kernels' matrix-core
// rates are read, next to the published 2.5 PFLOP/s (2.4 GHz x 256 CUs x
// 4096 FLOP/clock), since the clock under sustained matrix-core load sits
// below 2.4 GHz.
//
// Each lane loads 4 A and 4 B operand fragments (8 bf16 each) of caller
// data, e.g. N(0,1) draws, once; every iteration then issues 16 products
// that pair each A with each B into 4 fp32 accumulators, so consecutive
// products see different operand bits (the matrix cores' power, and with it
// the clock, depends on how much the operand bits toggle).  One workgroup is
// 4 waves, one per SIMD; `workgroups` = 256 x w gives w waves per SIMD.
#include <hip/hip_runtime.h>

#include "fa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void mfma_peak_bf16_kernel(const bf16x8* __restrict__ ops,
                                                                  float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(4 + i) * 64 + lane];
  }
  f32x16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + j) & 3], c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int fa_probe_mfma_bf16(const void* operands, float* sink, int workgroups, int iters, void* stream) {
  if (!operands || !sink) return 1;
  if (workgroups <= 0 || workgroups > (1 << 20) || iters <= 0) return 2;
  hipLaunchKernelGGL(mfma_peak_bf16_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const bf16x8*>(operands), sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

extern "C" double fa_probe_mfma_bf16_flops(int workgroups, int iters) {
  return (double)workgroups * (kThreads / 64) * (double)iters * 16.0 * (32.0 * 32.0 * 16.0 * 2.0);
}
