// Calibration kernel (include/ra_probe.h): the rate that the bf16 matrix
// instruction of the attention kernels sustains from registers on a full chip.
// Each wave keeps 4 independent accumulators in flight so that no MFMA waits
// for the previous one's result; there is no memory traffic inside the loop.
#include "../../include/ra_probe.h"
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES) mfma_loop_kernel(int iters, float* sink) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // small values derived from the lane, so nothing folds and the sums stay finite
    a[i] = (__bf16)(0.125f * (float)((tid + i) & 7));
    b[i] = (__bf16)(0.0625f * (float)((3 * tid + i) & 7));
  }
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[(size_t)blockIdx.x * (64 * WAVES) + tid] = s;
}

}  // namespace
}  // namespace ra

extern "C" ra_status ra_probe_mfma(int32_t iters, int32_t workgroups, int32_t waves, float* sink, void* stream) {
  if (!sink) return RA_ERR_NULL;
  if (iters < 1 || iters > (1 << 24) || workgroups < 1 || workgroups > (1 << 20) || (waves != 4 && waves != 8))
    return RA_ERR_SHAPE;
  const hipStream_t st = (hipStream_t)stream;
  if (waves == 4)
    hipLaunchKernelGGL(ra::mfma_loop_kernel<4>, dim3(workgroups), dim3(256), 0, st, iters, sink);
  else
    hipLaunchKernelGGL(ra::mfma_loop_kernel<8>, dim3(workgroups), dim3(512), 0, st, iters, sink);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}
