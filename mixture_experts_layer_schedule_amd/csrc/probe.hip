// Measurement only: the scaled MXFP8 matrix-core issue rate of the device, against which the
// layer's GEMM phases are reported next to the published dense peak.  Every wave multiplies
// register operands back to back (four independent accumulators, no memory traffic in the loop)
// and stores one float per lane at the end so the work is kept.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeAcc = 4;

__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(float* sink, int iters) {
  v16f acc[kProbeAcc];
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) acc[j] = (v16f){};
  const int l = lane_id();
  // arbitrary codes (any e4m3 pattern is a valid operand); scale byte 127 is 2^0
  const v8i a = (v8i){l, l + 1, l + 2, l + 3, l + 4, l + 5, l + 6, l + 7};
  const v8i b = (v8i){3 * l, 5, 7, l, 9, 11, 13, l + 17};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) s += acc[j][0] + acc[j][15];
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

int probe_mfma_blocks(int cus) { return 2 * cus; }  // four waves per SIMD
size_t probe_mfma_sink_bytes(int cus) { return sizeof(float) * (size_t)probe_mfma_blocks(cus) * kProbeThreads; }

hipError_t launch_probe_mfma(float* sink, int cus, int iters, double* flop, hipStream_t st) {
  const int blocks = probe_mfma_blocks(cus);
  *flop = 2.0 * 32 * 32 * 64 * kProbeAcc * (double)iters * (kProbeThreads / 64) * blocks;
  hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(kProbeThreads), 0, st, sink, iters);
  return hipGetLastError();
}

}  // namespace moe
