// The unfused forward's own passes (MOE_F_UNFUSED): the in-house baseline that runs the layer as
// the conventional pipeline of separate kernels the pages contrast the fused design with (route,
// permute, expert GEMMs, activation, unpermute, combine, each boundary a trip through HBM:
// commentary "Cursor 开源 MoK：把 MoE 的通信和计算焊进一个内核…", sections 瓶颈的真正来源 and
// 两份成绩单).  The arithmetic is the fused forward's, so both produce the same bits; only where
// the intermediate rows live differs.  Every pass is an HBM stream: one workgroup per row,
// 16-byte vector accesses.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {

namespace {

// xp[r] = xq[token of permuted row r], codes and scale bytes.
__global__ __launch_bounds__(256) void k_permute_rows(SchedView s, const uint8_t* __restrict__ xq,
                                                      const uint8_t* __restrict__ xs, int d, uint8_t* __restrict__ xp,
                                                      uint8_t* __restrict__ xps) {
  const int r = blockIdx.x;
  const int tok = row_token(s, r);
  const v4i* src = (const v4i*)(xq + (size_t)tok * d);
  v4i* dst = (v4i*)(xp + (size_t)r * d);
  for (int c = threadIdx.x; c < d / 16; c += blockDim.x) dst[c] = src[c];
  const uint32_t* ss = (const uint32_t*)(xs + (size_t)tok * (d / 32));
  uint32_t* ds = (uint32_t*)(xps + (size_t)r * (d / 32));
  for (int c = threadIdx.x; c < d / 128; c += blockDim.x) ds[c] = ss[c];
}

// H = silu(G) U quantised along I in blocks of 32 columns (one block per half-wave): the
// fused gate/up epilogue's arithmetic on G and U read back from HBM.
__global__ __launch_bounds__(256) void k_swiglu_quant(const float* __restrict__ g, const float* __restrict__ u, int I,
                                                      uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  const int r = blockIdx.x;
  const int n = blockIdx.y * blockDim.x + threadIdx.x;
  // past I (whole 32-column blocks, I % 32 == 0) the lanes repeat the last column so that every
  // lane of a block takes part in its maximum; they store nothing
  const size_t o = (size_t)r * I + min(n, I - 1);
  uint32_t sc;
  const uint32_t code = quant_lane32(silu(g[o]) * u[o], &sc);
  if (n < I) {
    hq[o] = (uint8_t)code;
    if ((n & 31) == 0) hs[(size_t)r * (I / 32) + (n >> 5)] = (uint8_t)sc;
  }
}

// yslot[slot of permuted row r] = yrows[r].
__global__ __launch_bounds__(256) void k_unpermute_rows(SchedView s, const float* __restrict__ yrows, int d,
                                                        float* __restrict__ yslot) {
  const int r = blockIdx.x;
  const v4f* src = (const v4f*)(yrows + (size_t)r * d);
  v4f* dst = (v4f*)(yslot + row_slot(s, r) * d);
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) dst[c] = src[c];
}

}  // namespace

hipError_t launch_permute_rows(const SchedView& s, const uint8_t* xq, const uint8_t* xs, int d, int RS, uint8_t* xp,
                               uint8_t* xps, hipStream_t st) {
  if (RS == 0) return hipSuccess;
  hipLaunchKernelGGL(k_permute_rows, dim3(RS), dim3(256), 0, st, s, xq, xs, d, xp, xps);
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const float* g, const float* u, int RS, int I, uint8_t* hq, uint8_t* hs,
                               hipStream_t st) {
  if (RS == 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_quant, dim3(RS, (I + 255) / 256), dim3(256), 0, st, g, u, I, hq, hs);
  return hipGetLastError();
}

hipError_t launch_unpermute_rows(const SchedView& s, const float* yrows, int RS, int d, float* yslot,
                                 hipStream_t st) {
  if (RS == 0) return hipSuccess;
  hipLaunchKernelGGL(k_unpermute_rows, dim3(RS), dim3(256), 0, st, s, yrows, d, yslot);
  return hipGetLastError();
}

}  // namespace moe
