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

// H = silu(G) U quantised along I in blocks of 32 columns: the fused gate/up epilogue's
// arithmetic on G and U read back from HBM.  Each lane takes 4 consecutive columns (16-byte loads
// of G and U, one 4-byte store of their codes), so a block is 8 lanes and its maximum a 3-step
// exchange among them; every value goes through the same scaling and conversion as in the
// epilogue, so the codes are the same bits.
__global__ __launch_bounds__(256) void k_swiglu_quant(const float* __restrict__ g, const float* __restrict__ u, int I,
                                                      uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  const int r = blockIdx.x;
  const int n = blockIdx.y * blockDim.x + threadIdx.x;  // 4-column group of the row
  const int n4 = I / 4;
  // past I (whole 8-lane blocks, I % 32 == 0) the lanes repeat the last group: they store nothing
  const size_t o = (size_t)r * I + 4 * (size_t)min(n, n4 - 1);
  const v4f gv = *(const v4f*)(g + o), uv = *(const v4f*)(u + o);
  // the block maximum on the bit patterns of |h|, as the epilogue takes it (a NaN wins there too)
  float h[4];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = silu(gv[j]) * uv[j];
    m = max(m, __float_as_uint(fabsf(h[j])));
  }
#pragma unroll
  for (int x = 1; x < 8; x <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, x));
  const uint32_t byte = e8m0_from_amax(__uint_as_float(m));
  const float inv = e8m0_inv_scale(byte);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(h[0] * inv), clamp448(h[1] * inv), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(h[2] * inv), clamp448(h[3] * inv), w, true);
  if (n < n4) {
    *(uint32_t*)(hq + o) = (uint32_t)w;
    if ((n & 7) == 0) hs[(size_t)r * (I / 32) + (n >> 3)] = (uint8_t)byte;
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
  hipLaunchKernelGGL(k_swiglu_quant, dim3(RS, (I / 4 + 255) / 256), dim3(256), 0, st, g, u, I, hq, hs);
  return hipGetLastError();
}

hipError_t launch_unpermute_rows(const SchedView& s, const float* yrows, int RS, int d, float* yslot,
                                 hipStream_t st) {
  if (RS == 0) return hipSuccess;
  hipLaunchKernelGGL(k_unpermute_rows, dim3(RS), dim3(256), 0, st, s, yrows, d, yslot);
  return hipGetLastError();
}

}  // namespace moe
