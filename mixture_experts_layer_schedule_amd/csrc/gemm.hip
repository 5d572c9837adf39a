// Grouped MXFP8 GEMMs of the expert FFN (forward, dgrad and wgrad) on gfx950; the tile core is
// in gemm_core.h.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// Forward gate/up: [G U] = X_e W1_e^T (pull dispatch: rows gathered from xq through the
// schedule), epilogue h = silu(G) U quantised along I.  Tile columns: 64 gate + the matching
// 64 up columns, so each lane holds G and U of the same element.

__global__ __launch_bounds__(256) void k_gemm_gateup(GateUpArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int tile = blockIdx.y;
  if (tile >= s.tile_start[s.n_exp]) return;
  const int e = tile_expert(s.tile_start, s.n_exp, tile);
  const int m0 = s.offsets[e] + (tile - s.tile_start[e]) * BM;
  const int mend = s.offsets[e + 1];
  const int nt = blockIdx.x;  // 64 columns of I
  const int I = p.I, d = p.d;
  const uint8_t* w1 = p.w1q + (size_t)e * 2 * I * d;
  const uint8_t* w1s = p.w1s + (size_t)e * 2 * I * (d / 32);

  const uint8_t* arow[4];
  const uint8_t* brow[4];
  for (int q = 0; q < 4; ++q) {
    int row = (threadIdx.x >> 3) + 32 * q;
    int r = min(m0 + row, mend - 1);
    arow[q] = p.xq + (size_t)row_token(s, r) * d;
    int brow_i = row < 64 ? nt * 64 + row : I + nt * 64 + (row - 64);
    brow[q] = w1 + (size_t)brow_i * d;
  }
  const uint8_t* srow;
  if (threadIdx.x < BM) {
    int r = min(m0 + (int)threadIdx.x, mend - 1);
    srow = p.xs + (size_t)row_token(s, r) * (d / 32);
  } else {
    int row = threadIdx.x - BM;
    int brow_i = row < 64 ? nt * 64 + row : I + nt * 64 + (row - 64);
    srow = w1s + (size_t)brow_i * (d / 32);
  }
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int b_row0[2] = {wn * 32, 64 + wn * 32};
  v16f acc[2][2];
  mainloop(lds, arow, brow, srow, d, wm * 64, b_row0, acc);

  gateup_epilogue(acc, m0, mend, nt, wm, wn, I, p.g, p.u, p.hq, p.hs);
}

// ---------------------------------------------------------------------------------------------
// Forward down: Y_r = H_r W2_e^T, pushed to its slot Yslot[t, j] (push combine).

__global__ __launch_bounds__(256) void k_gemm_down(DownArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int tile = blockIdx.y;
  if (tile >= s.tile_start[s.n_exp]) return;
  const int e = tile_expert(s.tile_start, s.n_exp, tile);
  const int m0 = s.offsets[e] + (tile - s.tile_start[e]) * BM;
  const int mend = s.offsets[e + 1];
  const int nt = blockIdx.x;  // 128 columns of d
  const int I = p.I, d = p.d;
  const uint8_t* w2 = p.w2q + (size_t)e * d * I;
  const uint8_t* w2s = p.w2s + (size_t)e * d * (I / 32);

  const uint8_t* arow[4];
  const uint8_t* brow[4];
  for (int q = 0; q < 4; ++q) {
    int row = (threadIdx.x >> 3) + 32 * q;
    int r = min(m0 + row, mend - 1);
    arow[q] = p.hq + (size_t)r * I;
    brow[q] = w2 + (size_t)(nt * BN + row) * I;
  }
  const uint8_t* srow;
  if (threadIdx.x < BM) {
    int r = min(m0 + (int)threadIdx.x, mend - 1);
    srow = p.hs + (size_t)r * (I / 32);
  } else {
    srow = w2s + (size_t)(nt * BN + threadIdx.x - BM) * (I / 32);
  }
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int b_row0[2] = {wn * 64, wn * 64 + 32};
  v16f acc[2][2];
  mainloop(lds, arow, brow, srow, I, wm * 64, b_row0, acc);

  const int l = lane_id(), i = l & 31, h = l >> 5;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int r = m0 + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (r >= mend) continue;
      float* dst = p.yslot + row_slot(s, r) * d + nt * BN + wn * 64 + i;
      dst[0] = acc[mi][0][v];
      dst[32] = acc[mi][1][v];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Backward dgrad of the down GEMM with the SwiGLU backward in the epilogue:
// dH = w * (dY_t W2t_e^T) (rows pulled from dYq: reverse-combine), dG = dH U s (1 + G (1 - s)),
// dU = dH silu(G); [dG dU] quantised along 2I.

__global__ __launch_bounds__(256) void k_gemm_dgrad_down(DgradDownArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int tile = blockIdx.y;
  if (tile >= s.tile_start[s.n_exp]) return;
  const int e = tile_expert(s.tile_start, s.n_exp, tile);
  const int m0 = s.offsets[e] + (tile - s.tile_start[e]) * BM;
  const int mend = s.offsets[e + 1];
  const int nt = blockIdx.x;  // 128 columns of I
  const int I = p.I, d = p.d;
  const uint8_t* w2t = p.w2tq + (size_t)e * I * d;
  const uint8_t* w2ts = p.w2ts + (size_t)e * I * (d / 32);

  const uint8_t* arow[4];
  const uint8_t* brow[4];
  for (int q = 0; q < 4; ++q) {
    int row = (threadIdx.x >> 3) + 32 * q;
    int r = min(m0 + row, mend - 1);
    arow[q] = p.dyq + (size_t)row_token(s, r) * d;
    brow[q] = w2t + (size_t)(nt * BN + row) * d;
  }
  const uint8_t* srow;
  if (threadIdx.x < BM) {
    int r = min(m0 + (int)threadIdx.x, mend - 1);
    srow = p.dys + (size_t)row_token(s, r) * (d / 32);
  } else {
    srow = w2ts + (size_t)(nt * BN + threadIdx.x - BM) * (d / 32);
  }
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int b_row0[2] = {wn * 64, wn * 64 + 32};
  v16f acc[2][2];
  mainloop(lds, arow, brow, srow, d, wm * 64, b_row0, acc);

  const int l = lane_id(), i = l & 31, h = l >> 5;
  const int I2 = 2 * I;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int r = m0 + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      int rc = min(r, mend - 1);
      float wr = row_weight(s, p.w, rc);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        int n = nt * BN + wn * 64 + ni * 32 + i;
        size_t o = (size_t)rc * I + n;
        float g = p.g[o], u = p.u[o];
        float dh = wr * acc[mi][ni][v];
        float sg = 1.0f / (1.0f + __expf(-g));
        float dg = dh * u * sg * (1.0f + g * (1.0f - sg));
        float du = dh * g * sg;
        uint32_t sc_g, sc_u;
        uint32_t cg = quant_lane32(dg, &sc_g);
        uint32_t cu = quant_lane32(du, &sc_u);
        if (r < mend) {
          size_t ro = (size_t)r * I2;
          p.dguq[ro + n] = (uint8_t)cg;
          p.dguq[ro + I + n] = (uint8_t)cu;
          if (i == 0) {
            p.dgus[(size_t)r * (I2 / 32) + (n >> 5)] = (uint8_t)sc_g;
            p.dgus[(size_t)r * (I2 / 32) + ((I + n) >> 5)] = (uint8_t)sc_u;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Backward dgrad of the gate/up GEMM: dX_r = dGU_r W1t_e^T, pushed to dXslot[t, j]
// (push reverse-dispatch).

__global__ __launch_bounds__(256) void k_gemm_dgrad_gateup(DgradGateUpArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int tile = blockIdx.y;
  if (tile >= s.tile_start[s.n_exp]) return;
  const int e = tile_expert(s.tile_start, s.n_exp, tile);
  const int m0 = s.offsets[e] + (tile - s.tile_start[e]) * BM;
  const int mend = s.offsets[e + 1];
  const int nt = blockIdx.x;  // 128 columns of d
  const int I2 = 2 * p.I, d = p.d;
  const uint8_t* w1t = p.w1tq + (size_t)e * d * I2;
  const uint8_t* w1ts = p.w1ts + (size_t)e * d * (I2 / 32);

  const uint8_t* arow[4];
  const uint8_t* brow[4];
  for (int q = 0; q < 4; ++q) {
    int row = (threadIdx.x >> 3) + 32 * q;
    int r = min(m0 + row, mend - 1);
    arow[q] = p.dguq + (size_t)r * I2;
    brow[q] = w1t + (size_t)(nt * BN + row) * I2;
  }
  const uint8_t* srow;
  if (threadIdx.x < BM) {
    int r = min(m0 + (int)threadIdx.x, mend - 1);
    srow = p.dgus + (size_t)r * (I2 / 32);
  } else {
    srow = w1ts + (size_t)(nt * BN + threadIdx.x - BM) * (I2 / 32);
  }
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int b_row0[2] = {wn * 64, wn * 64 + 32};
  v16f acc[2][2];
  mainloop(lds, arow, brow, srow, I2, wm * 64, b_row0, acc);

  const int l = lane_id(), i = l & 31, h = l >> 5;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int r = m0 + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (r >= mend) continue;
      float* dst = p.dxslot + row_slot(s, r) * d + nt * BN + wn * 64 + i;
      dst[0] = acc[mi][0][v];
      dst[32] = acc[mi][1][v];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Weight gradients: dW_e[m, n] = sum over the expert's tokens of At[m, tok] Bt[n, tok], both
// operands requantised along the token axis and stored token-contiguous at the expert's padded
// offset.  An expert with no tokens writes zeros.

__global__ __launch_bounds__(256) void k_gemm_wgrad(WgradArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int e = blockIdx.z;
  const int mt = blockIdx.y, nt = blockIdx.x;
  const int64_t k0 = p.tok_off[e];
  const int K = (int)(p.tok_off[e + 1] - k0);  // multiple of 128
  const int64_t ld = p.ld;                      // token stride of At / Bt rows
  const uint8_t* arow[4];
  const uint8_t* brow[4];
  for (int q = 0; q < 4; ++q) {
    int row = (threadIdx.x >> 3) + 32 * q;
    arow[q] = p.at + (size_t)(mt * BM + row) * ld + k0;
    brow[q] = p.bt + (size_t)(nt * BN + row) * ld + k0;
  }
  const uint8_t* srow;
  if (threadIdx.x < BM)
    srow = p.ats + (size_t)(mt * BM + threadIdx.x) * (ld / 32) + k0 / 32;
  else
    srow = p.bts + (size_t)(nt * BN + threadIdx.x - BM) * (ld / 32) + k0 / 32;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int b_row0[2] = {wn * 64, wn * 64 + 32};
  v16f acc[2][2];
  mainloop(lds, arow, brow, srow, K, wm * 64, b_row0, acc);

  const int l = lane_id(), i = l & 31, h = l >> 5;
  float* out = p.dw + (size_t)e * p.M * p.N;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int m = mt * BM + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      float* dst = out + (size_t)m * p.N + nt * BN + wn * 64 + i;
      __builtin_nontemporal_store(acc[mi][0][v], dst);
      __builtin_nontemporal_store(acc[mi][1][v], dst + 32);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launchers

size_t gemm_lds_bytes() { return 2 * STAGE_BYTES; }

hipError_t launch_gemm_gateup(const GateUpArgs& a, int tiles_bound, hipStream_t st) {
  dim3 grid(a.I / 64, tiles_bound);
  hipLaunchKernelGGL(k_gemm_gateup, grid, dim3(256), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const DownArgs& a, int tiles_bound, hipStream_t st) {
  dim3 grid(a.d / BN, tiles_bound);
  hipLaunchKernelGGL(k_gemm_down, grid, dim3(256), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_dgrad_down(const DgradDownArgs& a, int tiles_bound, hipStream_t st) {
  dim3 grid(a.I / BN, tiles_bound);
  hipLaunchKernelGGL(k_gemm_dgrad_down, grid, dim3(256), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_dgrad_gateup(const DgradGateUpArgs& a, int tiles_bound, hipStream_t st) {
  dim3 grid(a.d / BN, tiles_bound);
  hipLaunchKernelGGL(k_gemm_dgrad_gateup, grid, dim3(256), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad(const WgradArgs& a, int n_exp, hipStream_t st) {
  dim3 grid(a.N / BN, a.M / BM, n_exp);
  hipLaunchKernelGGL(k_gemm_wgrad, grid, dim3(256), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
hipError_t gemm_init() {
  const int bytes = (int)gemm_lds_bytes();
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_gateup, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_down, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_dgrad_down, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_dgrad_gateup, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_wgrad, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  return hipSuccess;
}
}  // namespace moe
