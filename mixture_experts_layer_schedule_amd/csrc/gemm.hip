// Grouped MXFP8 GEMMs of the expert FFN (forward, dgrad and wgrad) on gfx950.
//
// Every GEMM here is "NT": both operands are stored with the reduction axis K
// contiguous and MXFP8-quantised along K (one e8m0 byte per 32 values).  The
// product runs on v_mfma_scale_f32_32x32x64_f8f6f4, which applies the block
// scales inside the matrix core, with float32 accumulation.
//
// Operand layout of that instruction, measured on the device: lane l = i + 32h
// (i = l % 32, h = l / 32) holds row i; its 32 bytes are elements
// [16h, 16h + 16) of the step's first 32-wide K block followed by elements
// [16h, 16h + 16) of the second block.  Lane l's scale byte is that of row i,
// K block h.  The 32x32 float32 result sits in lane l, register v at row
// 8(v/4) + 4h + v%4, column i.
//
// Work tile: 128 rows x 128 columns per 256-thread workgroup; each of the four
// waves owns a 64 x 64 quarter as 2 x 2 MFMA tiles.  K advances 128 at a time
// through double-buffered LDS (rows padded to 144 bytes: conflict-free 16-byte
// reads).  Each output tile is owned by exactly one workgroup and K is summed in
// a fixed order, so results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 16;               // bytes per staged row
constexpr int TILE_BYTES = BM * LDS_STRIDE;       // one operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES + 2 * BM * 4;  // A, B, A scales, B scales

// Row of the tile table: which expert a 128-row tile of permuted rows belongs to.
MOE_DEV int tile_expert(const int32_t* tile_start, int n_exp, int tile) {
  int lo = 0, hi = n_exp;  // tile_start[lo] <= tile < tile_start[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// Slot (t * (k + S) + j) of permuted row r.
MOE_DEV int64_t row_slot(const SchedView& s, int r) {
  if (r < s.R) {
    int sid = s.perm[r];
    int t = sid / s.k;
    return (int64_t)t * (s.k + s.S) + (sid - t * s.k);
  }
  int q = r - s.R;
  int sh = q / s.T;
  return (int64_t)(q - sh * s.T) * (s.k + s.S) + s.k + sh;
}

MOE_DEV int row_token(const SchedView& s, int r) {
  if (r < s.R) return s.perm[r] / s.k;
  return (r - s.R) % s.T;
}

MOE_DEV float row_weight(const SchedView& s, const float* w, int r) {
  return r < s.R ? w[s.perm[r]] : 1.0f;
}

struct Frag {
  v8i a[2], b[2];
  int sa[2], sb[2];
};

// Loads of one BK slice into registers: 4 x 16 B of A and of B per thread, plus one
// 4-byte scale word (threads 0..127: A rows, 128..255: B rows).
struct Stage {
  v4i a[4], b[4];
  uint32_t s;
};

MOE_DEV void load_stage(Stage& st, const uint8_t* const* arow, const uint8_t* const* brow,
                        const uint8_t* srow, int k0) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int col = (threadIdx.x & 7) * 16;
    st.a[q] = *(const v4i*)(arow[q] + k0 + col);
    st.b[q] = *(const v4i*)(brow[q] + k0 + col);
  }
  st.s = *(const uint32_t*)(srow + (k0 >> 5));
}

MOE_DEV void store_stage(const Stage& st, uint8_t* lds) {
  int row0 = threadIdx.x >> 3;
  int col = (threadIdx.x & 7) * 16;
  uint8_t* A = lds;
  uint8_t* B = lds + TILE_BYTES;
  uint32_t* S = (uint32_t*)(lds + 2 * TILE_BYTES);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int row = row0 + 32 * q;
    *(v4i*)(A + row * LDS_STRIDE + col) = st.a[q];
    *(v4i*)(B + row * LDS_STRIDE + col) = st.b[q];
  }
  S[threadIdx.x] = st.s;  // [0, 128): A rows, [128, 256): B rows
}

// One 128-deep slice: two MFMA K-steps over the wave's 2 x 2 tiles.
// b_row0[ni]: first B-tile row of the wave's ni-th 32-column group.
MOE_DEV void compute_stage(const uint8_t* lds, int a_row0, const int* b_row0, v16f (&acc)[2][2]) {
  const int l = lane_id();
  const int i = l & 31, h = l >> 5;
  const uint8_t* A = lds;
  const uint8_t* B = lds + TILE_BYTES;
  const uint32_t* S = (const uint32_t*)(lds + 2 * TILE_BYTES);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    v8i a[2], b[2];
    int sa[2], sb[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      int row = a_row0 + mi * 32 + i;
      const uint8_t* p = A + row * LDS_STRIDE + kk * 64 + 16 * h;
      v4i lo = *(const v4i*)p, hi = *(const v4i*)(p + 32);
      a[mi] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sa[mi] = (int)((S[row] >> (8 * (2 * kk + h))) & 0xFFu);
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      int row = b_row0[ni] + i;
      const uint8_t* p = B + row * LDS_STRIDE + kk * 64 + 16 * h;
      v4i lo = *(const v4i*)p, hi = *(const v4i*)(p + 32);
      b[ni] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sb[ni] = (int)((S[BM + row] >> (8 * (2 * kk + h))) & 0xFFu);
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[mi], b[ni], acc[mi][ni], 0, 0, 0,
                                                                        sa[mi], 0, sb[ni]);
  }
}

// Main loop: acc = A_tile * B_tile^T over K.
MOE_DEV void mainloop(uint8_t* lds, const uint8_t* const* arow, const uint8_t* const* brow,
                      const uint8_t* srow, int K, int a_row0, const int* b_row0, v16f (&acc)[2][2]) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
  const int nk = K / BK;
  if (nk == 0) return;
  Stage st;
  load_stage(st, arow, brow, srow, 0);
  store_stage(st, lds);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * STAGE_BYTES;
    if (kt + 1 < nk) load_stage(st, arow, brow, srow, (kt + 1) * BK);
    compute_stage(cur, a_row0, b_row0, acc);
    if (kt + 1 < nk) store_stage(st, lds + ((kt + 1) & 1) * STAGE_BYTES);
    __syncthreads();
  }
}

// Quantise 32 consecutive columns of one row held by the 32 lanes of a half-wave:
// returns this lane's code; *scale receives the block's e8m0 byte.
MOE_DEV uint32_t quant_lane32(float v, uint32_t* scale) {
  float amax = group_max<32>(fabsf(v));
  uint32_t byte = e8m0_from_amax(amax);
  *scale = byte;
  float x = clamp448(v * e8m0_inv_scale(byte));
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFFu;
}

MOE_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace

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

  const int l = lane_id(), i = l & 31, h = l >> 5;
  const int n = nt * 64 + wn * 32 + i;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int r = m0 + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      float g = acc[mi][0][v], u = acc[mi][1][v];
      float hv = silu(g) * u;
      uint32_t sc;
      uint32_t code = quant_lane32(hv, &sc);
      if (r < mend) {
        size_t o = (size_t)r * I + n;
        p.g[o] = g;
        p.u[o] = u;
        p.hq[o] = (uint8_t)code;
        if (i == 0) p.hs[(size_t)r * (I / 32) + (n >> 5)] = (uint8_t)sc;
      }
    }
  }
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
