// Core of the grouped MXFP8 GEMMs (shared by the direct kernels and the ring kernel).
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
// 8(v/4) + 4h + v%4, column i.  The instruction must run with every lane active.
//
// Work tile: 128 rows x 128 columns per 256-thread workgroup; each of the four
// waves owns a 64 x 64 quarter as 2 x 2 MFMA tiles.  K advances 128 at a time
// through double-buffered LDS (rows padded to 144 bytes: conflict-free 16-byte
// reads).  Each output tile is owned by exactly one workgroup and K is summed in
// a fixed order, so results are bitwise reproducible.
#pragma once
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

// Device-coherent 16-byte read as two relaxed agent-scope 64-bit atomic loads: it observes data
// another workgroup published (release) without invalidating any cache level.
MOE_DEV v4i load16_coherent(const uint8_t* p) {
  uint64_t* q = (uint64_t*)p;
  uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (v4i){(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi, (int)(uint32_t)(hi >> 32)};
}

// kCoherentA: the A operand (rows and their scales) was written by other workgroups of the same
// kernel (ring buffers) and is read with device-coherent loads.
template <bool kCoherentA = false>
MOE_DEV void load_stage(Stage& st, const uint8_t* const* arow, const uint8_t* const* brow,
                        const uint8_t* srow, int k0) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int col = (threadIdx.x & 7) * 16;
    st.a[q] = kCoherentA ? load16_coherent(arow[q] + k0 + col) : *(const v4i*)(arow[q] + k0 + col);
    st.b[q] = *(const v4i*)(brow[q] + k0 + col);
  }
  if (kCoherentA && threadIdx.x < BM)
    st.s = __hip_atomic_load((uint32_t*)(srow + (k0 >> 5)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
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
template <bool kCoherentA = false>
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
  load_stage<kCoherentA>(st, arow, brow, srow, 0);
  store_stage(st, lds);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * STAGE_BYTES;
    if (kt + 1 < nk) load_stage<kCoherentA>(st, arow, brow, srow, (kt + 1) * BK);
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


// Gate/up epilogue shared by the direct and the ring kernels: G and U of the same element sit
// in the same lane (the tile's columns are 64 gate + the matching 64 up columns); h = silu(G) U
// is quantised along I in 32-column blocks held by the 32 lanes of a half-wave.
MOE_DEV void gateup_epilogue(const v16f (&acc)[2][2], int m0, int mend, int nt, int wm, int wn, int I, float* g_out,
                             float* u_out, uint8_t* hq, uint8_t* hs) {
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
        g_out[o] = g;
        u_out[o] = u;
        hq[o] = (uint8_t)code;
        if (i == 0) hs[(size_t)r * (I / 32) + (n >> 5)] = (uint8_t)sc;
      }
    }
  }
}

}  // namespace
}  // namespace moe
