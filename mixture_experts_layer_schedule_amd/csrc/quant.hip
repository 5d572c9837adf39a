// MXFP8 quantisation kernels: along rows, transposed requantisation of expert weights, and
// token-axis requantisation of expert rows for the weight-gradient GEMMs.
//
// MXFP8 is the OCP Microscaling v1.0 format named by the pages for the whole layer
// (knowledge card "Mixture-of-Kittens——面向NVL72的开源MoE训练megakernel", 方法/产品要点):
// blocks of 32 values share an e8m0 exponent floor(log2 amax) - 8; elements are e4m3 with
// round-to-nearest-even and saturation at 448.  All three kernels stream HBM: loads and stores
// are 16 bytes per lane and every block is reduced across the lanes that hold it.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// ----------------------------------------------------------------------------- along rows

// Each lane owns 8 consecutive values; 4 lanes form a 32-value block.
template <bool F32>
__global__ __launch_bounds__(256) void k_quant_rows(const void* __restrict__ src, int64_t n8,
                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n8; g += stride) {
    float v[8];
    if (F32) {
      const v4f* p = (const v4f*)src + 2 * g;
      v4f a = p[0], b = p[1];
      v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
      v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    } else {
      v4i a = ((const v4i*)src)[g];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = (uint32_t)a[j];
        v[2 * j] = __uint_as_float(w << 16);
        v[2 * j + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    m = group_max<4>(m);
    uint32_t byte = e8m0_from_amax(m);
    float inv = e8m0_inv_scale(byte);
    v2i out;
    out[0] = (int)pack4_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    out[1] = (int)pack4_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    ((v2i*)q)[g] = out;
    if ((g & 3) == 0) s[g >> 2] = (uint8_t)byte;
  }
}

// ----------------------------------------------------------------------------- transposed tiles
//
// A 64 x 64 float tile is staged in LDS transposed (tile[c][r]); each output row c is then
// quantised along r in two 32-value blocks.  Lane t handles output row t / 4, values
// [16 (t % 4), +16); lanes t and t ^ 1 share a block.

constexpr int TS = 64;
constexpr int TP = TS + 1;  // padded row of the LDS tile (floats)

MOE_DEV void quant_tile_out(const float* tile, uint8_t* out_row, uint8_t* out_scale_row, int part) {
  const int c = threadIdx.x >> 2;
  const float* src = tile + c * TP + 16 * part;
  float v[16];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    v[j] = src[j];
    m = fmaxf(m, fabsf(v[j]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  uint32_t byte = e8m0_from_amax(m);
  float inv = e8m0_inv_scale(byte);
  v4i o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = (int)pack4_e4m3(v[4 * j] * inv, v[4 * j + 1] * inv, v[4 * j + 2] * inv, v[4 * j + 3] * inv);
  *(v4i*)(out_row + 16 * part) = o;
  if ((part & 1) == 0) out_scale_row[part >> 1] = (uint8_t)byte;
}

// Dequantise 16 codes that share one scale byte into floats.
MOE_DEV void dq16(v4i codes, uint32_t sbyte, float* v) {
  float sc = e8m0_scale(sbyte);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = (uint32_t)codes[j];
#pragma unroll
    for (int b = 0; b < 4; ++b) v[4 * j + b] = e4m3_to_f32((w >> (8 * b)) & 0xFFu) * sc;
  }
}

// [batch][rows][cols] (blocks along cols) -> [batch][cols][rows] (blocks along rows)
__global__ __launch_bounds__(256) void k_requant_t(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                   int64_t rows, int64_t cols, uint8_t* __restrict__ qt,
                                                   uint8_t* __restrict__ st) {
  __shared__ float tile[TS * TP];
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * TS, c0 = (int64_t)blockIdx.x * TS;
  const int t = threadIdx.x;
  {
    const int r = t >> 2, part = t & 3;
    const int64_t row = r0 + r, col = c0 + 16 * part;
    v4i codes = *(const v4i*)(q + (b * rows + row) * cols + col);
    uint32_t sb = s[(b * rows + row) * (cols / 32) + col / 32];
    float v[16];
    dq16(codes, sb, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) tile[(16 * part + j) * TP + r] = v[j];
  }
  __syncthreads();
  const int c = t >> 2, part = t & 3;
  quant_tile_out(tile, qt + (b * cols + c0 + c) * rows + r0, st + (b * cols + c0 + c) * (rows / 32) + r0 / 32,
                 part);
}


// [batch][rows][cols] (blocks along cols) -> [batch][cols][rows] (blocks along rows) on 128 x 128
// tiles, staged in LDS as fp8 codes (17 KB per tile, so many tiles are in flight per CU).
// Loads: thread t reads rows 4(t/8) .. +4, columns 16(t%8) .. +16 (8 lanes cover a whole
// 128-byte line of a row) and writes each column's 4 codes as one LDS word.  Stores: thread t
// produces output row t/2 (input column), input rows [64 (t%2), +64): two output blocks whose
// maxima need no cross-lane traffic, written as one 64-byte run.  Codes are decoded two at a
// time by the hardware conversion (exact for e4m3) and scaled by their e8m0 factor.
constexpr int RT = 128;
constexpr int RPITCH = RT + 4;  // bytes per LDS code row: word reads and writes are conflict-light

__global__ __launch_bounds__(256) void k_requant_t128(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                     int64_t rows, int64_t cols, uint8_t* __restrict__ qt,
                                                     uint8_t* __restrict__ st) {
  __shared__ __align__(16) uint8_t ct[RT * RPITCH];  // ct[c][r]: code of input (r, c)
  __shared__ __align__(16) uint8_t sct[4][RT];       // sct[c / 32][r]: scale byte of input (r, c)
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * RT, c0 = (int64_t)blockIdx.x * RT;
  const int t = threadIdx.x;
  {
    const int rg = t >> 3, cg = t & 7;
    v4i w[4];
    uint32_t sb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = b * rows + r0 + 4 * rg + j;
      w[j] = *(const v4i*)(q + row * cols + c0 + 16 * cg);
      sb |= (uint32_t)s[row * (cols / 32) + (c0 + 16 * cg) / 32] << (8 * j);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int sh = 8 * (m & 3);
      const uint32_t col4 = (((uint32_t)w[0][m >> 2] >> sh) & 0xFFu) | ((((uint32_t)w[1][m >> 2] >> sh) & 0xFFu) << 8) |
                            ((((uint32_t)w[2][m >> 2] >> sh) & 0xFFu) << 16) | ((((uint32_t)w[3][m >> 2] >> sh) & 0xFFu) << 24);
      *(uint32_t*)(ct + (16 * cg + m) * RPITCH + 4 * rg) = col4;
    }
    if ((cg & 1) == 0) *(uint32_t*)(&sct[cg >> 1][4 * rg]) = sb;
  }
  __syncthreads();
  const int c = t >> 1, half = t & 1;
  const uint32_t* crow = (const uint32_t*)(ct + c * RPITCH + 64 * half);
  const uint32_t* srow = (const uint32_t*)(&sct[c >> 5][64 * half]);
  uint8_t* dst = qt + (b * cols + c0 + c) * rows + r0 + 64 * half;
  uint8_t* sdst = st + (b * cols + c0 + c) * (rows / 32) + (r0 + 64 * half) / 32;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float v[32];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // 4 codes of 4 consecutive rows per word
      const uint32_t codes = crow[8 * blk + k];
      const uint32_t sc4 = srow[8 * blk + k];
      const v2f p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);
      const v2f p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);
      v[4 * k + 0] = p0[0] * e8m0_scale(sc4 & 0xFFu);
      v[4 * k + 1] = p0[1] * e8m0_scale((sc4 >> 8) & 0xFFu);
      v[4 * k + 2] = p1[0] * e8m0_scale((sc4 >> 16) & 0xFFu);
      v[4 * k + 3] = p1[1] * e8m0_scale(sc4 >> 24);
#pragma unroll
      for (int x = 0; x < 4; ++x) m = fmaxf(m, fabsf(v[4 * k + x]));
    }
    const uint32_t byte = e8m0_from_amax(m);
    const float inv = e8m0_inv_scale(byte);
    v4i o0, o1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o0[k] = (int)pack4_e4m3(v[4 * k] * inv, v[4 * k + 1] * inv, v[4 * k + 2] * inv, v[4 * k + 3] * inv);
      o1[k] = (int)pack4_e4m3(v[16 + 4 * k] * inv, v[16 + 4 * k + 1] * inv, v[16 + 4 * k + 2] * inv,
                              v[16 + 4 * k + 3] * inv);
    }
    ((v4i*)dst)[2 * blk] = o0;
    ((v4i*)dst)[2 * blk + 1] = o1;
    sdst[blk] = (uint8_t)byte;
  }
}

MOE_DEV int find_tile(const int32_t* start, int n, int tile) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (start[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// Token-axis requantisation: 128 tokens of one expert x 128 columns per workgroup, the
// 128 x 128 transposed scheme above with the rows gathered through the schedule.  Token x of
// the tile is the expert's row tl + x (zero past its rows: the segment's padding); for X and w*dY
// the source row is that row's token, for H and [dG dU] the permuted row itself.  Loads: 8 lanes
// cover a whole 128-byte line of a source row; stores: each output row (a column of the source)
// gets 128 contiguous token codes from two lanes.  w*dY multiplies the exactly dequantised value
// by the row's combine weight before the requantisation.
__global__ __launch_bounds__(256) void k_token_requant(TokArgs p) {
  __shared__ __align__(16) uint8_t ct[RT * RPITCH];  // ct[c][x]: code of token x, column c
  __shared__ __align__(16) uint8_t sct[4][RT];       // sct[c / 32][x]: its scale byte
  __shared__ float wt[RT];                            // combine weight of token x (w*dY)
  const SchedView& s = p.s;
  const int t128 = blockIdx.y;
  if (2 * t128 >= p.tile64[s.n_exp]) return;
  const int e = find_tile(p.tile64, s.n_exp, 2 * t128);  // segments are 128-padded: even 64-tiles
  const int tl = (2 * t128 - p.tile64[e]) * TS;            // first local token of the tile
  const int r0 = s.offsets[e];
  const int cnt = s.offsets[e + 1] - r0;
  const int64_t c0 = (int64_t)blockIdx.x * RT;
  const int t = threadIdx.x;
  {
    const int rg = t >> 3, cg = t & 7;
    v4i w[4];
    uint32_t sb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = 4 * rg + j;
      if (tl + x < cnt) {
        const int r = r0 + tl + x;
        int64_t srow;
        if (p.src == TOK_X || p.src == TOK_DYW) srow = r < s.R ? s.perm[r] / s.k : (r - s.R) % s.T;
        else srow = r;
        w[j] = *(const v4i*)(p.q + srow * p.cols + c0 + 16 * cg);
        sb |= (uint32_t)p.qs[srow * (p.cols / 32) + (c0 + 16 * cg) / 32] << (8 * j);
      } else {
        w[j] = (v4i){0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int sh = 8 * (m & 3);
      const uint32_t col4 = (((uint32_t)w[0][m >> 2] >> sh) & 0xFFu) | ((((uint32_t)w[1][m >> 2] >> sh) & 0xFFu) << 8) |
                            ((((uint32_t)w[2][m >> 2] >> sh) & 0xFFu) << 16) | ((((uint32_t)w[3][m >> 2] >> sh) & 0xFFu) << 24);
      *(uint32_t*)(ct + (16 * cg + m) * RPITCH + 4 * rg) = col4;
    }
    if ((cg & 1) == 0) *(uint32_t*)(&sct[cg >> 1][4 * rg]) = sb;
    if (t < RT) {
      const int r = r0 + tl + t;
      wt[t] = (p.src == TOK_DYW && tl + t < cnt && r < s.R) ? p.w[s.perm[r]] : 1.0f;
    }
  }
  __syncthreads();
  const int c = t >> 1, half = t & 1;
  const uint32_t* crow = (const uint32_t*)(ct + c * RPITCH + 64 * half);
  const uint32_t* srow = (const uint32_t*)(&sct[c >> 5][64 * half]);
  const int64_t o = p.tok_off[e] + tl + 64 * half;  // output token column
  uint8_t* dst = p.out + (c0 + c) * p.ld + o;
  uint8_t* sdst = p.outs + (c0 + c) * (p.ld / 32) + o / 32;
  const bool dyw = p.src == TOK_DYW;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float v[32];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // 4 codes of 4 consecutive tokens per word
      const uint32_t codes = crow[8 * blk + k];
      const uint32_t sc4 = srow[8 * blk + k];
      const v2f p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);
      const v2f p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);
      v[4 * k + 0] = p0[0] * e8m0_scale(sc4 & 0xFFu);
      v[4 * k + 1] = p0[1] * e8m0_scale((sc4 >> 8) & 0xFFu);
      v[4 * k + 2] = p1[0] * e8m0_scale((sc4 >> 16) & 0xFFu);
      v[4 * k + 3] = p1[1] * e8m0_scale(sc4 >> 24);
      if (dyw) {
#pragma unroll
        for (int x = 0; x < 4; ++x) v[4 * k + x] *= wt[64 * half + 32 * blk + 4 * k + x];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) m = fmaxf(m, fabsf(v[4 * k + x]));
    }
    const uint32_t byte = e8m0_from_amax(m);
    const float inv = e8m0_inv_scale(byte);
    v4i o0, o1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o0[k] = (int)pack4_e4m3(v[4 * k] * inv, v[4 * k + 1] * inv, v[4 * k + 2] * inv, v[4 * k + 3] * inv);
      o1[k] = (int)pack4_e4m3(v[16 + 4 * k] * inv, v[16 + 4 * k + 1] * inv, v[16 + 4 * k + 2] * inv,
                              v[16 + 4 * k + 3] * inv);
    }
    ((v4i*)dst)[2 * blk] = o0;
    ((v4i*)dst)[2 * blk + 1] = o1;
    sdst[blk] = (uint8_t)byte;
  }
}

}  // namespace

hipError_t launch_quant_rows(const void* src, int src_f32, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                             hipStream_t st) {
  int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (src_f32)
    hipLaunchKernelGGL(k_quant_rows<true>, dim3((unsigned)blocks), dim3(256), 0, st, src, n8, q, s);
  else
    hipLaunchKernelGGL(k_quant_rows<false>, dim3((unsigned)blocks), dim3(256), 0, st, src, n8, q, s);
  return hipGetLastError();
}

hipError_t launch_requant_t(const uint8_t* q, const uint8_t* s, int64_t batch, int64_t rows, int64_t cols,
                            uint8_t* qt, uint8_t* st, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (rows % RT == 0 && cols % RT == 0) {
    dim3 grid((unsigned)(cols / RT), (unsigned)(rows / RT), (unsigned)batch);
    hipLaunchKernelGGL(k_requant_t128, grid, dim3(256), 0, stream, q, s, rows, cols, qt, st);
  } else {
    dim3 grid((unsigned)(cols / TS), (unsigned)(rows / TS), (unsigned)batch);
    hipLaunchKernelGGL(k_requant_t, grid, dim3(256), 0, stream, q, s, rows, cols, qt, st);
  }
  return hipGetLastError();
}

hipError_t launch_token_requant(const TokArgs& a, int tiles_bound, hipStream_t stream) {
  if (a.cols % RT) return hipErrorInvalidValue;
  // tiles_bound counts 64-token tiles; the kernel takes 128 tokens per workgroup
  dim3 grid((unsigned)(a.cols / RT), (unsigned)((tiles_bound + 1) / 2));
  hipLaunchKernelGGL(k_token_requant, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
