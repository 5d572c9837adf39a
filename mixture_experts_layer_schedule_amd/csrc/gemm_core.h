// Core of the grouped MXFP8 GEMMs (shared by the direct kernels and the ring kernel).
//
// Every GEMM here is "NT": both operands are stored with the reduction axis K contiguous and
// MXFP8-quantised along K (one e8m0 byte per 32 values).  The product runs on
// v_mfma_scale_f32_32x32x64_f8f6f4, which applies the block scales inside the matrix core, with
// float32 accumulation.
//
// Operand layout of that instruction, measured on the device: lane l = i + 32h (i = l % 32,
// h = l / 32) holds row i; its 32 bytes are elements [16h, 16h + 16) of the step's first 32-wide
// K block followed by elements [16h, 16h + 16) of the second block.  Lane l's scale byte is that
// of row i, K block h.  The 32x32 float32 result sits in lane l, register v at row
// 8(v/4) + 4h + v%4, column i.  The instruction must run with every lane active.
//
// Work tile: up to 256 rows (F row fragments of 32) x 256 columns per 256-thread workgroup.
// Wave w owns columns [64w, 64w + 64) as two 32-column fragments and every row fragment, so a
// ragged row count shortens every wave's work equally.  The accumulators (F x 2 MFMA tiles)
// stay in registers for the whole K loop.
//
// K pipeline: stages of 64 (one MFMA step) in an NST-deep ring of LDS buffers, filled by
// direct-to-LDS loads (global_load_lds_dwordx4: no registers in between), so NST - 1 stages
// are in flight while one is multiplied.  Each staged row is 64 bytes; its four 16-byte chunks
// are XOR-swizzled by the row index so that the fragment reads (lane i reads row i) hit
// distinct banks.  Scales travel the same way, one 4-byte word per row every other stage.
// One barrier per stage: it publishes the stage every wave loaded a share of and retires the
// buffer that the next loads overwrite.
//
// Each output tile is owned by exactly one workgroup and K is summed in a fixed order, so
// results are bitwise reproducible.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int TM = 256;                      // rows of a full tile (8 fragments of 32)
constexpr int TN = 256;                      // columns of a tile (4 waves x 64)
constexpr int KS = 64;                       // K per pipeline stage
constexpr int A_STAGE = TM * KS;             // bytes of one staged A slice
constexpr int STAGE_BYTES = (TM + TN) * KS;  // A then B
constexpr int EPOCH_BYTES = (TM + TN) * 4;   // one scale word (4 K blocks) per row
constexpr int NEPOCH = 3;                    // scale-word buffers

constexpr size_t lds_bytes_for(int nst) { return (size_t)nst * STAGE_BYTES + NEPOCH * EPOCH_BYTES; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Physical 16-byte chunk slot of logical chunk g in staged row r is g ^ swz(r).  For any 16
// consecutive rows (and any 8), rows with equal r % 4 (r % 2) get distinct slots, so the
// fragment reads are conflict-free whether the LDS serves 16 or 8 lanes per cycle.
MOE_DEV int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Which expert a tile belongs to, from a prefix table of tiles per expert.
MOE_DEV int tile_expert(const int32_t* tile_start, int n_exp, int tile) {
  int lo = 0, hi = n_exp;  // tile_start[lo] <= tile < tile_start[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// Rows [r0, r0 + rows) of expert e covered by its m-th row tile.  An expert with c rows has
// ceil(c / 256) tiles; the rows are split evenly between them in multiples of 32, so a 300-row
// expert runs as two 160-row tiles rather than 256 + 44.  rows <= 0 only for experts of more
// than 2048 rows, whose last tile can come out empty.
struct RowTile {
  int e, r0, rows;
};
MOE_DEV RowTile row_tile(const SchedView& s, int tile) {
  RowTile t;
  t.e = tile_expert(s.tile_start, s.n_exp, tile);
  const int m = tile - s.tile_start[t.e];
  const int nm = s.tile_start[t.e + 1] - s.tile_start[t.e];
  const int c = s.offsets[t.e + 1] - s.offsets[t.e];
  const int per = ((c + nm - 1) / nm + 31) & ~31;
  t.r0 = s.offsets[t.e] + m * per;
  t.rows = min(per, c - m * per);
  return t;
}

// Work item of a grouped launch.  Blocks are dealt round-robin to the 8 XCDs, so the linear
// block id is remapped to give each XCD a contiguous range of (row tile, column tile) items:
// consecutive items share the A rows (one row tile, successive column tiles) and the items of
// one expert share its weights, so both are reused from that XCD's L2.  false past the end.
MOE_DEV bool xcd_item(int total, int* item) {
  const int b = blockIdx.x;
  if (b >= total) return false;
  const int x = b & 7, q = b >> 3;
  const int base = total >> 3, rem = total & 7;
  *item = x * base + min(x, rem) + q;
  return true;
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

// Per-thread source addresses of the direct-to-LDS loads of one tile.  Staged rows are filled
// 16 per wave instruction: instruction q (wave q % 4) covers rows [16q, 16q + 16), lane l the
// row 16q + l / 4, chunk slot l % 4.  a_rows(r) / b_rows(r) return the K data of staged row r
// (callers clamp rows past the operand to a valid one; such rows are never stored) and
// a_srows / b_srows its scale bytes.
template <int F>
struct TileLoads {
  static constexpr int NA = (F + 1) / 2;  // A instructions per wave and stage (2F over 4 waves)
  const uint8_t* a[NA];
  const uint8_t* b[4];
  const uint8_t* as;
  const uint8_t* bs;

  template <class ARow, class BRow, class ASRow, class BSRow>
  MOE_DEV void init(ARow a_rows, BRow b_rows, ASRow a_srows, BSRow b_srows) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int sub = l >> 2, slot = l & 3;
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int r = 16 * (w + 4 * u) + sub;  // for odd F the last rows are filled, never read
      a[u] = a_rows(r) + 16 * (slot ^ swz(r));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 16 * (w + 4 * u) + sub;
      b[u] = b_rows(r) + 16 * (slot ^ swz(r));
    }
    as = a_srows(64 * w + l);
    bs = b_srows(64 * w + l);
  }
};

template <int AUX>
MOE_DEV void lds_load16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)dst, 16, 0, AUX);
}
template <int AUX>
MOE_DEV void lds_load4(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)dst, 4, 0, AUX);
}

// Loads of stage t (K offset 64t) into its buffer; even stages also bring the scale words of
// K range [64t, 64t + 128).  AUX_A: cache-policy bits of the A loads (16 = sc1: device-coherent
// reads of rows that other workgroups of the same kernel wrote).
template <int F, int NST, int AUX_A>
MOE_DEV void issue_stage(const TileLoads<F>& L, uint8_t* lds, int t) {
  const int w = threadIdx.x >> 6;
  const int k0 = t * KS;
  uint8_t* st = lds + (t % NST) * STAGE_BYTES;
  if ((t & 1) == 0) {
    uint8_t* ep = lds + NST * STAGE_BYTES + ((t >> 1) % NEPOCH) * EPOCH_BYTES;
    lds_load4<AUX_A>(L.as + (k0 >> 5), ep + 256 * w);
    lds_load4<0>(L.bs + (k0 >> 5), ep + TM * 4 + 256 * w);
  }
#pragma unroll
  for (int u = 0; u < TileLoads<F>::NA; ++u) lds_load16<AUX_A>(L.a[u] + k0, st + 1024 * (w + 4 * u));
#pragma unroll
  for (int u = 0; u < 4; ++u) lds_load16<0>(L.b[u] + k0, st + A_STAGE + 1024 * (w + 4 * u));
}

// Wait until at most N of this wave's loads are outstanding, then meet the other waves.  The
// wait and the barrier are one statement so that no LDS access moves across either.
template <int N>
MOE_DEV void wait_loads_and_sync() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Multiply one staged K slice: acc[mi][ni] += A_frag(mi) * B_frag(ni).  sa/sb hold this lane's
// scale words (already shifted to its K block h); p selects the stage's half of the word.
template <int F>
MOE_DEV void compute_stage(const uint8_t* st, const uint32_t (&sa)[F], const uint32_t (&sb)[2], int p,
                           v16f (&acc)[F][2]) {
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int o_lo = 16 * (h ^ swz(i)), o_hi = 16 * ((2 + h) ^ swz(i));
  v8i b[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const uint8_t* rp = st + A_STAGE + (64 * w + 32 * ni + i) * KS;
    const v4i lo = *(const v4i*)(rp + o_lo), hi = *(const v4i*)(rp + o_hi);
    b[ni] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  const int sh = 16 * p;
  const int sb0 = (int)(sb[0] >> sh), sb1 = (int)(sb[1] >> sh);
  static_for<F>([&]<int mi>() {
    const uint8_t* rp = st + (32 * mi + i) * KS;
    const v4i lo = *(const v4i*)(rp + o_lo), hi = *(const v4i*)(rp + o_hi);
    const v8i a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const int s_a = (int)(sa[mi] >> sh);
    acc[mi][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[0], acc[mi][0], 0, 0, 0, s_a, 0, sb0);
    acc[mi][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[1], acc[mi][1], 0, 0, 0, s_a, 0, sb1);
  });
}

// acc = A_tile * B_tile^T over K = 64 * nk.  active (wave-uniform): this wave's columns exist;
// an inactive wave still loads its share and meets every barrier.
// Loads per wave and stage: NA + 4 data instructions, plus 2 scale words on even stages.
template <int F, int NST, int AUX_A = 0>
MOE_DEV void mainloop(uint8_t* lds, const TileLoads<F>& L, int nk, bool active, v16f (&acc)[F][2]) {
  static_assert(NST >= 2 && NST <= 4, "pipeline depth");
  constexpr int LD = TileLoads<F>::NA + 4;  // data loads of one stage
  static_for<F>([&]<int mi>() {
    acc[mi][0] = (v16f){};
    acc[mi][1] = (v16f){};
  });
  const int w = threadIdx.x >> 6, l = lane_id(), i = l & 31, h = l >> 5;
  for (int t = 0; t < NST - 1 && t < nk; ++t) issue_stage<F, NST, AUX_A>(L, lds, t);
  uint32_t sa[F], sb[2];
  for (int t = 0; t < nk; ++t) {
    // this wave's loads of stages t+1 .. t+ahead may stay in flight
    const int ahead = min(nk - 1 - t, NST - 2);
    if (NST == 4 && ahead == 2) {
      wait_loads_and_sync<2 * LD + 2>();  // one of the two stages is even (+2 scale words)
    } else if (ahead == 1) {
      if ((t + 1) & 1) wait_loads_and_sync<LD>();
      else wait_loads_and_sync<LD + 2>();
    } else {
      wait_loads_and_sync<0>();
    }
    if (t + NST - 1 < nk) issue_stage<F, NST, AUX_A>(L, lds, t + NST - 1);
    if ((t & 1) == 0) {
      const uint32_t* ep = (const uint32_t*)(lds + NST * STAGE_BYTES + ((t >> 1) % NEPOCH) * EPOCH_BYTES);
      static_for<F>([&]<int mi>() { sa[mi] = ep[32 * mi + i] >> (8 * h); });
      sb[0] = ep[TM + 64 * w + i] >> (8 * h);
      sb[1] = ep[TM + 64 * w + 32 + i] >> (8 * h);
    }
    if (active) compute_stage<F>(lds + (t % NST) * STAGE_BYTES, sa, sb, t & 1, acc);
  }
}

// Quantise 32 consecutive columns of one row held by the 32 lanes of a half-wave:
// returns this lane's code; *scale receives the block's e8m0 byte.
MOE_DEV uint32_t quant_lane32(float v, uint32_t* scale) {
  float amax = group_max32(fabsf(v));
  uint32_t byte = e8m0_from_amax(amax);
  *scale = byte;
  float x = clamp448(v * e8m0_inv_scale(byte));
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFFu;
}

// silu(g) = g * sigmoid(g) with the hardware reciprocal (1 ulp).
MOE_DEV float sigmoid(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
MOE_DEV float silu(float g) { return g * sigmoid(g); }

// Gate/up epilogue shared by the direct and the ring kernels.  For wave w the tile's B rows are
// 32 gate rows followed by the 32 matching up rows, so G and U of an element sit in the same
// lane; h = silu(G) U is quantised along I in 32-column blocks held by the 32 lanes of a
// half-wave.  n0: first I column of the tile (128 per tile).
template <int F>
MOE_DEV void gateup_epilogue(const v16f (&acc)[F][2], int r0, int rows, int n0, int I, float* g_out,
                             float* u_out, uint8_t* hq, uint8_t* hs) {
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int n = n0 + 32 * w + i;
  static_for<F>([&]<int mi>() {
    static_for<16>([&]<int v>() {
      const int r = 32 * mi + 8 * (v >> 2) + 4 * h + (v & 3);
      const float g = acc[mi][0][v], u = acc[mi][1][v];
      uint32_t sc;
      const uint32_t code = quant_lane32(silu(g) * u, &sc);
      if (r < rows) {
        const size_t o = (size_t)(r0 + r) * I + n;
        g_out[o] = g;
        u_out[o] = u;
        hq[o] = (uint8_t)code;
        if (i == 0) hs[(size_t)(r0 + r) * (I / 32) + (n >> 5)] = (uint8_t)sc;
      }
      if ((v & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the registers in flight
    });
  });
}

// B rows of a gate/up tile: staged row r of wave r / 64 is gate row n0 + 32(r / 64) + r % 32
// for r % 64 < 32, else the matching up row (I further on).
MOE_DEV int gateup_brow(int r, int n0, int I) {
  const int w = r >> 6, j = r & 63;
  return j < 32 ? n0 + 32 * w + j : I + n0 + 32 * w + (j - 32);
}

}  // namespace
}  // namespace moe
