// Core of the grouped MXFP8 GEMMs (shared by the expert GEMM kernels, which also run the ring
// dispatch rounds, and the persistent ring kernel, which is not launched).
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
// K pipeline: stages of 128 (two MFMA steps) in an NST-deep ring of LDS buffers, filled by
// direct-to-LDS loads (global_load_lds_dwordx4: no registers in between) while the previous
// stage is multiplied.  A load instruction moves 8 whole staged rows of 128 bytes, so every
// request is a full cache line.  Each staged row's eight 16-byte chunks are XOR-swizzled by the
// row index so that the fragment reads (lane i reads row i) hit distinct banks.  One barrier per
// stage: it publishes the stage every wave loaded a share of and retires the buffer that the
// next loads overwrite.
//
// Scales: a stage needs one 4-byte word (4 K blocks) per row, and every operand row's scales
// lie in a cache line of their own, so loading them stage by stage costs one request per row and
// stage: as many line requests as the stage's data.  They travel instead in groups of four
// stages (16 bytes per row, fetched as 4 words by 4 lanes), a quarter of the requests, into two
// group buffers behind the stage buffers (scale_group below).  Weight scales that are already
// stored stage-major (the transposed weights of the dgrad GEMMs) keep the per-stage word loads:
// a stage's words are contiguous there.
//
// Each output tile is owned by exactly one workgroup and K is summed in a fixed order, so
// results are bitwise reproducible.
#pragma once
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int TM = 256;                      // rows of a full tile (8 fragments of 32)
constexpr int TN = 256;                      // columns of a tile (4 waves x 64)
constexpr int KS = 128;                      // K per pipeline stage (two MFMA steps)
constexpr int A_STAGE = TM * KS;             // bytes of one staged A slice
constexpr int DATA_BYTES = (TM + TN) * KS;   // A then B
constexpr int SCALE_BYTES = (TM + TN) * 4;   // one scale word (4 K blocks) per row
constexpr int STAGE_BYTES = DATA_BYTES + SCALE_BYTES;

constexpr size_t lds_bytes_for(int nst) { return (size_t)nst * STAGE_BYTES; }

// Scale groups.  Group g holds the words of stages 4g .. 4g + 3 for the tile's A rows (group rows
// 0 .. 255) and B rows (256 .. 511), 16 bytes per row, in buffer g % 2 behind the two stage
// buffers.  Group g travels with the data of stage 4g; the buffer's previous group was last read
// four barriers earlier.  Word c of row r sits at 16 r + 4 (c ^ ((r >> 3) & 3)): 32 consecutive
// rows reading one word hit 32 distinct banks.
constexpr int SG_ROW = 16;
constexpr int SG_BYTES = (TM + TN) * SG_ROW;
constexpr int SG_BASE = 2 * STAGE_BYTES;
// byte offsets (from the operand's scale base) of the tile's 512 group rows' scales, written once
// per tile: the group loads read them from here rather than holding them in registers
constexpr int SGT_BASE = SG_BASE + 2 * SG_BYTES;
constexpr size_t GEMM_LDS_BYTES = (size_t)SGT_BASE + (TM + TN) * 4;

MOE_DEV const uint8_t* sg_buf(const uint8_t* lds, int t) { return lds + SG_BASE + ((t >> 2) & 1) * SG_BYTES; }
MOE_DEV uint8_t* sg_buf(uint8_t* lds, int t) { return lds + SG_BASE + ((t >> 2) & 1) * SG_BYTES; }
// byte of stage t's word of group row r (r a multiple of 32 plus lane i < 32 in the readers)
MOE_DEV int sg_pos(int r, int t) { return SG_ROW * r + 4 * ((t & 3) ^ ((r >> 3) & 3)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Physical 16-byte chunk slot of logical chunk g in staged row r is g ^ swz(r).  Rows with
// equal r % 2 among any 16 consecutive rows, and any 8 consecutive rows, get distinct slots, so
// the fragment reads are conflict-free whether the LDS serves 16 or 8 lanes per cycle.
MOE_DEV int swz(int r) { return (r ^ (r >> 3)) & 7; }

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
// ceil(c / tile rows) tiles (tile rows: the configured chunk, 256 by default); the rows are split
// evenly between them in multiples of 32, so a 300-row expert runs as two 160-row tiles rather
// than 256 + 44.  The rounding to 32 could in principle leave the last tile empty (rows <= 0;
// no expert below 70,000 rows does, for any tile height up to 256), and every kernel skips such a
// tile.  (A wider tile would need more than the 256 accumulator registers per lane.)
struct RowTile {
  int e, r0, rows;
  int m, nm;  // index of the tile among the expert's nm row tiles
};
MOE_DEV RowTile row_tile(const SchedView& s, int tile) {
  RowTile t;
  t.e = tile_expert(s.tile_start, s.n_exp, tile);
  t.m = tile - s.tile_start[t.e];
  t.nm = s.tile_start[t.e + 1] - s.tile_start[t.e];
  const int c = s.offsets[t.e + 1] - s.offsets[t.e];
  const int per = ((c + t.nm - 1) / t.nm + 31) & ~31;
  t.r0 = s.offsets[t.e] + t.m * per;
  t.rows = min(per, c - t.m * per);
  return t;
}

// Item `item` of a routed grouped GEMM with NT column tiles.  The items of one expert are
// ordered column tile major, row tile minor, so the row tiles that share a weight slice are
// neighbours (their weight reads meet in L2) and a row tile's column tiles lie within 2 x NT
// consecutive items (their A reads meet in L2 too).  Returns the row tile and the column tile.
MOE_DEV RowTile item_tile(const SchedView& s, int item, int NT, int* n) {
  const int e = tile_expert(s.tile_start, s.n_exp, item / NT);
  const int nm = s.tile_start[e + 1] - s.tile_start[e];
  const int j = item - s.tile_start[e] * NT;
  *n = j / nm;
  return row_tile(s, s.tile_start[e] + j % nm);
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

// Per-thread source addresses of the direct-to-LDS loads of one tile, as 32-bit byte offsets
// from wave-uniform bases (the loads then take a scalar base and one offset register each).
// Staged rows are filled 8 per wave instruction: instruction q (wave q % 4) covers rows
// [8q, 8q + 8), lane l the row 8q + l / 8, chunk slot l % 8.  a_rows(r) / b_rows(r) return the
// K data of staged row r (callers clamp rows past the operand to a valid one; such rows are
// never stored) and a_srows / b_srows its scale bytes; every operand lies within 4 GiB of its
// base.
template <int F>
struct TileLoads {
  const uint8_t *abase, *bbase, *asbase, *bsbase;
  uint32_t a[F];   // A: 4F instructions per stage, F per wave
  uint32_t b[8];   // B: 32 instructions per stage, 8 per wave
  uint32_t as, bs;       // scale words of rows 64w + l
  uint32_t bk = KS, bsk = KS / 32;  // bytes between the B data / scale words of successive stages

  template <class ARow, class BRow, class ASRow, class BSRow>
  MOE_DEV void init(const uint8_t* ab, ARow a_rows, const uint8_t* bb, BRow b_rows, const uint8_t* asb,
                    ASRow a_srows, const uint8_t* bsb, BSRow b_srows) {
    abase = ab; bbase = bb; asbase = asb; bsbase = bsb;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int sub = l >> 3, slot = l & 7;
    static_for<F>([&]<int u>() {
      const int r = 8 * (w + 4 * u) + sub;
      a[u] = (uint32_t)(a_rows(r) - ab) + 16 * (slot ^ swz(r));
    });
    static_for<8>([&]<int u>() {
      const int r = 8 * (w + 4 * u) + sub;
      b[u] = (uint32_t)(b_rows(r) - bb) + 16 * (slot ^ swz(r));
    });
    as = (uint32_t)(a_srows(64 * w + l) - asb);
    bs = (uint32_t)(b_srows(64 * w + l) - bsb);
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

// Scale group of stage t (t % 4 == 0) for 64 group rows [64q, 64q + 64) of one operand: tbl
// holds the rows' scale offsets from base (the table entry of row 64q); dst = group buffer +
// 1024 q.  Instruction u fetches rows 64q + 16u .. + 16, lane l word (l % 4) ^ swizzle of row
// 16u + l / 4 (the lane's LDS word is 4l after 256u); words past the operand's last stage nk - 1
// repeat that stage's (never read).
MOE_DEV uint32_t* sg_table(uint8_t* lds) { return (uint32_t*)(lds + SGT_BASE); }

template <int AUX>
MOE_DEV void scale_group(const uint8_t* base, uint8_t* lds, int q, int dst_off, int t, int nk) {
  int l = lane_id();
  // opaque per call: the lane's rows and swizzled words would otherwise be hoisted out of the K
  // loop and held in registers across the matrix work
  asm volatile("" : "+v"(l));
  const uint32_t* tbl = sg_table(lds) + 64 * q;
  uint8_t* dst = sg_buf(lds, t) + dst_off;
  static_for<4>([&]<int u>() {
    const int rl = 16 * u + (l >> 2);
    const int c = (l & 3) ^ ((rl >> 3) & 3);
    lds_load4<AUX>(base + (tbl[rl] + 4u * (uint32_t)min(t + c, nk - 1)), dst + 256 * u);
  });
}

// Loads of stage t into buffer t % NST: the scale groups every fourth stage, then F + 8 data
// instructions per wave.  AUX_A: cache-policy bits of the A loads (16 = sc1: device-coherent
// reads of rows that other workgroups of the same kernel wrote).
// kGB: B scales in groups (row-major scales); else one word per row and stage, stage t's words
// at t * L.bsk from the row's (stage-major scales).
template <int F, int NST, int AUX_A, bool kGB>
MOE_DEV void issue_stage(const TileLoads<F>& L, uint8_t* lds, int t, int nk) {
  const int w = threadIdx.x >> 6;
  const int k0 = t * KS;
  uint8_t* st = lds + (t % NST) * STAGE_BYTES;
  uint8_t* sc = st + DATA_BYTES;
  if ((t & 3) == 0) {
    const int wu = __builtin_amdgcn_readfirstlane(w);
    scale_group<AUX_A>(L.asbase, lds, wu, 1024 * wu, t, nk);
    if constexpr (kGB) scale_group<0>(L.bsbase, lds, 4 + wu, TM * SG_ROW + 1024 * wu, t, nk);
  }
  if constexpr (!kGB) lds_load4<0>(L.bsbase + (L.bs + (uint32_t)t * L.bsk), sc + TM * 4 + 256 * w);
  static_for<F>([&]<int u>() { lds_load16<AUX_A>(L.abase + (L.a[u] + (uint32_t)k0), st + 1024 * (w + 4 * u)); });
  const uint32_t kb = (uint32_t)t * L.bk;
  static_for<8>([&]<int u>() { lds_load16<0>(L.bbase + (L.b[u] + kb), st + A_STAGE + 1024 * (w + 4 * u)); });
}

// Wait until at most N of this wave's memory operations are outstanding (and its LDS reads have
// returned), then meet the other waves.  The wait and the barrier are one statement so that no
// LDS access moves across either.
template <int N>
MOE_DEV void wait_loads_and_sync() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// An empty statement that reads and rewrites two accumulator tiles in place: code after it
// cannot start before the matrix instructions that produce them have been issued.
MOE_DEV void pin_agprs(v16f& a, v16f& b) { asm volatile("" : "+a"(a), "+a"(b)::"memory"); }

// Multiply one staged K slice (two MFMA steps): acc[mi][ni] += A_frag(mi) * B_frag(ni).
// Staged row 32m + i (B: 64w + 32m + i) has swizzle swz(i) ^ 4(m & 1).  The A fragments are
// read two at a time, one pair ahead of the matrix instructions that use the previous pair
// (scheduling barriers keep that order): LDS returns in order, so each instruction waits only
// for its own operands while the next pair is arriving, and few registers hold fragments.
template <int F, bool kGB>
MOE_DEV void compute_stage(const uint8_t* st, const uint8_t* sg, int t, v16f (&acc)[F][2]) {
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int sw = swz(i);
  int sa[F], sb[2];
  static_for<F>([&]<int mi>() { sa[mi] = (int)(*(const uint32_t*)(sg + sg_pos(32 * mi + i, t)) >> (8 * h)); });
  if constexpr (kGB) {
    sb[0] = (int)(*(const uint32_t*)(sg + sg_pos(TM + 64 * w + i, t)) >> (8 * h));
    sb[1] = (int)(*(const uint32_t*)(sg + sg_pos(TM + 64 * w + 32 + i, t)) >> (8 * h));
  } else {
    const uint32_t* sc = (const uint32_t*)(st + DATA_BYTES);
    sb[0] = (int)(sc[TM + 64 * w + i] >> (8 * h));
    sb[1] = (int)(sc[TM + 64 * w + 32 + i] >> (8 * h));
  }
  constexpr int NG = (F + 1) / 2;
  static_for<2>([&]<int kk>() {
    auto frag = [&](const uint8_t* rp, int s2) {
      const v4i lo = *(const v4i*)(rp + 16 * ((4 * kk + h) ^ s2));
      const v4i hi = *(const v4i*)(rp + 16 * ((4 * kk + 2 + h) ^ s2));
      return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    const v8i b0 = frag(st + A_STAGE + (64 * w + i) * KS, sw);
    const v8i b1 = frag(st + A_STAGE + (64 * w + 32 + i) * KS, sw ^ 4);
    v8i pair[NG + 1][2];
    static_for<2>([&]<int j>() {
      if constexpr (j < F) pair[0][j] = frag(st + (32 * j + i) * KS, sw ^ (4 * (j & 1)));
    });
    static_for<NG>([&]<int g>() {
      static_for<2>([&]<int j>() {
        constexpr int mi = 2 * (g + 1) + j;
        if constexpr (mi < F) pair[g + 1][j] = frag(st + (32 * mi + i) * KS, sw ^ (4 * (mi & 1)));
      });
      __builtin_amdgcn_sched_barrier(0);
      static_for<2>([&]<int j>() {
        constexpr int mi = 2 * g + j;
        if constexpr (mi < F) {
          const int s_a = sa[mi] >> (16 * kk);
          acc[mi][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pair[g][j], b0, acc[mi][0], 0, 0, 0, s_a, 0,
                                                                        sb[0] >> (16 * kk));
          acc[mi][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pair[g][j], b1, acc[mi][1], 0, 0, 0, s_a, 0,
                                                                        sb[1] >> (16 * kk));
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// acc = A_tile * B_tile^T over K = 128 * nk.  Every wave multiplies, also one whose columns lie
// past N (its B rows are clamped copies and its results are dropped): a branch around the
// matrix instructions would make the accumulators change register class every iteration.
template <int F, int NST, int AUX_A = 0, bool kGB = true>
MOE_DEV void mainloop(uint8_t* lds, const TileLoads<F>& L, int nk, v16f (&acc)[F][2]) {
  static_assert(NST == 2, "two LDS stages");
  static_for<F>([&]<int mi>() {
    acc[mi][0] = (v16f){};
    acc[mi][1] = (v16f){};
  });
  if (nk <= 0) return;
  // this wave's rows' scale offsets (read back by the same wave only: no barrier needed)
  sg_table(lds)[threadIdx.x] = L.as;
  if constexpr (kGB) sg_table(lds)[TM + threadIdx.x] = L.bs;
  issue_stage<F, NST, AUX_A, kGB>(L, lds, 0, nk);
  for (int t = 0; t < nk; ++t) {
    wait_loads_and_sync<0>();  // stage t has landed; every wave is done with stage t - 1
    if (t + 1 < nk) issue_stage<F, NST, AUX_A, kGB>(L, lds, t + 1, nk);
    compute_stage<F, kGB>(lds + (t % NST) * STAGE_BYTES, sg_buf(lds, t), t, acc);
  }
}

// ---------------------------------------------------------------------------------------------
// Two waves per SIMD (every expert GEMM; the one-wave-per-SIMD loop above serves the ring
// kernel).  A workgroup with one wave per SIMD keeps one stage (64 KB) of loads in flight and a
// wave's loads return at a bounded rate,
// so the loop above spends most of each stage waiting for its loads (measured: about 1.5 us per
// 64 KB per workgroup even from L2, while two workgroups per compute unit move twice as much).
// Here 512 threads (8 waves, two per SIMD) share the same 256 x 256 tile and its loads: wave w
// owns the column group wc = w % 4 (columns [64 wc, 64 wc + 64) as two fragments, as in the
// 4-wave tile) and the row half wr = w / 4 (row fragments [wr FH, wr FH + FH), FH = ceil(F / 2)),
// so each wave holds FH x 2 accumulator tiles (at most 128 registers).  With an odd F the last
// fragment of the upper half lies past the tile: it multiplies stale LDS rows and its results
// are dropped.  Loads: the 4F A and 32 B instructions of a stage are dealt to the 8 waves in
// turn; waves 0-3 load the A scale words, waves 4-7 the B ones.  The stage layout is the 4-wave
// core's.

template <int F>
struct TileLoads8 {
  static constexpr int NA = (4 * F + 7) / 8;  // A instructions per wave (q = w + 8u < 4F)
  const uint8_t *abase, *bbase, *asbase, *bsbase;
  uint32_t a[NA];
  uint32_t b[4];
  uint32_t sc;  // A scale word of row 64w + l (w < 4) or B scale word of row 64(w - 4) + l
  uint32_t bsk = 0;  // stage-major B scales (kGB false): bytes between the planes of successive stages

  template <class ARow, class BRow, class ASRow, class BSRow>
  MOE_DEV void init(const uint8_t* ab, ARow a_rows, const uint8_t* bb, BRow b_rows, const uint8_t* asb,
                    ASRow a_srows, const uint8_t* bsb, BSRow b_srows) {
    abase = ab; bbase = bb; asbase = asb; bsbase = bsb;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int sub = l >> 3, slot = l & 7;
    static_for<NA>([&]<int u>() {
      const int r = 8 * min(w + 8 * u, 4 * F - 1) + sub;
      a[u] = (uint32_t)(a_rows(r) - ab) + 16 * (slot ^ swz(r));
    });
    static_for<4>([&]<int u>() {
      const int r = 8 * (w + 8 * u) + sub;
      b[u] = (uint32_t)(b_rows(r) - bb) + 16 * (slot ^ swz(r));
    });
    sc = w < 4 ? (uint32_t)(a_srows(64 * w + l) - asb) : (uint32_t)(b_srows(64 * (w - 4) + l) - bsb);
  }
};

// Loads of stage t into buffer t % 2: the scales and this wave's share of the data.  kGB: B
// scales in groups like A's; else (stage-major B scales, a stage's words contiguous) waves 4-7
// load stage t's word of B rows 64(w - 4) .. every stage.
template <int F, bool kGB = true>
MOE_DEV void issue_stage8(const TileLoads8<F>& L, uint8_t* lds, int t, int nk) {
  const int w = threadIdx.x >> 6;
  const uint32_t k0 = (uint32_t)t * KS;
  uint8_t* st = lds + (t % 2) * STAGE_BYTES;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // scale group: waves 0-3 the A rows 64w .., waves 4-7 the B rows 64(w - 4) .. (group rows 64w ..)
  if (kGB || wu < 4) {
    if ((t & 3) == 0) scale_group<0>(wu < 4 ? L.asbase : L.bsbase, lds, wu, 1024 * wu, t, nk);
  } else {
    lds_load4<0>(L.bsbase + (L.sc + (uint32_t)t * L.bsk), st + DATA_BYTES + TM * 4 + 256 * (wu - 4));
  }
  static_for<TileLoads8<F>::NA>([&]<int u>() {
    const int q = w + 8 * u;
    if (q < 4 * F) lds_load16<0>(L.abase + (L.a[u] + k0), st + 1024 * q);
  });
  static_for<4>([&]<int u>() { lds_load16<0>(L.bbase + (L.b[u] + k0), st + A_STAGE + 1024 * (w + 8 * u)); });
}

// Multiply one staged K slice (two MFMA steps) for this wave's FH row fragments and two column
// fragments; A fragments read two at a time ahead of the matrix instructions.
template <int F, bool kGB = true>
MOE_DEV void compute_stage8(const uint8_t* st, const uint8_t* sg, int t, v16f (&acc)[(F + 1) / 2][2]) {
  constexpr int FH = (F + 1) / 2;
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int wc = w & 3, m0 = (w >> 2) * FH;
  const int sw = swz(i);
  int sa[FH], sb[2];
  static_for<FH>([&]<int m>() { sa[m] = (int)(*(const uint32_t*)(sg + sg_pos(32 * (m0 + m) + i, t)) >> (8 * h)); });
  if constexpr (kGB) {
    sb[0] = (int)(*(const uint32_t*)(sg + sg_pos(TM + 64 * wc + i, t)) >> (8 * h));
    sb[1] = (int)(*(const uint32_t*)(sg + sg_pos(TM + 64 * wc + 32 + i, t)) >> (8 * h));
  } else {
    const uint32_t* sc = (const uint32_t*)(st + DATA_BYTES);
    sb[0] = (int)(sc[TM + 64 * wc + i] >> (8 * h));
    sb[1] = (int)(sc[TM + 64 * wc + 32 + i] >> (8 * h));
  }
  constexpr int NG = (FH + 1) / 2;
  static_for<2>([&]<int kk>() {
    auto frag = [&](const uint8_t* rp, int s2) {
      const v4i lo = *(const v4i*)(rp + 16 * ((4 * kk + h) ^ s2));
      const v4i hi = *(const v4i*)(rp + 16 * ((4 * kk + 2 + h) ^ s2));
      return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto afrag = [&](int m) { return frag(st + (32 * (m0 + m) + i) * KS, sw ^ (4 * ((m0 + m) & 1))); };
    const v8i b0 = frag(st + A_STAGE + (64 * wc + i) * KS, sw);
    const v8i b1 = frag(st + A_STAGE + (64 * wc + 32 + i) * KS, sw ^ 4);
    v8i pair[NG + 1][2];
    static_for<2>([&]<int j>() {
      if constexpr (j < FH) pair[0][j] = afrag(j);
    });
    static_for<NG>([&]<int g>() {
      static_for<2>([&]<int j>() {
        constexpr int m = 2 * (g + 1) + j;
        if constexpr (m < FH) pair[g + 1][j] = afrag(m);
      });
      __builtin_amdgcn_sched_barrier(0);
      static_for<2>([&]<int j>() {
        constexpr int m = 2 * g + j;
        if constexpr (m < FH) {
          const int s_a = sa[m] >> (16 * kk);
          acc[m][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pair[g][j], b0, acc[m][0], 0, 0, 0, s_a, 0,
                                                                       sb[0] >> (16 * kk));
          acc[m][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pair[g][j], b1, acc[m][1], 0, 0, 0, s_a, 0,
                                                                       sb[1] >> (16 * kk));
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// An empty statement that reads and rewrites the accumulators in place: code after it cannot
// start before the matrix instructions that produce them have been issued.
MOE_DEV void pin_vgprs(v16f& a, v16f& b) { asm volatile("" : "+v"(a), "+v"(b)::"memory"); }
template <int FH>
MOE_DEV void pin_acc(v16f (&acc)[FH][2]) {
  static_for<FH>([&]<int m>() { pin_vgprs(acc[m][0], acc[m][1]); });
}

struct NoSideWork {
  static constexpr bool kEnabled = false;
  MOE_DEV bool wants(int) const { return false; }
  MOE_DEV void run(const uint8_t*, const uint8_t*, int) {}
};

// acc = this wave's part of A_tile * B_tile^T over K = 128 nk; one barrier per stage.
//
// Optional side work on the streamed stages (the transposed weight requantisation): once stage
// t has landed and the loads of stage t + 1 are issued, the wave does the side work on stage t
// (side.run, when side.wants(t)) and then multiplies stage t.  Its stores thus follow the loads
// of stage t + 1 in issue order and retire while the matrix work runs, so the wait at the top of
// the next iteration (a wave's memory counter retires in issue order) is not lengthened by them.
template <int F, bool kGB = true, class Side = NoSideWork>
MOE_DEV void mainloop8(uint8_t* lds, const TileLoads8<F>& L, int nk, v16f (&acc)[(F + 1) / 2][2],
                       Side&& side = Side{}) {
  static_for<(F + 1) / 2>([&]<int m>() {
    acc[m][0] = (v16f){};
    acc[m][1] = (v16f){};
  });
  if (nk <= 0) return;
  // group row 64w + l's scale offset (read back by the same wave only: no barrier needed)
  sg_table(lds)[threadIdx.x] = L.sc;
  issue_stage8<F, kGB>(L, lds, 0, nk);
  for (int t = 0; t < nk; ++t) {
    wait_loads_and_sync<0>();  // stage t has landed; every wave is done with stage t - 1
    if (t + 1 < nk) issue_stage8<F, kGB>(L, lds, t + 1, nk);
    if constexpr (std::remove_reference_t<Side>::kEnabled) {
      // the previous stage's matrix instructions are issued before the side work (a branch
      // could otherwise let the compiler sink them past it)
      pin_acc<(F + 1) / 2>(acc);
      if (side.wants(t)) side.run((const uint8_t*)(lds + (t % 2) * STAGE_BYTES), sg_buf(lds, t), t);
    }
    compute_stage8<F, kGB>(lds + (t % 2) * STAGE_BYTES, sg_buf(lds, t), t, acc);
  }
}

// ---------------------------------------------------------------------------------------------
// Transposed requantisation of a staged weight slice (512 threads).
//
// The backward pass contracts the expert weights over the other axis (dgrad of the down GEMM
// over d, of the gate/up GEMM over 2I), so it needs W^T quantised along that axis: every 32
// consecutive weight rows of one column are dequantised exactly (e4m3 code x 2^(e - 127) is a
// float32) and quantised again with their own e8m0 exponent.  The forward GEMMs stream every
// weight slice through LDS anyway; a stage's B part holds 256 weight rows x 128 K values, i.e.
// whole 32-row blocks of 128 columns, so the transposed codes are produced there and written
// to HBM once (no separate pass that reads the weights again).
//
// The tile's 256 weight rows form two halves of 128 rows that are contiguous in the transposed
// weight (gate rows n0 .. n0 + 128 and up rows I + n0 .. of W1; W2 rows n0 .. n0 + 128 and
// n0 + 128 .. n0 + 256).  Wave w takes half w / 4 and stage columns 32 (w % 4) .. + 32, in two
// passes of 16; lane l reads 8 rows 8 (l % 16) .. + 8 of the half at 4 columns 4 (l / 16) .. + 4
// of the pass (a 4-byte piece of each row) and the rows' scale bytes.  A 32-row block is held by
// the 4 lanes l ^ 1, l ^ 2, l ^ 3.  The hardware's scaled conversions decode a code pair times
// the row's scale and encode a value pair divided by the new scale (round to nearest even), so
// a value costs about four vector instructions.  Each column's 8 codes of a lane are one 8-byte
// store, and the 16 lanes that share a column write its 128 contiguous transposed bytes in one
// instruction: whole cache lines, written once.  The scales are stored word-major: transposed
// row k's blocks 4q .. 4q + 3 form word q of plane [q][k], which is the word a dgrad stage loads
// per row, and a wave's 16 columns of a pass write 64 contiguous bytes.

// e8m0 byte -> the float 2^(byte - 127) that the scaled conversions take (byte 0 is 2^-127:
// the instructions read the exponent field only).
MOE_DEV float e8m0_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// kGateUp: the staged rows of a gate/up tile alternate 32 gate and 32 up rows per wave; the
// down GEMM's are the weight rows in order.
template <bool kGateUp>
struct RequantT8 {
  static constexpr bool kEnabled = true;
  uint8_t* wt;   // [K][ldt] transposed codes of the expert (NULL: no requantisation)
  uint8_t* wts;  // [ldt / 128][K] words of 4 scale bytes (blocks 4q .. 4q + 3 of transposed row k)
  int ldt;       // transposed row length (the requantisation axis)
  int K;         // transposed rows (the forward GEMM's reduction axis)
  int obase;     // transposed-row index of row 0 of this wave's half, or -1 to skip the half
  int m, nm;     // stage t is requantised by the item with t % nm == m

  MOE_DEV bool wants(int t) const { return wt != nullptr && t % nm == m; }

  // staged row of row x (0 .. 127) of half hf
  static MOE_DEV int staged(int hf, int x) {
    return kGateUp ? 64 * (x >> 5) + 32 * hf + (x & 31) : 128 * hf + x;
  }

  // requantise staged stage t (K columns [128t, 128t + 128)) and store it
  MOE_DEV void run(const uint8_t* st, const uint8_t* sg, int t) {
    if (obase < 0) return;  // wave-uniform
    const int w = threadIdx.x >> 6, l = lane_id();
    const int hf = w >> 2, cq = w & 3, rg = l & 15, cgp = l >> 4;
    // the lane's 8 rows are staged rows r0 .. r0 + 8 (a multiple of 8: they share swz's high part)
    const int r0 = staged(hf, 8 * rg);
    float f[8];  // the rows' scales as conversion operands (one K block per wave: block cq)
    static_for<8>([&]<int j>() { f[j] = e8m0_operand(sg[sg_pos(TM + r0 + j, t) + cq]); });
    int ld = ldt;
    // opaque per call: keeps the compiler from hoisting the columns' addresses out of the GEMM's
    // K loop, where they would stay live (and spill) across the matrix work
    asm volatile("" : "+s"(ld));
    static_for<2>([&]<int pass>() {
      const int c16 = 32 * cq + 16 * pass + 4 * cgp;  // first stage column of the lane
      uint32_t raw[8];
      const uint8_t* rp = st + A_STAGE + r0 * KS + (c16 & 15);
      const int x = ((c16 >> 4) ^ (r0 >> 3)) & 7;  // chunk slot of row r0 + j is x ^ j (swz)
      static_for<8>([&]<int j>() { raw[j] = *(const uint32_t*)(rp + j * KS + 16 * (x ^ j)); });
      const size_t col0 = (size_t)(KS * t + c16);
      uint8_t* out = wt + col0 * ld + obase + 8 * rg;
      uint8_t* sout = wts + ((size_t)(obase >> 7) * K + col0) * 4 + (rg >> 2);
      // two column pairs: byte pair P of every row's piece
      static_for<2>([&]<int P>() {
        float v[8][2];
        static_for<8>([&]<int j>() {
          const v2f x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw[j], f[j], P != 0);
          v[j][0] = x[0];
          v[j][1] = x[1];
        });
        static_for<2>([&]<int c>() {
          float mx = fabsf(v[0][c]);
          static_for<7>([&]<int j>() { mx = fmaxf(mx, fabsf(v[j + 1][c])); });
          // non-negative floats order like their bit patterns: the lane maxima cross as integers
          uint32_t u = __float_as_uint(mx);
          u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, false));  // l ^ 1
          u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, false));  // l ^ 2
          const uint32_t byte = e8m0_from_amax(__uint_as_float(u));
          const float sc = e8m0_operand(byte);
          // the encode saturates values above 448 except one: exactly 480 (mantissa 1.875 in
          // the top binade, the block maximum in about one column in eight) comes out as the
          // NaN pattern 0x7F (measured on the device), so values are clamped to
          // +-448 x 2^(byte - 127)
          const float lim = 1.75f * __uint_as_float((byte + 8) << 23);
          typedef short v2s __attribute__((ext_vector_type(2)));
          v2i codes;
          static_for<2>([&]<int q>() {
            v2s wv = {0, 0};
            wv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(wv, __builtin_amdgcn_fmed3f(v[4 * q][c], -lim, lim),
                                                          __builtin_amdgcn_fmed3f(v[4 * q + 1][c], -lim, lim), sc,
                                                          false);
            wv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(wv, __builtin_amdgcn_fmed3f(v[4 * q + 2][c], -lim, lim),
                                                          __builtin_amdgcn_fmed3f(v[4 * q + 3][c], -lim, lim), sc,
                                                          true);
            codes[q] = __builtin_bit_cast(int, wv);
          });
          constexpr int col = 2 * P + c;
          // non-temporal: the forward pass never reads these back, so they stream past the
          // caches instead of evicting the weight slices and rows the neighbouring tiles reuse
          __builtin_nontemporal_store(codes, (v2i*)(out + (size_t)col * ld));
          // the 4 lanes of a block store its scale byte (the same value): the words of the 16
          // columns of a pass are contiguous, so the bytes of a line meet in L2 at once
          sout[4 * col] = (uint8_t)byte;
        });
        __builtin_amdgcn_sched_barrier(0);  // one pair's values live at a time
      });
    });
  }
};

// Quantise 32 consecutive columns of one row held by the 32 lanes of a half-wave:
// returns this lane's code; *scale receives the block's e8m0 byte.
MOE_DEV uint32_t quant_lane32(float v, uint32_t* scale) {
  float amax = group_max32(fabsf(v));
  uint32_t byte = e8m0_from_amax(amax);
  *scale = byte;
  float x = clamp448(v * e8m0_inv_scale(byte));
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, __float_as_int(x), false) & 0xFFu;
}

// silu(g) = g * sigmoid(g) with the hardware reciprocal (1 ulp).
MOE_DEV float sigmoid(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
MOE_DEV float silu(float g) { return g * sigmoid(g); }

// Gate/up epilogue (direct and persistent-ring gate/up kernels).  For wave w the tile's B rows are
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

// The gate/up epilogue for the 8-wave tile: this wave's FH row fragments (from m0) of the
// column group wc.
template <int F>
MOE_DEV void gateup_epilogue8(const v16f (&acc)[(F + 1) / 2][2], int r0, int rows, int n0, int I, float* g_out,
                              float* u_out, uint8_t* hq, uint8_t* hs) {
  constexpr int FH = (F + 1) / 2;
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int wc = w & 3, m0 = (w >> 2) * FH;
  const int n = n0 + 32 * wc + i;
  static_for<FH>([&]<int m>() {
    static_for<16>([&]<int v>() {
      const int r = 32 * (m0 + m) + 8 * (v >> 2) + 4 * h + (v & 3);
      const float g = acc[m][0][v], u = acc[m][1][v];
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

// G and U of the 8-wave gate/up tile stored without the activation (the unfused forward applies
// SwiGLU and the quantisation in a pass of its own).
template <int F>
MOE_DEV void gu_store8(const v16f (&acc)[(F + 1) / 2][2], int r0, int rows, int n0, int I, float* g_out,
                       float* u_out) {
  constexpr int FH = (F + 1) / 2;
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int wc = w & 3, m0 = (w >> 2) * FH;
  const int n = n0 + 32 * wc + i;
  static_for<FH>([&]<int m>() {
    static_for<16>([&]<int v>() {
      const int r = 32 * (m0 + m) + 8 * (v >> 2) + 4 * h + (v & 3);
      if (r < rows) {
        const size_t o = (size_t)(r0 + r) * I + n;
        g_out[o] = acc[m][0][v];
        u_out[o] = acc[m][1][v];
      }
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
