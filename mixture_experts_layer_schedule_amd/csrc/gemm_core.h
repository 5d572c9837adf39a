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
// K pipeline: stages of 128 (two MFMA steps) in an NST-deep ring of LDS buffers, filled by
// direct-to-LDS loads (global_load_lds_dwordx4: no registers in between) while the previous
// stage is multiplied.  A load instruction moves 8 whole staged rows of 128 bytes, so every
// request is a full cache line.  Each staged row's eight 16-byte chunks are XOR-swizzled by the
// row index so that the fragment reads (lane i reads row i) hit distinct banks.  Scales travel
// the same way, one 4-byte word (4 K blocks) per row and stage.  One barrier per stage: it
// publishes the stage every wave loaded a share of and retires the buffer that the next loads
// overwrite.
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
constexpr int KS = 128;                      // K per pipeline stage (two MFMA steps)
constexpr int A_STAGE = TM * KS;             // bytes of one staged A slice
constexpr int DATA_BYTES = (TM + TN) * KS;   // A then B
constexpr int SCALE_BYTES = (TM + TN) * 4;   // one scale word (4 K blocks) per row
constexpr int STAGE_BYTES = DATA_BYTES + SCALE_BYTES;

constexpr size_t lds_bytes_for(int nst) { return (size_t)nst * STAGE_BYTES; }

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
// ceil(c / 256) tiles; the rows are split evenly between them in multiples of 32, so a 300-row
// expert runs as two 160-row tiles rather than 256 + 44.  rows <= 0 only for experts of more
// than 2048 rows, whose last tile can come out empty.  (A wider tile would need more than the
// 256 accumulator registers per lane.)
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

// A half of the loads of stage t (K range [128t, 128t + 128)) into buffer t % NST: one scale
// word and F data instructions per wave.  AUX_A: cache-policy bits of the A loads (16 = sc1:
// device-coherent reads of rows that other workgroups of the same kernel wrote).
template <int F, int NST, int AUX_A>
MOE_DEV void issue_a_stage(const TileLoads<F>& L, uint8_t* lds, int t) {
  const int w = threadIdx.x >> 6;
  const int k0 = t * KS;
  uint8_t* st = lds + (t % NST) * STAGE_BYTES;
  uint8_t* sc = st + DATA_BYTES;
  lds_load4<AUX_A>(L.asbase + (L.as + ((uint32_t)k0 >> 5)), sc + 256 * w);
  static_for<F>([&]<int u>() { lds_load16<AUX_A>(L.abase + (L.a[u] + (uint32_t)k0), st + 1024 * (w + 4 * u)); });
}

// Loads of stage t into buffer t % NST: 2 scale words, then F + 8 data instructions per wave.
template <int F, int NST, int AUX_A>
MOE_DEV void issue_stage(const TileLoads<F>& L, uint8_t* lds, int t) {
  const int w = threadIdx.x >> 6;
  const int k0 = t * KS;
  uint8_t* st = lds + (t % NST) * STAGE_BYTES;
  uint8_t* sc = st + DATA_BYTES;
  lds_load4<AUX_A>(L.asbase + (L.as + ((uint32_t)k0 >> 5)), sc + 256 * w);
  lds_load4<0>(L.bsbase + (L.bs + (uint32_t)t * L.bsk), sc + TM * 4 + 256 * w);
  static_for<F>([&]<int u>() { lds_load16<AUX_A>(L.abase + (L.a[u] + (uint32_t)k0), st + 1024 * (w + 4 * u)); });
  const uint32_t kb = (uint32_t)t * L.bk;
  static_for<8>([&]<int u>() { lds_load16<0>(L.bbase + (L.b[u] + kb), st + A_STAGE + 1024 * (w + 4 * u)); });
}

// Wait until at most N of this wave's loads are outstanding, then meet the other waves.  The
// wait and the barrier are one statement so that no LDS access moves across either.
template <int N>
MOE_DEV void wait_loads_and_sync() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// An empty statement that reads and rewrites two accumulator tiles in place: code after it
// cannot start before the matrix instructions that produce them have been issued.
MOE_DEV void pin_agprs(v16f& a, v16f& b) { asm volatile("" : "+a"(a), "+a"(b)::"memory"); }

// Multiply one staged K slice (two MFMA steps): acc[mi][ni] += A_frag(mi) * B_frag(ni).
// Staged row 32m + i (B: 64w + 32m + i) has swizzle swz(i) ^ 4(m & 1).  The A fragments are
// read two at a time, one pair ahead of the matrix instructions that use the previous pair
// (scheduling barriers keep that order): LDS returns in order, so each instruction waits only
// for its own operands while the next pair is arriving, and few registers hold fragments.
template <int F, class Hook>
MOE_DEV void compute_stage(const uint8_t* st, v16f (&acc)[F][2], const Hook& hook) {
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int sw = swz(i);
  const uint32_t* sc = (const uint32_t*)(st + DATA_BYTES);
  int sa[F], sb[2];
  static_for<F>([&]<int mi>() { sa[mi] = (int)(sc[32 * mi + i] >> (8 * h)); });
  sb[0] = (int)(sc[TM + 64 * w + i] >> (8 * h));
  sb[1] = (int)(sc[TM + 64 * w + 32 + i] >> (8 * h));
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
      // independent vector work placed here issues while the matrix core runs the group
      if constexpr (!Hook::kEmpty) {
        hook.template operator()<kk * NG + g, 2 * NG>();
        // interleave: one matrix instruction, then a share of the hook's vector work, so the
        // vector work issues while the matrix core runs
        constexpr int NM = 2 * ((2 * g + 1 < F) ? 2 : 1);
        static_for<NM>([&]<int x>() {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 28, 0);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

struct NoHook {
  static constexpr bool kEmpty = true;
  template <int G, int NGROUPS>
  MOE_DEV void operator()() const {}
};
template <int F>
MOE_DEV void compute_stage(const uint8_t* st, v16f (&acc)[F][2]) {
  compute_stage<F>(st, acc, NoHook{});
}

// acc = A_tile * B_tile^T over K = 128 * nk.  Every wave multiplies, also one whose columns lie
// past N (its B rows are clamped copies and its results are dropped): a branch around the
// matrix instructions would make the accumulators change register class every iteration.
template <int F, int NST, int AUX_A = 0>
MOE_DEV void mainloop(uint8_t* lds, const TileLoads<F>& L, int nk, v16f (&acc)[F][2]) {
  static_assert(NST == 2, "two LDS stages");
  static_for<F>([&]<int mi>() {
    acc[mi][0] = (v16f){};
    acc[mi][1] = (v16f){};
  });
  if (nk <= 0) return;
  issue_stage<F, NST, AUX_A>(L, lds, 0);
  for (int t = 0; t < nk; ++t) {
    wait_loads_and_sync<0>();  // stage t has landed; every wave is done with stage t - 1
    if (t + 1 < nk) issue_stage<F, NST, AUX_A>(L, lds, t + 1);
    compute_stage<F>(lds + (t % NST) * STAGE_BYTES, acc);
  }
}

// B operand of a dgrad GEMM built in the kernel from a forward weight ("transposed
// requantisation").  The forward weight Wq of one expert is a K x N code matrix quantised along
// its rows (blocks of 32 of the N values); the dgrad GEMM contracts over K, so its B tile (N
// rows, K contiguous, blocks along K) is W^T requantised: every 32 K values of a column are
// dequantised exactly (e4m3 code x 2^(e - 127) is a float32) and quantised again with the
// block's own e8m0 exponent, the arithmetic of the standalone requantisation kernel.  Doing it
// here reads the weight once per tile instead of writing and re-reading a transposed copy.
//
// Stage t covers K rows [128t, 128t + 128): wave w requantises K block w (32 rows) of the 256
// tile columns; lane l holds columns [16 (l % 16), +16) of rows 8 (l / 16) .. +8 of that block,
// loaded as eight 16-byte pieces (four lanes of a wave instruction share a row, so one
// instruction reads four whole 256-byte row segments) plus one scale byte per row.  The block
// maximum of a column spans the four lanes l, l ^ 16, l ^ 32, l ^ 48.  Each column's 8 new codes
// go to the staged B row as one 8-byte LDS write and its new scale byte to the stage's B scale
// word (byte w = K block w).
struct TransB {
  const uint8_t* q;  // [K][N] codes of the expert
  const uint8_t* s;  // [K][N / 32] scale bytes
  int N;
  uint32_t qoff, soff;  // this lane's first piece / scale byte (K row 32w + 8(l / 16), stage 0)
  v4i raw[8];           // the stage being requantised: 8 row pieces,
  float f[8];           // their dequantisation factors 2^(e - 127)
  v4i nraw[8];          // the next stage, in flight: pieces and scale bytes
  uint32_t nsraw[8];

  // n0: first column of the tile; columns past N (N a multiple of 128) repeat the last valid
  // 16 (their results are dropped).
  MOE_DEV void init(const uint8_t* q_, const uint8_t* s_, int N_, int n0) {
    q = q_; s = s_; N = N_;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int col = min(n0 + 16 * (l & 15), N - 16);
    const int row = 32 * w + 8 * (l >> 4);
    qoff = (uint32_t)row * (uint32_t)N + (uint32_t)col;
    soff = (uint32_t)row * (uint32_t)(N / 32) + (uint32_t)(col >> 5);
  }

  // 16 loads per lane into the in-flight set: 8 pieces, then 8 scale bytes.
  MOE_DEV void load_next(int t) {
    const uint32_t r0 = (uint32_t)(128 * t);
    static_for<8>([&]<int j>() { nraw[j] = *(const v4i*)(q + (qoff + (r0 + j) * (uint32_t)N)); });
    static_for<8>([&]<int j>() { nsraw[j] = s[soff + (r0 + j) * (uint32_t)(N / 32)]; });
  }

  // The in-flight stage becomes the one to requantise (waits for its loads).  (Two register
  // sets alternating by stage parity would save these copies, but the two-stage loop body that
  // needs makes the kernel spill.)
  MOE_DEV void advance() {
    static_for<8>([&]<int j>() {
      raw[j] = nraw[j];
      f[j] = e8m0_scale(nsraw[j]);
    });
  }

  // Requantise column pair P of this lane (word P / 2 of every piece, half P % 2: columns
  // 16 (l % 16) + 2P, + 1) into stage buffer st.
  template <int P>
  MOE_DEV void requant_pair(uint8_t* st) const {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int cg = l & 15, ng = l >> 4;
    float v[8][2];
    static_for<8>([&]<int j>() {
      const v2f x = __builtin_amdgcn_cvt_pk_f32_fp8(raw[j][P >> 1], (P & 1) != 0);
      v[j][0] = x[0] * f[j];
      v[j][1] = x[1] * f[j];
    });
    static_for<2>([&]<int c>() {
      float m = 0.0f;
      static_for<8>([&]<int j>() { m = fmaxf(m, fabsf(v[j][c])); });
      // maximum over the lanes l ^ 16, l ^ 32, l ^ 48 (the other 24 rows of the block); the
      // maxima are non-negative, so they are compared as integers (no canonicalisation)
      uint32_t mu = __float_as_uint(m);
      const auto p16 = __builtin_amdgcn_permlane16_swap((int)mu, (int)mu, false, false);
      mu = max((uint32_t)p16[0], (uint32_t)p16[1]);
      const auto p32 = __builtin_amdgcn_permlane32_swap((int)mu, (int)mu, false, false);
      mu = max((uint32_t)p32[0], (uint32_t)p32[1]);
      const uint32_t byte = e8m0_from_amax(__uint_as_float(mu));
      const float inv = e8m0_inv_scale(byte);
      v2i codes;
      codes[0] = (int)pack4_e4m3(v[0][c] * inv, v[1][c] * inv, v[2][c] * inv, v[3][c] * inv);
      codes[1] = (int)pack4_e4m3(v[4][c] * inv, v[5][c] * inv, v[6][c] * inv, v[7][c] * inv);
      const int r = 16 * cg + 2 * P + c;  // staged B row = tile column
      const int chunk = 2 * w + (ng >> 1);
      *(v2i*)(st + A_STAGE + r * KS + 16 * (chunk ^ swz(r)) + 8 * (ng & 1)) = codes;
      st[DATA_BYTES + TM * 4 + 4 * r + w] = (uint8_t)byte;  // the 4 lanes of a column write the same byte
    });
  }

  template <int P0, int P1>
  MOE_DEV void requant_pairs(uint8_t* st) const {
    static_for<P1 - P0>([&]<int p>() { requant_pair<P0 + p>(st); });
  }
};

// Spreads the requantisation of the next stage (8 column pairs per lane) over the matrix
// groups of compute_stage, so that its vector work issues while the matrix core is busy.  No
// branch: a branch between the groups would let the compiler gather every fragment read ahead
// of the matrix instructions.
struct RequantHook {
  static constexpr bool kEmpty = false;
  const TransB& tb;
  uint8_t* st;
  template <int G, int NGROUPS>
  MOE_DEV void operator()() const {
    tb.requant_pairs<8 * G / NGROUPS, 8 * (G + 1) / NGROUPS>(st);
  }
};

// mainloop with the B tile requantised in the kernel from a forward weight (TransB).  Stage t:
// after the barrier the raw B of stage t + 2 and the A of stage t + 1 are loaded, and stage t
// is multiplied while the raw B of stage t + 1 (loaded during stage t - 1) is requantised into
// the other buffer between the matrix groups.  One barrier per stage, as in mainloop.
template <int F>
MOE_DEV void mainloop_tb(uint8_t* lds, const TileLoads<F>& L, TransB& tb, int nk, v16f (&acc)[F][2]) {
  static_for<F>([&]<int mi>() {
    acc[mi][0] = (v16f){};
    acc[mi][1] = (v16f){};
  });
  if (nk <= 0) return;
  tb.load_next(0);
  issue_a_stage<F, 2, 0>(L, lds, 0);
  tb.advance();
  tb.requant_pairs<0, 8>(lds);
  if (nk > 1) {
    tb.load_next(1);
    tb.advance();
  }
  for (int t = 0; t < nk; ++t) {
    // A of stage t has landed; every wave wrote its share of stage t's B and is done with t - 1
    wait_loads_and_sync<0>();
    if (t + 2 < nk) tb.load_next(t + 2);
    if (t + 1 < nk) issue_a_stage<F, 2, 0>(L, lds, t + 1);
    // (in the last stage this requantises stale registers into the B region of the free buffer,
    // which nothing reads afterwards: cheaper than a branch)
    compute_stage<F>(lds + (t % 2) * STAGE_BYTES, acc, RequantHook{tb, lds + ((t + 1) % 2) * STAGE_BYTES});
    // unconditional (past the last load it copies stale registers that nothing uses): a branch
    // after the matrix instructions would let the compiler sink them below the vector work
    tb.advance();
  }
}

// ---------------------------------------------------------------------------------------------
// Two waves per SIMD (the forward and weight-gradient GEMMs).  A workgroup with one wave per
// SIMD keeps one stage (64 KB) of loads in flight and a wave's loads return at a bounded rate,
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

// Loads of stage t into buffer t % 2: one scale word and this wave's share of the data.
template <int F>
MOE_DEV void issue_stage8(const TileLoads8<F>& L, uint8_t* lds, int t) {
  const int w = threadIdx.x >> 6;
  const uint32_t k0 = (uint32_t)t * KS;
  uint8_t* st = lds + (t % 2) * STAGE_BYTES;
  uint8_t* scp = st + DATA_BYTES;
  if (w < 4)
    lds_load4<0>(L.asbase + (L.sc + (k0 >> 5)), scp + 256 * w);
  else
    lds_load4<0>(L.bsbase + (L.sc + (k0 >> 5)), scp + TM * 4 + 256 * (w - 4));
  static_for<TileLoads8<F>::NA>([&]<int u>() {
    const int q = w + 8 * u;
    if (q < 4 * F) lds_load16<0>(L.abase + (L.a[u] + k0), st + 1024 * q);
  });
  static_for<4>([&]<int u>() { lds_load16<0>(L.bbase + (L.b[u] + k0), st + A_STAGE + 1024 * (w + 8 * u)); });
}

// Multiply one staged K slice (two MFMA steps) for this wave's FH row fragments and two column
// fragments; A fragments read two at a time ahead of the matrix instructions.
template <int F>
MOE_DEV void compute_stage8(const uint8_t* st, v16f (&acc)[(F + 1) / 2][2]) {
  constexpr int FH = (F + 1) / 2;
  const int l = lane_id(), i = l & 31, h = l >> 5, w = threadIdx.x >> 6;
  const int wc = w & 3, m0 = (w >> 2) * FH;
  const int sw = swz(i);
  const uint32_t* sc = (const uint32_t*)(st + DATA_BYTES);
  int sa[FH], sb[2];
  static_for<FH>([&]<int m>() { sa[m] = (int)(sc[32 * (m0 + m) + i] >> (8 * h)); });
  sb[0] = (int)(sc[TM + 64 * wc + i] >> (8 * h));
  sb[1] = (int)(sc[TM + 64 * wc + 32 + i] >> (8 * h));
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

// acc = this wave's part of A_tile * B_tile^T over K = 128 nk; one barrier per stage.
template <int F>
MOE_DEV void mainloop8(uint8_t* lds, const TileLoads8<F>& L, int nk, v16f (&acc)[(F + 1) / 2][2]) {
  static_for<(F + 1) / 2>([&]<int m>() {
    acc[m][0] = (v16f){};
    acc[m][1] = (v16f){};
  });
  if (nk <= 0) return;
  issue_stage8<F>(L, lds, 0);
  for (int t = 0; t < nk; ++t) {
    wait_loads_and_sync<0>();  // stage t has landed; every wave is done with stage t - 1
    if (t + 1 < nk) issue_stage8<F>(L, lds, t + 1);
    compute_stage8<F>(lds + (t % 2) * STAGE_BYTES, acc);
  }
}

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

// B rows of a gate/up tile: staged row r of wave r / 64 is gate row n0 + 32(r / 64) + r % 32
// for r % 64 < 32, else the matching up row (I further on).
MOE_DEV int gateup_brow(int r, int n0, int I) {
  const int w = r >> 6, j = r & 63;
  return j < 32 ? n0 + 32 * w + j : I + n0 + 32 * w + (j - 32);
}

}  // namespace
}  // namespace moe
