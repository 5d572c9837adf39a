// Grouped MXFP8 GEMMs of the expert FFN (forward, dgrad and wgrad) on gfx950; the tile core is
// in gemm_core.h.  The routed GEMMs run one (row tile, 256-column tile) item per workgroup; the
// row count of the item picks the instantiation with that many 32-row fragments.  Every GEMM runs
// the tile with 8 waves (two per SIMD, 512 threads).
//
// The forward GEMMs also produce the transposed, requantised weights the backward pass
// contracts with (W1 along 2I, W2 along d): each stage's staged weight slice is requantised
// along its rows by one of the row tiles that share it (stage t by row tile t % nm), so every
// weight element of an expert with rows is requantised exactly once per forward pass.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {

namespace {

// Calls body.template operator()<F>() with F = ceil(rows / 32) in [1, 8].
template <class Body>
MOE_DEV void dispatch_rows(int rows, Body&& body) {
  switch ((rows + 31) >> 5) {
    case 1: body.template operator()<1>(); break;
    case 2: body.template operator()<2>(); break;
    case 3: body.template operator()<3>(); break;
    case 4: body.template operator()<4>(); break;
    case 5: body.template operator()<5>(); break;
    case 6: body.template operator()<6>(); break;
    case 7: body.template operator()<7>(); break;
    default: body.template operator()<8>(); break;
  }
}

constexpr int kStages = 2;  // one K slice in flight while the other is multiplied

// Slot (t * (k + S) + j) of every row of a tile, computed once per row into LDS (buf: a stage
// buffer no wave reads any more) instead of once per lane and row in the epilogue.
MOE_DEV const int64_t* row_slot_table(const SchedView& s, const RowTile& rt, uint8_t* buf) {
  int64_t* tbl = (int64_t*)buf;
  if ((int)threadIdx.x < rt.rows) tbl[threadIdx.x] = row_slot(s, rt.r0 + threadIdx.x);
  __syncthreads();
  return tbl;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Forward gate/up: [G U] = X_e W1_e^T (pull dispatch: rows gathered from xq through the
// schedule), epilogue h = silu(G) U quantised along I.  A column tile is 128 I columns: for
// each wave 32 gate rows of W1 and the matching 32 up rows.

__global__ __launch_bounds__(512, 1) void k_gemm_gateup(GateUpArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int I = p.I, d = p.d, NT = I / 128;
  int item, nt;
  RowTile rt;
  const uint8_t *ra = nullptr, *ras = nullptr;  // ring dispatch: the chunk's slot
  if (p.ring) {
    // the round's chunks (those that exist), column tiles fastest
    const int nc = min(p.nchunks, s.tile_start[s.n_exp] - p.chunk0);
    if (nc <= 0 || !xcd_item(nc * NT, &item)) return;
    const int c = p.chunk0 + item / NT;
    nt = item - (item / NT) * NT;
    rt = row_tile(s, c);
    const size_t slot = (size_t)(c % p.nslots) * p.slot_rows;
    ra = p.ring + slot * d;
    ras = p.ring_s + slot * (d / 32);
  } else {
    if (!xcd_item(s.tile_start[s.n_exp] * NT, &item)) return;
    rt = item_tile(s, item, NT, &nt);
  }
  if (rt.rows <= 0) return;
  const int n0 = nt * 128;
  const uint8_t* w1 = p.w1q + (size_t)rt.e * 2 * I * d;
  const uint8_t* w1s = p.w1s + (size_t)rt.e * 2 * I * (d / 32);
  const int last = rt.rows - 1;
  // transposed weight W1t[e] [d][2I]: half 0 of the tile is gate rows n0 .. n0 + 128, half 1
  // the up rows I + n0 ..
  RequantT8<true> side;
  side.wt = p.w1t ? p.w1t + (size_t)rt.e * d * 2 * I : nullptr;
  side.wts = p.w1t ? p.w1ts + (size_t)rt.e * d * (2 * I / 32) : nullptr;
  side.ldt = 2 * I;
  side.K = d;
  side.obase = ((threadIdx.x >> 8) ? I : 0) + n0;
  side.m = rt.m;
  side.nm = rt.nm;
  // A row of staged row r: the token of permuted row r0 + r (pull dispatch), or with
  // `contiguous` that permuted row itself (rows already in expert order)
  const bool cont = p.contiguous != 0;
  auto arow = [&](int r) {
    const int rr = rt.r0 + min(r, last);
    return cont ? rr : row_token(s, rr);
  };
  dispatch_rows(rt.rows, [&]<int F>() {
    TileLoads8<F> L;
    if (ra) {  // ring dispatch: the rows sit in the chunk's slot in order
      L.init(ra, [&](int r) { return ra + (size_t)min(r, last) * d; },
             w1, [&](int r) { return w1 + (size_t)gateup_brow(r, n0, I) * d; },
             ras, [&](int r) { return ras + (size_t)min(r, last) * (d / 32); },
             w1s, [&](int r) { return w1s + (size_t)gateup_brow(r, n0, I) * (d / 32); });
    } else {
      L.init(p.xq, [&](int r) { return p.xq + (size_t)arow(r) * d; },
             w1, [&](int r) { return w1 + (size_t)gateup_brow(r, n0, I) * d; },
             p.xs, [&](int r) { return p.xs + (size_t)arow(r) * (d / 32); },
             w1s, [&](int r) { return w1s + (size_t)gateup_brow(r, n0, I) * (d / 32); });
    }
    v16f acc[(F + 1) / 2][2];
    mainloop8<F>(lds, L, d / KS, acc, side);
    if (p.hq)
      gateup_epilogue8<F>(acc, rt.r0, rt.rows, n0, I, p.g, p.u, p.hq, p.hs);
    else
      gu_store8<F>(acc, rt.r0, rt.rows, n0, I, p.g, p.u);
  });
}

// ---------------------------------------------------------------------------------------------
// Forward down: Y_r = H_r W2_e^T, pushed to its slot Yslot[t, j] (push combine).

__global__ __launch_bounds__(512, 1) void k_gemm_down(DownArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int I = p.I, d = p.d, NT = (d + TN - 1) / TN;
  int item;
  if (!xcd_item(s.tile_start[s.n_exp] * NT, &item)) return;
  int nt;
  const RowTile rt = item_tile(s, item, NT, &nt);
  if (rt.rows <= 0) return;
  const int n0 = nt * TN;
  const uint8_t* w2 = p.w2q + (size_t)rt.e * d * I;
  const uint8_t* w2s = p.w2s + (size_t)rt.e * d * (I / 32);
  const int last = rt.rows - 1;
  const int w = threadIdx.x >> 6, l = lane_id(), i = l & 31, h = l >> 5, wc = w & 3;
  const bool active = n0 + 64 * wc < d;
  // transposed weight W2t[e] [I][d]: half h of the tile is W2 rows n0 + 128h .. (none past d)
  RequantT8<false> side;
  side.wt = p.w2t ? p.w2t + (size_t)rt.e * I * d : nullptr;
  side.wts = p.w2t ? p.w2ts + (size_t)rt.e * I * (d / 32) : nullptr;
  side.ldt = d;
  side.K = I;
  side.obase = n0 + 128 * (w >> 2) < d ? n0 + 128 * (w >> 2) : -1;
  side.m = rt.m;
  side.nm = rt.nm;
  dispatch_rows(rt.rows, [&]<int F>() {
    constexpr int FH = (F + 1) / 2;
    const int m0 = (w >> 2) * FH;
    TileLoads8<F> L;
    const uint8_t* ha = p.hq + (size_t)rt.r0 * I;
    const uint8_t* hsa = p.hs + (size_t)rt.r0 * (I / 32);
    L.init(ha, [&](int r) { return ha + (size_t)min(r, last) * I; },
           w2, [&](int r) { return w2 + (size_t)min(n0 + r, d - 1) * I; },
           hsa, [&](int r) { return hsa + (size_t)min(r, last) * (I / 32); },
           w2s, [&](int r) { return w2s + (size_t)min(n0 + r, d - 1) * (I / 32); });
    v16f acc[FH][2];
    mainloop8<F>(lds, L, I / KS, acc, side);
    if (p.yrows) {  // the unfused forward: rows stay in expert order
      if (!active) return;
      static_for<FH>([&]<int m>() {
        static_for<16>([&]<int v>() {
          const int r = 32 * (m0 + m) + 8 * (v >> 2) + 4 * h + (v & 3);
          if (r < rt.rows) {
            float* dst = p.yrows + (size_t)(rt.r0 + r) * d + n0 + 64 * wc + i;
            dst[0] = acc[m][0][v];
            dst[32] = acc[m][1][v];
          }
        });
      });
      return;
    }
    const int64_t* slot = row_slot_table(s, rt, lds + ((I / KS) % kStages) * STAGE_BYTES);
    if (!active) return;
    static_for<FH>([&]<int m>() {
      static_for<16>([&]<int v>() {
        const int r = 32 * (m0 + m) + 8 * (v >> 2) + 4 * h + (v & 3);
        if (r < rt.rows) {
          float* dst = p.yslot + slot[r] * d + n0 + 64 * wc + i;
          dst[0] = acc[m][0][v];
          dst[32] = acc[m][1][v];
        }
      });
    });
  });
}

// ---------------------------------------------------------------------------------------------
// Backward dgrad of the down GEMM with the SwiGLU backward in the epilogue:
// dH = w * (dY_t W2t_e^T) (rows pulled from dYq: reverse-combine, straight from dYq or, with the
// ring dispatch, from the ring slots the producers filled), dG = dH U s (1 + G (1 - s)),
// dU = dH silu(G); [dG dU] quantised along 2I.

__global__ __launch_bounds__(512, 1) void k_gemm_dgrad_down(DgradDownArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int I = p.I, d = p.d, NT = (I + TN - 1) / TN;
  int item, nt;
  RowTile rt;
  const uint8_t *ra = nullptr, *ras = nullptr;  // ring dispatch: the chunk's slot
  if (p.ring) {
    // the round's chunks (those that exist), column tiles fastest
    const int nc = min(p.nchunks, s.tile_start[s.n_exp] - p.chunk0);
    if (nc <= 0 || !xcd_item(nc * NT, &item)) return;
    const int c = p.chunk0 + item / NT;
    nt = item - (item / NT) * NT;
    rt = row_tile(s, c);
    const size_t slot = (size_t)(c % p.nslots) * p.slot_rows;
    ra = p.ring + slot * d;
    ras = p.ring_s + slot * (d / 32);
  } else {
    if (!xcd_item(s.tile_start[s.n_exp] * NT, &item)) return;
    rt = item_tile(s, item, NT, &nt);
  }
  if (rt.rows <= 0) return;
  const int n0 = nt * TN;
  const int last = rt.rows - 1;
  const int w = threadIdx.x >> 6, l = lane_id(), i = l & 31, h = l >> 5, wc = w & 3;
  const bool active = n0 + 64 * wc < I;
  const uint8_t* w2t = p.w2t + (size_t)rt.e * I * d;  // W2^T [I][d], quantised along d; scales [d/128][I] words
  const uint8_t* w2ts = p.w2ts + (size_t)rt.e * I * (d / 32);
  dispatch_rows(rt.rows, [&]<int F>() {
    constexpr int FH = (F + 1) / 2;
    const int m0 = (w >> 2) * FH;
    TileLoads8<F> L;
    if (ra) {  // ring dispatch: the rows sit in the chunk's slot in order
      L.init(ra, [&](int r) { return ra + (size_t)min(r, last) * d; },
             w2t, [&](int r) { return w2t + (size_t)min(n0 + r, I - 1) * d; },
             ras, [&](int r) { return ras + (size_t)min(r, last) * (d / 32); },
             w2ts, [&](int r) { return w2ts + (size_t)min(n0 + r, I - 1) * 4; });
    } else {
      L.init(p.dyq, [&](int r) { return p.dyq + (size_t)row_token(s, rt.r0 + min(r, last)) * d; },
             w2t, [&](int r) { return w2t + (size_t)min(n0 + r, I - 1) * d; },
             p.dys, [&](int r) { return p.dys + (size_t)row_token(s, rt.r0 + min(r, last)) * (d / 32); },
             w2ts, [&](int r) { return w2ts + (size_t)min(n0 + r, I - 1) * 4; });
    }
    L.bsk = 4 * I;  // stage-major scales: stage t's words are plane t
    v16f acc[FH][2];
    mainloop8<F, false>(lds, L, d / KS, acc);
    // combine weight of every row of the tile, once, through LDS
    float* wt = (float*)(lds + ((d / KS) % kStages) * STAGE_BYTES);
    if ((int)threadIdx.x < rt.rows) wt[threadIdx.x] = row_weight(s, p.w, rt.r0 + threadIdx.x);
    __syncthreads();
    if (!active) return;
    const int I2 = 2 * I;
    static_for<FH>([&]<int m>() {
      const int mi = m0 + m;
      // G and U of the fragment's 16 rows x 2 columns first: their loads overlap
      float gv[2][16], uv[2][16], wv[16];
      static_for<16>([&]<int v>() {
        const int rg = rt.r0 + min(32 * mi + 8 * (v >> 2) + 4 * h + (v & 3), last);
        wv[v] = wt[rg - rt.r0];
        static_for<2>([&]<int ni>() {
          const size_t o = (size_t)rg * I + n0 + 64 * wc + 32 * ni + i;
          gv[ni][v] = p.g[o];
          uv[ni][v] = p.u[o];
        });
      });
      static_for<16>([&]<int v>() {
        const int r = 32 * mi + 8 * (v >> 2) + 4 * h + (v & 3);
        const int rg = rt.r0 + min(r, last);
        static_for<2>([&]<int ni>() {
          const int n = n0 + 64 * wc + 32 * ni + i;
          const float g = gv[ni][v], u = uv[ni][v];
          const float dh = wv[v] * acc[m][ni][v];
          const float sg = sigmoid(g);
          const float dg = dh * u * sg * (1.0f + g * (1.0f - sg));
          const float du = dh * g * sg;
          uint32_t sc_g, sc_u;
          const uint32_t cg = quant_lane32(dg, &sc_g);
          const uint32_t cu = quant_lane32(du, &sc_u);
          if (r < rt.rows) {
            const size_t ro = (size_t)rg * I2;
            p.dguq[ro + n] = (uint8_t)cg;
            p.dguq[ro + I + n] = (uint8_t)cu;
            if (i == 0) {
              p.dgus[(size_t)rg * (I2 / 32) + (n >> 5)] = (uint8_t)sc_g;
              p.dgus[(size_t)rg * (I2 / 32) + ((I + n) >> 5)] = (uint8_t)sc_u;
            }
          }
        });
        if ((v & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      });
    });
  });
}

// ---------------------------------------------------------------------------------------------
// Backward dgrad of the gate/up GEMM: dX_r = dGU_r W1t_e^T, pushed to dXslot[t, j]
// (push reverse-dispatch).

__global__ __launch_bounds__(512, 1) void k_gemm_dgrad_gateup(DgradGateUpArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SchedView& s = p.s;
  const int I2 = 2 * p.I, d = p.d, NT = (d + TN - 1) / TN;
  int item;
  if (!xcd_item(s.tile_start[s.n_exp] * NT, &item)) return;
  int nt;
  const RowTile rt = item_tile(s, item, NT, &nt);
  if (rt.rows <= 0) return;
  const int n0 = nt * TN;
  const int last = rt.rows - 1;
  const int w = threadIdx.x >> 6, l = lane_id(), i = l & 31, h = l >> 5, wc = w & 3;
  const bool active = n0 + 64 * wc < d;
  const uint8_t* w1t = p.w1t + (size_t)rt.e * d * I2;  // W1^T [d][2I], quantised along 2I; scales [2I/128][d] words
  const uint8_t* w1ts = p.w1ts + (size_t)rt.e * d * (I2 / 32);
  dispatch_rows(rt.rows, [&]<int F>() {
    constexpr int FH = (F + 1) / 2;
    const int m0 = (w >> 2) * FH;
    TileLoads8<F> L;
    const uint8_t* ga = p.dguq + (size_t)rt.r0 * I2;
    const uint8_t* gsa = p.dgus + (size_t)rt.r0 * (I2 / 32);
    L.init(ga, [&](int r) { return ga + (size_t)min(r, last) * I2; },
           w1t, [&](int r) { return w1t + (size_t)min(n0 + r, d - 1) * I2; },
           gsa, [&](int r) { return gsa + (size_t)min(r, last) * (I2 / 32); },
           w1ts, [&](int r) { return w1ts + (size_t)min(n0 + r, d - 1) * 4; });
    L.bsk = 4 * d;  // stage-major scales: stage t's words are plane t
    v16f acc[FH][2];
    mainloop8<F, false>(lds, L, I2 / KS, acc);
    const int64_t* slot = row_slot_table(s, rt, lds + ((I2 / KS) % kStages) * STAGE_BYTES);
    if (!active) return;
    static_for<FH>([&]<int m>() {
      static_for<16>([&]<int v>() {
        const int r = 32 * (m0 + m) + 8 * (v >> 2) + 4 * h + (v & 3);
        if (r < rt.rows) {
          float* dst = p.dxslot + slot[r] * d + n0 + 64 * wc + i;
          dst[0] = acc[m][0][v];
          dst[32] = acc[m][1][v];
        }
      });
    });
  });
}

// ---------------------------------------------------------------------------------------------
// Weight gradients: dW_e[m, n] = sum over the expert's tokens of At[m, tok] Bt[n, tok], both
// operands requantised along the token axis and stored token-contiguous at the expert's padded
// offset.  An expert with no tokens writes zeros.  Tiles are 256 x 256 (128 x 256 when M is not
// a multiple of 256): the token count is short, so a bigger tile amortises each load latency.
// They run on the 8-wave core (both operands' scales in groups).

// kWhich only names the launch (0: dW2, 1: dW1) so that traces tell the two GEMMs apart.
template <int kWgradF, int kWhich>
__global__ __launch_bounds__(512, 1) void k_gemm_wgrad(WgradArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int MT = p.M / (32 * kWgradF), NT = (p.N + TN - 1) / TN;
  int item;
  if (!xcd_item(p.n_exp * MT * NT, &item)) return;
  // Items of one expert in blocks of NB column tiles, row tiles within a block: the items in
  // flight on an XCD (one contiguous item range per XCD) share the block's NB B tiles, which
  // stay in its L2 while the row tiles' A tiles stream past once per block.  With every column
  // tile in one block (NT <= 16) this is row-tile-major, column tiles fastest.
  const int NB = NT <= 16 ? NT : (NT + 1) / 2;
  const int e = item / (NT * MT), j = item - e * NT * MT;
  const int nb0 = (j / (MT * NB)) * NB, nbs = min(NB, NT - nb0);
  const int rr = j - nb0 * MT;
  const int mt = rr / nbs, nt = nb0 + rr % nbs;
  const int64_t k0 = p.tok_off[e];
  const int K = (int)(p.tok_off[e + 1] - k0);  // multiple of 128
  const int64_t ld = p.ld;                      // token stride of At / Bt rows
  const int m0 = mt * 32 * kWgradF, n0 = nt * TN;
  const int w = threadIdx.x >> 6, l = lane_id(), i = l & 31, h = l >> 5, wc = w & 3;
  const bool active = n0 + 64 * wc < p.N;
  constexpr int FH = (kWgradF + 1) / 2;
  const int mh = (w >> 2) * FH;
  TileLoads8<kWgradF> L;
  const uint8_t* at = p.at + (size_t)m0 * ld + k0;
  const uint8_t* bt = p.bt + (size_t)n0 * ld + k0;
  const uint8_t* ats = p.ats + (size_t)m0 * (ld / 32) + k0 / 32;
  const uint8_t* bts = p.bts + (size_t)n0 * (ld / 32) + k0 / 32;
  // With bf16 weight gradients the B rows are staged in pair order: in each wave's 64 columns,
  // fragment 0's lane i computes column 2i and fragment 1's lane i column 2i + 1, so that a lane
  // packs two neighbouring bf16 values into one word (the same dot products, other labels).
  // float32 keeps the plain order: 4-byte stores of 32 neighbouring columns fill a line already.
  const bool pairs = p.dw_bf16 != 0;
  auto bcol = [&](int r) {
    const int j = r & 63;
    return pairs ? (r & ~63) + (j < 32 ? 2 * j : 2 * (j - 32) + 1) : r;
  };
  L.init(at, [&](int r) { return at + (size_t)min(r, 32 * kWgradF - 1) * ld; },
         bt, [&](int r) { return bt + (size_t)(min(n0 + bcol(r), p.N - 1) - n0) * ld; },
         ats, [&](int r) { return ats + (size_t)min(r, 32 * kWgradF - 1) * (ld / 32); },
         bts, [&](int r) { return bts + (size_t)(min(n0 + bcol(r), p.N - 1) - n0) * (ld / 32); });
  v16f acc[FH][2];
  mainloop8<kWgradF>(lds, L, K / KS, acc);
  if (!active) return;
  if (pairs) {
    // the same float32 values rounded to bf16: half the bytes of the store stream; lane i writes
    // columns 2i, 2i + 1 as one word, so each half-wave writes one whole 128-byte line
    uint16_t* out = (uint16_t*)p.dw + (size_t)e * p.M * p.N;
    static_for<FH>([&]<int mi>() {
      static_for<16>([&]<int v>() {
        const int m = m0 + 32 * (mh + mi) + 8 * (v >> 2) + 4 * h + (v & 3);
        const uint32_t word =
            (uint32_t)f32_to_bf16(acc[mi][0][v]) | ((uint32_t)f32_to_bf16(acc[mi][1][v]) << 16);
        __builtin_nontemporal_store(word, (uint32_t*)(out + (size_t)m * p.N + n0 + 64 * wc + 2 * i));
      });
    });
    return;
  }
  float* out = (float*)p.dw + (size_t)e * p.M * p.N;
  static_for<FH>([&]<int mi>() {
    static_for<16>([&]<int v>() {
      const int m = m0 + 32 * (mh + mi) + 8 * (v >> 2) + 4 * h + (v & 3);
      float* dst = out + (size_t)m * p.N + n0 + 64 * wc + i;
      __builtin_nontemporal_store(acc[mi][0][v], dst);
      __builtin_nontemporal_store(acc[mi][1][v], dst + 32);
    });
  });
}

// ---------------------------------------------------------------------------------------------
// launchers

size_t gemm_lds_bytes() { return GEMM_LDS_BYTES; }
static size_t wgrad_lds_bytes() { return GEMM_LDS_BYTES; }

hipError_t launch_gemm_gateup(const GateUpArgs& a, int tiles_bound, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_gateup, dim3(tiles_bound * (a.I / 128)), dim3(512), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const DownArgs& a, int tiles_bound, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_down, dim3(tiles_bound * ((a.d + TN - 1) / TN)), dim3(512), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_dgrad_down(const DgradDownArgs& a, int tiles_bound, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_dgrad_down, dim3(tiles_bound * ((a.I + TN - 1) / TN)), dim3(512), gemm_lds_bytes(),
                     st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_dgrad_gateup(const DgradGateUpArgs& a, int tiles_bound, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_dgrad_gateup, dim3(tiles_bound * ((a.d + TN - 1) / TN)), dim3(512), gemm_lds_bytes(),
                     st, a);
  return hipGetLastError();
}

template <int kWhich>
static hipError_t launch_wgrad(const WgradArgs& a, hipStream_t st) {
  // 256-row tiles when M allows (half the workgroups, each with twice the work per load latency)
  if (a.M % 256 == 0) {
    const int blocks = a.n_exp * (a.M / 256) * ((a.N + TN - 1) / TN);
    hipLaunchKernelGGL((k_gemm_wgrad<8, kWhich>), dim3(blocks), dim3(512), wgrad_lds_bytes(), st, a);
  } else if (a.M % 128 == 0) {
    const int blocks = a.n_exp * (a.M / 128) * ((a.N + TN - 1) / TN);
    hipLaunchKernelGGL((k_gemm_wgrad<4, kWhich>), dim3(blocks), dim3(512), wgrad_lds_bytes(), st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad(const WgradArgs& a, int which, hipStream_t st) {
  return which ? launch_wgrad<1>(a, st) : launch_wgrad<0>(a, st);
}

hipError_t gemm_init() {
  const int bytes = (int)gemm_lds_bytes();
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_gateup, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_down, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_dgrad_down, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm_dgrad_gateup, hipFuncAttributeMaxDynamicSharedMemorySize, bytes))) return e;
  for (const void* k : {(const void*)k_gemm_wgrad<8, 0>, (const void*)k_gemm_wgrad<8, 1>,
                        (const void*)k_gemm_wgrad<4, 0>, (const void*)k_gemm_wgrad<4, 1>})
    if ((e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)wgrad_lds_bytes()))) return e;
  return hipSuccess;
}

}  // namespace moe
