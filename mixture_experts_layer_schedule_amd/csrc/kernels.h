// Internal kernel launchers and their argument blocks (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Device-side view of the schedule built by the router/schedule kernels.
// Tokens per block of the schedule builder (per-block expert histograms, scanned per expert).
constexpr int kSchedBlockTokens = 64;

struct SchedView {
  const int32_t* perm;        // [R] slot id t*k + j of each routed permuted row
  const int32_t* offsets;     // [n_exp + 1] first permuted row of each expert
  const int32_t* tile_start;  // [n_exp + 1] first row tile of each expert (ceil(count / tile rows) each)
  int n_exp;                  // routed + shared experts
  int R;                      // routed rows T * k (shared rows follow)
  int T, k, S;
};

struct GateUpArgs {
  SchedView s;
  const uint8_t *xq, *xs, *w1q, *w1s;  // xq, xs: [T, d] gathered through the schedule, or with
                                       // `contiguous` [RS, d] already in expert order
  float *g, *u;
  uint8_t *hq, *hs;     // NULL with `contiguous`: G and U only (the unfused forward)
  uint8_t *w1t, *w1ts;  // [NX][d][2I] + [NX][2I/128][d][4]: W1 transposed, requantised along 2I (NULL: skip)
  int d, I;
  int contiguous;
  // ring dispatch (ring != NULL): the launch runs chunks [chunk0, chunk0 + nchunks) (chunk =
  // row tile), whose rows the producers staged in slot c % nslots: ring [nslots][slot_rows][d],
  // ring_s [nslots][slot_rows][d/32]
  const uint8_t *ring, *ring_s;
  int chunk0, nchunks, nslots, slot_rows;
};

struct DownArgs {
  SchedView s;
  const uint8_t *hq, *hs, *w2q, *w2s;
  float* yslot;          // each row pushed to its (token, slot) row
  float* yrows;          // or, when not NULL, [RS, d] rows in expert order (the unfused forward)
  uint8_t *w2t, *w2ts;  // [NX][I][d] + [NX][d/128][I][4]: W2 transposed, requantised along d (NULL: skip)
  int d, I;
};

struct DgradDownArgs {
  SchedView s;
  const uint8_t *dyq, *dys;
  const uint8_t *w2t, *w2ts;  // [NX][I][d] + [NX][d/128][I][4] (written by the forward down GEMM)
  const float *w, *g, *u;
  uint8_t *dguq, *dgus;
  int d, I;
  // ring dispatch (ring != NULL): as GateUpArgs, the slots holding dYq / dYs rows
  const uint8_t *ring, *ring_s;
  int chunk0, nchunks, nslots, slot_rows;
};

struct DgradGateUpArgs {
  SchedView s;
  const uint8_t *dguq, *dgus;
  const uint8_t *w1t, *w1ts;  // [NX][d][2I] + [NX][2I/128][d][4] (written by the forward gate/up GEMM)
  float* dxslot;
  int d, I;
};

struct WgradArgs {
  const uint8_t *at, *ats, *bt, *bts;  // [M][ld], [M][ld/32]; [N][ld], [N][ld/32]
  const int64_t* tok_off;              // [n_exp + 1] padded token offsets (multiples of 128)
  void* dw;                            // [n_exp][M][N] float, or bf16 with dw_bf16
  int64_t ld;
  int M, N, n_exp;                     // M a multiple of 128
  int dw_bf16;                         // store dw rounded to bf16 (nearest, ties to even)
};

// Persistent gate/up kernel fed through ring token buffers (producer / consumer workgroups).
struct RingArgs {
  SchedView s;
  const uint8_t *xq, *xs, *w1q, *w1s;
  float *g, *u;
  uint8_t *hq, *hs;
  uint8_t *ring, *ring_s;          // [nslots][256][d], [nslots][256][d/32]
  int32_t *ready, *done;           // [nslots] each: published lap + 1; finished work units (cumulative)
  int32_t* abort_flag;             // set when a bounded wait expires
  int32_t* status;                 // device status word (sticky)
  int32_t* flags;                  // ready | done | abort, zeroed before every launch
  int n_flags;
  int d, I, nslots, producers, spin_limit;
};

size_t gemm_lds_bytes();
hipError_t gemm_init();
hipError_t ring_init();
int ring_max_resident();
hipError_t launch_ring_gateup(const RingArgs&, hipStream_t);
hipError_t launch_gemm_gateup(const GateUpArgs&, int tiles_bound, hipStream_t);
// Producer side of the ring dispatch: rows of chunks [chunk0, chunk0 + nchunks) into their slots.
hipError_t launch_ring_gather(const SchedView& s, const uint8_t* xq, const uint8_t* xs, int d, uint8_t* ring,
                              uint8_t* ring_s, int slot_rows, int nslots, int chunk0, int nchunks, int producers,
                              hipStream_t st);
hipError_t launch_gemm_down(const DownArgs&, int tiles_bound, hipStream_t);
hipError_t launch_gemm_dgrad_down(const DgradDownArgs&, int tiles_bound, hipStream_t);
hipError_t launch_gemm_dgrad_gateup(const DgradGateUpArgs&, int tiles_bound, hipStream_t);
// which: 0 for dW2, 1 for dW1 (separate kernel names in traces)
hipError_t launch_gemm_wgrad(const WgradArgs&, int which, hipStream_t);

// The unfused forward's own passes: xp[r] = xq[token of permuted row r] (codes and scales);
// H = quantise(silu(G) U) along I; yslot[slot of row r] = yrows[r].
hipError_t launch_permute_rows(const SchedView& s, const uint8_t* xq, const uint8_t* xs, int d, int RS, uint8_t* xp,
                               uint8_t* xps, hipStream_t);
hipError_t launch_swiglu_quant(const float* g, const float* u, int RS, int I, uint8_t* hq, uint8_t* hs, hipStream_t);
hipError_t launch_unpermute_rows(const SchedView& s, const float* yrows, int RS, int d, float* yslot, hipStream_t);

// Measurement: the matrix core's MXFP8 issue rate (register operands only).
size_t probe_mfma_sink_bytes(int cus);
hipError_t launch_probe_mfma(float* sink, int cus, int iters, double* flop, hipStream_t);

// MXFP8 quantisation along the contiguous axis of a [rows, cols] bf16 (src_f32 = 0) or
// float32 (src_f32 = 1) matrix.
hipError_t launch_quant_rows(const void* src, int src_f32, int64_t rows, int64_t cols, uint8_t* q,
                             uint8_t* s, hipStream_t);
// Batched transposed requantisation: [batch][rows][cols] quantised along cols ->
// [batch][cols][rows] quantised along rows.
hipError_t launch_requant_t(const uint8_t* q, const uint8_t* s, int64_t batch, int64_t rows, int64_t cols,
                            uint8_t* qt, uint8_t* st, hipStream_t);

// Token-axis requantisation of expert rows into token-contiguous operands of the weight
// gradient GEMMs.
enum TokSrc { TOK_X = 0, TOK_H = 1, TOK_DGU = 2, TOK_DYW = 3 };
struct TokArgs {
  SchedView s;
  const uint8_t *q, *qs;     // source codes and scales (rows: tokens for X/DYW, permuted rows else)
  const float* w;            // combine weights [T*k] (TOK_DYW)
  const int64_t* tok_off;    // [n_exp + 1] padded token offsets
  const int32_t* tile64;     // [n_exp + 1] first 64-token tile of each expert
  uint8_t *out, *outs;       // [cols][ld], [cols][ld/32]
  int64_t ld;
  int cols;
  int src;
};
hipError_t launch_token_requant(const TokArgs&, int tiles_bound, hipStream_t);

// Router, top-k and schedule.
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_r, const float* bias, float* logits,
                                int T, int d, int E, hipStream_t);
// status: device status word (MOE_DEV_NONFINITE_LOGIT when a logit is NaN or infinite)
hipError_t launch_topk(const float* logits, int T, int E, int k, int score, int32_t* idx, float* w,
                       int32_t* status, hipStream_t);
struct SchedBuild {
  const int32_t* idx;   // [T, k]
  int32_t* blkcnt;      // [nblk, E] scratch
  int32_t* counts;      // [n_exp]
  int32_t* offsets;     // [n_exp + 1]
  int32_t* poffsets;    // [n_exp + 1] padded to 32
  int64_t* tok_off;     // [n_exp + 1] padded to 128 (weight-gradient operands)
  int32_t* tile_start;  // [n_exp + 1] row tiles of up to tile_rows rows
  int32_t* tile64;      // [n_exp + 1] 64-token tiles over the 128-padded segments
  int32_t* perm;        // [R]
  int32_t* pos;         // [T, k]
  int T, E, k, S;
  int tile_rows;        // rows per GEMM row tile at most (32 .. 256, a multiple of 32)
};
hipError_t launch_schedule(const SchedBuild&, hipStream_t);

// Combine and backward helpers.
// Combine check mode: yslot[t, j, :] = x[t, :] (bf16 widened exactly) for all j < slots.
hipError_t launch_identity_slots(const uint16_t* x, int T, int slots, int d, float* yslot, hipStream_t);
hipError_t launch_combine(const float* yslot, const float* w, int T, int k, int S, int d, uint16_t* y_bf16,
                          float* y_f32, hipStream_t);
hipError_t launch_router_bwd(const uint16_t* dy, const float* yslot, const float* logits, const int32_t* idx,
                             const float* w, int T, int E, int k, int S, int d, int score, float* dw_out,
                             float* dl_out, hipStream_t);
hipError_t launch_router_wgrad(const SchedView& s, const float* dl, const uint16_t* x, int d, int E,
                               float* dw_r, hipStream_t);
hipError_t launch_dx_reduce(const float* dxslot, const float* dl, const int32_t* idx, const uint16_t* w_r,
                            int T, int k, int S, int d, uint16_t* dx_bf16, float* dx_f32, hipStream_t);

}  // namespace moe
