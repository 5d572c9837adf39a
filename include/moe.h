/* moe.h -- C ABI of the MI355X (gfx950) MoE-layer library (libmoe_mi355x.so).
 *
 * One DeepSeek-V3-style mixture-of-experts layer, forward and backward, computed in MXFP8 on
 * one GPU with every expert resident in HBM.  The method is the one the pages describe for
 * Cursor's Mixture-of-Kittens training megakernel (knowledge card
 * "Mixture-of-Kittens——面向NVL72的开源MoE训练megakernel", sections 一句话结论 and
 * 方法/产品要点; article "Cursor 為 Composer 改造 MoE 訓練：MoK 點樣拆走跨 GPU 樽頸", section
 * "MoK 將運算同通訊塞入同一個核心"): a device-side schedule reused by the backward pass,
 * pull-based dispatch, push-based combine, pull-based reverse-combine, push-based
 * reverse-dispatch, fixed-capacity ring token buffers, no CPU-GPU synchronisation inside the
 * layer, deterministic results.
 *
 * Conventions for every entry point
 *   - Pointers are device pointers unless stated otherwise; the caller allocates and frees
 *     every buffer.  The library never allocates device memory, never frees, and never
 *     synchronises the host inside moe_fwd / moe_bwd: work is enqueued on the caller's stream
 *     and the call returns (knowledge card, 方法/产品要点: no CPU-GPU synchronisation).
 *   - Tensors are dense, row-major, contiguous.  "bf16" is bfloat16 stored as uint16_t,
 *     "fp8" is OCP e4m3 ("fn") stored as uint8_t, "e8m0" is a biased-127 exponent byte.
 *   - MXFP8: a tensor quantised along an axis holds fp8 codes of the same shape plus one
 *     e8m0 byte per 32 consecutive values along that axis (OCP Microscaling v1.0).
 *   - Argument errors are detected on the host before anything is enqueued and returned as a
 *     moe_status; nothing is launched then.  Launch failures return MOE_ELAUNCH.
 *   - Tensor pointers must be 16-byte aligned; `saved` and `workspace` 256-byte aligned.
 *   - Concurrency: calls on different streams may overlap as long as they use different
 *     `saved` and `workspace` buffers; the library's own streams and the events that order
 *     them are kept per host thread and device, so calls from different threads never share
 *     them.  moe_set_phase_events is process-wide and meant for single-threaded measurement.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,      /* null pointer or unsupported option */
  MOE_ESHAPE = 2,      /* sizes outside the supported set (see moe_config) */
  MOE_EALIGN = 3,      /* a pointer is not aligned as required */
  MOE_EWORKSPACE = 4,  /* `saved` or `workspace` smaller than moe_query reports */
  MOE_ELAUNCH = 5,     /* a kernel launch failed */
  MOE_EDEVICE = 6      /* reported by moe_device_status: the device flagged an anomaly */
} moe_status;

/* Codes the device writes into the workspace status word (read with moe_device_status).  The
 * word is sticky: a later call does not clear it. */
#define MOE_DEV_RING_TIMEOUT 1   /* a bounded wait of the persistent ring kernel expired (that
                                    kernel is not launched; the stream-ordered ring of
                                    MOE_F_RING_DISPATCH has no device-side waits) */
#define MOE_DEV_NONFINITE_LOGIT 2 /* a router logit was NaN or infinite (its token is still
                                     routed to k distinct valid experts; NaN ranks as -inf) */

typedef enum moe_score_fn {
  MOE_SCORE_SOFTMAX = 0, /* softmax over the k selected logits */
  MOE_SCORE_SIGMOID = 1  /* sigmoid scores of the k selected experts, normalised to sum 1 */
} moe_score_fn;

/* Layer shape and tuning.  Supported: T >= 1; d and inter multiples of 128; 1 <= k <= 16;
 * k <= E <= 512; n_shared in {0, 1}; T*(k + n_shared) < 2^30; T*d < 2^32; 2*inter*d < 2^32;
 * the token-axis operand stride of the weight-gradient GEMMs (about T*(k + n_shared) + 128*(E +
 * n_shared)) below 2^24 (several kernels address an operand with 32-bit byte offsets).
 * The tuning fields are the pages' per-workload knobs (buffer capacity, minibatch and number of
 * communication SMs: article "Cursor 為 Composer 改造 MoE 訓練…", section "2.37 倍同 1.41 倍係兩份
 * 成績").  chunk_rows, the rows of one GEMM row tile (the unit of work the grouped GEMMs and the
 * ring hand out), acts on every path: smaller tiles give more work items per GEMM for few rows
 * per expert, at the cost of streaming each weight slice once more per extra tile.  ring_rows and
 * producer_wgs act on the ring dispatch (MOE_F_RING_DISPATCH) only and must be 0 otherwise.  0
 * picks a default.  They never change results.  moe_bwd must see the chunk_rows of the moe_fwd
 * whose saved schedule it reuses (the saved row-tile table is built for it). */
typedef struct moe_config {
  int32_t T;          /* tokens */
  int32_t d;          /* hidden size */
  int32_t E;          /* routed experts */
  int32_t k;          /* experts per token */
  int32_t inter;      /* SwiGLU intermediate size I */
  int32_t n_shared;   /* always-on shared experts (weight 1), stored after the E routed ones */
  int32_t score_fn;   /* moe_score_fn */
  int32_t ring_rows;  /* ring token buffer capacity in rows (0 = 16384; a multiple of the row-tile
                         height chunk_rows, at least one tile) */
  int32_t chunk_rows; /* rows per GEMM row tile at most (0 = 256; a multiple of 32 up to 256);
                         with the ring dispatch also the rows of one ring slot */
  int32_t producer_wgs; /* workgroups gathering rows into the ring (0 = 128, max 128) */
  uint32_t flags;     /* MOE_F_* */
} moe_config;

/* Forward dispatch.  By default the gate/up GEMM pulls its rows straight from the quantised
 * activations through the schedule (MOE_F_DIRECT_GATHER names that default explicitly).
 * MOE_F_RING_DISPATCH stages them instead in the fixed-capacity ring token buffer of the
 * workspace, reused cyclically (knowledge card "Mixture-of-Kittens——面向NVL72的开源MoE训练
 * megakernel", 方法/产品要点: ring buffers, pull dispatch; article "Cursor 為 Composer 改造 MoE
 * 訓練…", section "MoK 將運算同通訊塞入同一個核心": part of the GPU moves data while the rest
 * computes): the chunks (GEMM row tiles, one per slot of chunk_rows rows) go in rounds of half
 * the slots; producer_wgs workgroups on a stream of the library's own gather a round's rows into
 * its slots while the gate/up GEMM on the caller's stream runs the previous round from the
 * other half, ordered by events (no device-side waits, no host synchronisation).  moe_bwd does
 * the same for its pull reverse-combine (same pages: the dY rows each expert needs, staged in
 * the ring for the dgrad-down GEMM; the producers have a stream of their own beside the
 * backward's second-stream branch, and MOE_F_SERIAL_BWD puts them in launch order).  Every row is
 * processed at any capacity down to one slot, and the results are bitwise those of direct
 * gather.  Both flags together: MOE_EINVAL. */
#define MOE_F_DIRECT_GATHER 1u
#define MOE_F_RING_DISPATCH 2u

/* Backward schedule.  By default moe_bwd runs the branch that needs only the forward's saved
 * rows and dy (token-axis requantisation of X, H and w*dY, then dW2) on a second stream of the
 * device, created by the library on first use in each host thread with default priority and
 * kept until the process ends, beside the router backward and the dgrad chain; the caller's
 * stream waits for it before dW1, so the call stays ordered on the caller's stream as a whole.
 * MOE_F_SERIAL_BWD runs every kernel in launch order on the caller's stream instead (phase
 * timing then covers every phase; results are identical either way). */
#define MOE_F_SERIAL_BWD 4u

/* Check mode of the combine: every expert is replaced by the identity (the row of expert e for
 * token t is x[t] itself), so moe_fwd runs the router, top-k, schedule and x quantisation, writes
 * x into every (token, slot) row of the saved Y slots and then the ordinary fixed-order weighted
 * combine.  The combine weights sum to 1 (knowledge card "Mixture-of-Kittens——面向NVL72的开源MoE
 * 训练megakernel", 方法/产品要点: deterministic combine), so the bf16 output is x (times 1 + n_shared
 * with shared experts) bit for bit.  The weight pointers are still required and are not read;
 * moe_bwd rejects the flag with MOE_EINVAL (there is no saved expert state to differentiate). */
#define MOE_F_IDENTITY_EXPERTS 8u

/* Forward only: moe_fwd skips what only the backward pass reads (the transposed requantised
 * expert weights w1t / w2t of the saved buffer, which then take no space); moe_bwd rejects the
 * flag with MOE_EINVAL. */
#define MOE_F_FORWARD_ONLY 16u

/* The unfused forward: the same arithmetic as the default forward, bit for bit, as the
 * conventional pipeline of separate kernels with a trip through HBM at every boundary (route,
 * permute, expert GEMMs, activation, unpermute, combine: commentary "Cursor 开源 MoK…", sections
 * 瓶颈的真正来源 and 两份成绩单), kept as the in-house baseline that measures what the fused forward
 * buys: a permute pass gathers the quantised rows into expert order, the gate/up GEMM reads them
 * contiguously and stores G and U, a separate pass applies SwiGLU and quantises H, the down GEMM
 * writes its rows in expert order and an unpermute pass moves them to their (token, slot) rows
 * before the combine.  Needs MOE_F_FORWARD_ONLY and T*(k + n_shared)*d < 2^32 (else MOE_EINVAL /
 * MOE_ESHAPE); the workspace then holds the permuted rows (moe_workspace_layout xp, xps, yrows).
 * moe_fwd_noalloc rejects it (MOE_EINVAL). */
#define MOE_F_UNFUSED 32u

/* Weight gradients in bfloat16: moe_bwd writes dw1 and dw2 as bf16 (2 bytes per element, same
 * shapes and layouts), each the round-to-nearest-even of the float32 value the default path
 * writes, bit for bit.  The fp32 weight gradients are most of the backward's HBM traffic (the
 * byte floor of the DeepSeek-V3-shape layer drops by about a quarter); callers that keep their
 * gradient accumulation elsewhere can take them in bf16.  moe_fwd ignores it. */
#define MOE_F_DW_BF16 64u

/* Byte offsets inside the caller-owned `saved` buffer that moe_fwd fills and moe_bwd reads
 * (the schedule is built once and reused by the backward pass: knowledge card, 方法/产品要点).
 * R = T*k routed rows, RS = R + n_shared*T rows in expert-major ("permuted") order,
 * S = n_shared, NX = E + S. */
typedef struct moe_saved_layout {
  size_t logits;     /* float [T, E]       router logits (+ bias) */
  size_t idx;        /* int32 [T, k]       selected experts, best first */
  size_t w;          /* float [T, k]       combine weights */
  size_t counts;     /* int32 [NX]         rows per expert */
  size_t offsets;    /* int32 [NX + 1]     first permuted row of each expert */
  size_t poffsets;   /* int32 [NX + 1]     offsets with every count rounded up to 32 */
  size_t tok_off;    /* int64 [NX + 1]     offsets with every count rounded up to 128 */
  size_t tile_start; /* int32 [NX + 1]     first row tile of each expert (ceil(count / chunk_rows) each) */
  size_t tile64;     /* int32 [NX + 1]     first 64-row tile of each 128-padded segment */
  size_t perm;       /* int32 [R]          slot id t*k + j of each routed permuted row */
  size_t pos;        /* int32 [T, k]       permuted row of slot (t, j) */
  size_t xq;         /* fp8   [T, d]       x quantised along d */
  size_t xs;         /* e8m0  [T, d/32] */
  size_t g;          /* float [RS, I]      gate pre-activations */
  size_t u;          /* float [RS, I]      up projections */
  size_t hq;         /* fp8   [RS, I]      silu(g) * u quantised along I */
  size_t hs;         /* e8m0  [RS, I/32] */
  size_t yslot;      /* float [T, k + S, d] expert output of every (token, slot) */
  size_t w1t;        /* fp8   [NX, d, 2I]  W1 transposed, requantised along 2I (experts with rows) */
  size_t w1ts;       /* e8m0  [NX, 2I/128, d, 4]  its scales, word-major: [e][q][k][b] is the
                        scale of block 4q + b of transposed row k */
  size_t w2t;        /* fp8   [NX, I, d]   W2 transposed, requantised along d (experts with rows) */
  size_t w2ts;       /* e8m0  [NX, d/128, I, 4]  its scales, word-major as for w1ts */
  size_t total;      /* bytes of `saved` */
} moe_saved_layout;

/* Byte offsets inside the caller-owned `workspace` (scratch of moe_fwd and moe_bwd; exported
 * so that tests can read the stage results of the backward pass).  ld = tok_stride. */
typedef struct moe_workspace_layout {
  size_t status;     /* int32              device status word (MOE_DEV_*), sticky */
  size_t ring;       /* fp8   [ring_rows, d] ring token buffer (ring dispatch only): ring_rows /
                        chunk_rows slots of chunk_rows rows; sized by ring_rows alone, so one
                        workspace serves every chunk_rows */
  size_t ring_s;     /* e8m0  [ring_rows, d/32] */
  size_t ring_flags; /* int32 [2 ring_rows/32 + 1] (unused by the stream-ordered ring; kept for layout) */
  size_t blkcnt;     /* int32 [ceil(T/64), E] per-block expert counts, then their scans */
  size_t dyq;        /* fp8   [T, d]       dy quantised along d */
  size_t dys;        /* e8m0  [T, d/32] */
  size_t dw;         /* float [T, k]       gradient of the combine weights */
  size_t dl;         /* float [T, k]       gradient of the selected logits */
  size_t dguq;       /* fp8   [RS, 2I]     [dG dU] quantised along 2I (permuted rows) */
  size_t dgus;       /* e8m0  [RS, 2I/32] */
  size_t dxslot;     /* float [T, k + S, d] input gradient of every (token, slot) */
  size_t xt;         /* fp8   [d, ld]      X rows of each expert, requantised along tokens */
  size_t xts;        /* e8m0  [d, ld/32] */
  size_t ht;         /* fp8   [I, ld]      H, same */
  size_t hts;        /* e8m0  [I, ld/32] */
  size_t dyt;        /* fp8   [d, ld]      w * dY, same */
  size_t dyts;       /* e8m0  [d, ld/32] */
  size_t dgut;       /* fp8   [2I, ld]     [dG dU], same */
  size_t dguts;      /* e8m0  [2I, ld/32] */
  size_t xp;         /* fp8   [RS, d]      quantised rows in expert order (MOE_F_UNFUSED only, else empty) */
  size_t xps;        /* e8m0  [RS, d/32] */
  size_t yrows;      /* float [RS, d]      down GEMM rows in expert order (MOE_F_UNFUSED only) */
  size_t tok_stride; /* ld: tokens per row of the token-axis operands (a size, not an offset);
                        expert e occupies columns [tok_off[e], tok_off[e + 1]) */
  size_t total;      /* bytes of `workspace` */
} moe_workspace_layout;

/* Sizes of the caller-owned buffers for `cfg`: *workspace_bytes for the workspace shared by
 * moe_fwd and moe_bwd, *saved for the layout of the saved buffer (the schedule and activations
 * the forward pass hands to the backward pass: knowledge card, 方法/产品要点, reusable schedule),
 * *work for the layout of the workspace.  Any output pointer may be NULL.  Host-only; no GPU
 * needed.  Returns MOE_ESHAPE / MOE_EINVAL for a configuration outside the supported set. */
moe_status moe_query(const moe_config* cfg, size_t* workspace_bytes, moe_saved_layout* saved,
                     moe_workspace_layout* work);

/* MXFP8 quantisation (the format the pages name for the whole layer: knowledge card,
 * 方法/产品要点, "MXFP8") of a [rows, cols] matrix along its contiguous axis (cols % 32 == 0):
 * src is bf16 (src_is_f32 = 0) or float32 (src_is_f32 = 1); q [rows, cols] fp8 and
 * scales [rows, cols/32] e8m0 receive the result.  Block scale 2^(floor(log2 amax) - 8), codes
 * rounded to nearest even and saturated at +-448.  Used for expert weights and by the layer for
 * x and dy.  src and q 16-byte aligned.  Enqueued on `stream`; MOE_ESHAPE for cols % 32 != 0. */
moe_status moe_quantize_mxfp8(const void* src, int src_is_f32, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* scales, hipStream_t stream);

/* Transposed requantisation (the backward pass's requantisation of transposed operands, for an
 * MXFP8 layer that also trains: knowledge card, 方法/产品要点, MXFP8 forward and backward):
 * q [batch, rows, cols] fp8 with scales [batch, rows, cols/32] (quantised along cols) is
 * dequantised exactly and quantised again along rows into qt [batch, cols, rows] with
 * st [batch, cols, rows/32].  rows and cols multiples of 64 (else MOE_ESHAPE).  moe_fwd writes
 * the expert weights' transposes (W1 along 2I, W2 along d) with the same arithmetic from its
 * GEMMs' weight stream; this standalone form serves tests and callers that want them. */
moe_status moe_requant_transpose(const uint8_t* q, const uint8_t* scales, int64_t batch, int64_t rows, int64_t cols,
                                 uint8_t* qt, uint8_t* st, hipStream_t stream);

/* Forward pass of the layer (knowledge card, 方法/产品要点: DSV3-style MoE layer in MXFP8, pull-based
 * forward dispatch, push-based forward combine, device-side schedule; commentary "Cursor 开源
 * MoK…", section 什么是MoK: route, dispatch, expert FFN, combine).
 *   x [T, d] bf16; w_router [E, d] bf16; router_bias [E] float or NULL (added to every
 *   token's logits); w1q [NX, 2I, d] fp8 with w1s [NX, 2I, d/32] (gate rows 0..I-1, up rows
 *   I..2I-1, quantised along d); w2q [NX, d, I] fp8 with w2s [NX, d, I/32] (quantised along I).
 *   Outputs: y_bf16 [T, d]; y_f32 [T, d] float or NULL (the same sum before bf16 rounding);
 *   saved (moe_saved_layout) for moe_bwd.  saved_bytes / workspace_bytes: the sizes of the
 *   caller's buffers (MOE_EWORKSPACE if below what moe_query reports).
 * Steps (all on `stream`, no host sync): quantise x; router logits; top-k and weights; schedule
 * (counts, offsets, stable expert-major permutation); gate/up grouped GEMM with rows pulled
 * through the schedule, SwiGLU and H quantisation in the epilogue; down grouped GEMM pushing
 * each row to its (token, slot); combine in fixed slot order.  Unless MOE_F_FORWARD_ONLY, the
 * two GEMMs also requantise the weight slices they stream along the other axis into saved
 * w1t / w2t, for the backward pass. */
moe_status moe_fwd(const moe_config* cfg, const void* x, const void* w_router, const float* router_bias,
                   const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q, const uint8_t* w2s, void* y_bf16,
                   float* y_f32, void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* moe_fwd without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  Same arguments and
 * results as moe_fwd (bit for bit); the forward's scratch (the device status word and the
 * schedule's per-block expert counts, 256 + 4 * ceil(T / 64) * E bytes) lives in a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends.  Returns MOE_EWORKSPACE when the configuration needs more scratch than that,
 * MOE_EINVAL with MOE_F_RING_DISPATCH.  Nothing is allocated or freed.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (different streams, threads) race and
 * must be ordered by the caller.  The status word is not readable through moe_device_status. */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_fwd_noalloc(const moe_config* cfg, const void* x, const void* w_router, const float* router_bias,
                           const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q, const uint8_t* w2s,
                           void* y_bf16, float* y_f32, void* saved, size_t saved_bytes, hipStream_t stream);

/* Backward pass for upstream gradient dy [T, d] bf16, reusing `saved` from moe_fwd of the same
 * inputs and configuration (knowledge card, 方法/产品要点: pull-based reverse-combine, push-based
 * reverse-dispatch, schedule reused; article "Cursor 為 Composer 改造 MoE 訓練…", section
 * "2.37 倍同 1.41 倍係兩份成績": the layer's backward).  The expert weights enter through their
 * transposes in `saved`.  Outputs: dx_bf16 [T, d] and dx_f32 [T, d] float (or NULL);
 * dw_router [E, d] float; dw1 [NX, 2I, d] and dw2 [NX, d, I] (same layouts as w1q / w2q), float,
 * or bf16 with MOE_F_DW_BF16.
 * Steps: quantise dy; combine-weight and router gradients; dgrad of the down GEMM (rows pulled
 * from dy: reverse-combine) with the SwiGLU backward and quantisation along 2I; dgrad of the
 * gate/up GEMM pushing rows to their (token, slot) (reverse-dispatch); fixed-order reduction of
 * dx; token-axis requantisation of the wgrad operands; weight-gradient GEMMs. */
moe_status moe_bwd(const moe_config* cfg, const void* dy, const void* x, const void* w_router, const void* saved,
                   size_t saved_bytes, void* dx_bf16, float* dx_f32, float* dw_router, void* dw1, void* dw2,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Phase timing, for measurement only (the pages attribute the layer's time to its phases:
 * commentary "Cursor 开源 MoK…", section 瓶颈的真正来源).  Phases of moe_fwd / moe_bwd, in launch
 * order; the library records events[p] on the call's stream right after phase p has been
 * enqueued (and events[MOE_PH_FWD_BEGIN] / events[MOE_PH_BWD_BEGIN] before the first launch),
 * so the time of phase p is the elapsed time between the previous recorded event and events[p].
 * Without MOE_F_SERIAL_BWD the phases of the second-stream branch (MOE_PH_TOKEN_REQUANT's X / H /
 * dY part, MOE_PH_WGRAD_DOWN) overlap the others and their intervals do not measure them alone;
 * events[MOE_PH_WGRAD_DOWN] is then recorded after the join, so MOE_PH_WGRAD_GATEUP still times
 * dW1 alone.  The caller creates the events (hipEventCreate) and keeps them alive; n_events = 0
 * turns timing off.  Process-wide setting, not synchronised between threads.  Results are
 * unaffected. */
enum {
  MOE_PH_FWD_BEGIN = 0, MOE_PH_QUANT_X, MOE_PH_ROUTER, MOE_PH_TOPK, MOE_PH_SCHEDULE, MOE_PH_GATEUP,
  MOE_PH_DOWN, MOE_PH_COMBINE,
  MOE_PH_BWD_BEGIN, MOE_PH_QUANT_DY, MOE_PH_ROUTER_BWD, MOE_PH_ROUTER_WGRAD, MOE_PH_REQUANT_W,
  MOE_PH_DGRAD_DOWN, MOE_PH_DGRAD_GATEUP, MOE_PH_DX_REDUCE, MOE_PH_TOKEN_REQUANT, MOE_PH_WGRAD_DOWN,
  MOE_PH_WGRAD_GATEUP,
  MOE_PH_COUNT
};
moe_status moe_set_phase_events(hipEvent_t* events, int32_t n_events);

/* Measurement only (the MXFP8 roofline the layer's GEMM phases are reported against, next to
 * the published dense peak): enqueues on `stream` one launch of register-only scaled MXFP8
 * matrix instructions (v_mfma_scale_f32_32x32x64_f8f6f4, four waves per SIMD on every compute
 * unit, `iters` x 4 instructions per wave) and returns its algorithmic flop count in *flop; the
 * caller times the launch.  `sink` (device, sink_bytes) receives one float per thread; too small
 * a sink: MOE_EWORKSPACE, with *flop set to 0 and the size needed in *sink_needed when not NULL.
 * iters < 1: MOE_EINVAL. */
moe_status moe_probe_mfma(float* sink, size_t sink_bytes, int32_t iters, double* flop, size_t* sink_needed,
                          hipStream_t stream);

/* Reads the device status word of `workspace` (0 = fine; else a MOE_DEV_* code) into
 * *device_code: the layer's way to report a device-side anomaly without a host sync inside the
 * layer (knowledge card, 方法/产品要点: no CPU-GPU synchronisation).  Blocking copy: call after
 * the caller has synchronised the stream.  Returns MOE_EDEVICE if the code is non-zero. */
moe_status moe_device_status(const void* workspace, int32_t* device_code);

/* Static text for a status (never NULL). */
const char* moe_strerror(moe_status status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
