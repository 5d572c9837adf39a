// Router logits, top-k selection with combine weights, and the device-side schedule.
//
// The pages' layer starts by routing every token to a few experts, and its schedule is built
// on the GPU with no CPU involvement and reused by the backward pass (knowledge card
// "Mixture-of-Kittens——面向NVL72的开源MoE训练megakernel", 方法/产品要点; commentary "Cursor 开源
// MoK…", 什么是MoK).  Everything here runs on the caller's stream with no host synchronisation.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// ----------------------------------------------------------------------------- logits
//
// L = x W_r^T on v_mfma_f32_32x32x16_bf16 (lane l = i + 32h holds row i, 8 K values; result
// layout as for every 32x32 MFMA).  Four MFMA steps cover 64 K values; lane half h takes the
// 32 consecutive values [32h, 32h + 32) of that span (8 per step), which only reorders the
// float32 accumulation, identically on every run.
//
// A workgroup computes a 64-token x 64-expert tile: each of its 4 waves takes a quarter of the
// 64-value K steps for all four 32 x 32 fragments (2 token x 2 expert fragments, so every
// operand row it loads feeds two fragments), and the quarters are added in LDS in a fixed order
// (quarter 0 + 1 + 2 + 3).  Operand rows past T or E are clamped copies whose results are not
// stored.

__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                       const float* __restrict__ bias, float* __restrict__ L, int T,
                                                       int d, int E) {
  __shared__ float part[4][4][16][64];  // [quarter][fragment][register][lane]
  const int wave = threadIdx.x >> 6, l = lane_id(), i = l & 31, h = l >> 5;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const uint16_t* pa[2];
  const uint16_t* pb[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    pa[f] = x + (size_t)min(t0 + 32 * f + i, T - 1) * d + 32 * h;
    pb[f] = wr + (size_t)min(e0 + 32 * f + i, E - 1) * d + 32 * h;
  }
  const int nsteps = d / 64, s0 = wave * nsteps / 4, s1 = (wave + 1) * nsteps / 4;
  v16f acc[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][g][v] = 0.0f;
  // The operands of step k + 1 are loaded before the matrix instructions of step k, so each
  // step's load latency overlaps the previous step's products (the summation order is unchanged).
  v8bf a[2][4], b[2][4], na[2][4], nb[2][4];
  auto load = [&](int k0, v8bf (&ra)[2][4], v8bf (&rb)[2][4]) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ra[f][s] = *(const v8bf*)(pa[f] + k0 + 8 * s);
        rb[f][s] = *(const v8bf*)(pb[f] + k0 + 8 * s);
      }
  };
  if (s0 < s1) load(64 * s0, a, b);
  for (int st = s0; st < s1; ++st) {
    if (st + 1 < s1) load(64 * (st + 1), na, nb);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g) acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f][s], b[g][s], acc[f][g], 0, 0, 0);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        a[f][s] = na[f][s];
        b[f][s] = nb[f][s];
      }
  }
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) part[wave][2 * f + g][v][l] = acc[f][g][v];
  __syncthreads();
  // wave w finishes fragment w: token fragment w / 2, expert fragment w % 2
  const int f = wave >> 1, g = wave & 1;
  const int e = e0 + 32 * g + i;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
    const float sum = ((part[0][wave][v][l] + part[1][wave][v][l]) + part[2][wave][v][l]) + part[3][wave][v][l];
    if (t < T && e < E) L[(size_t)t * E + e] = sum + (bias ? bias[e] : 0.0f);
  }
}

// ----------------------------------------------------------------------------- top-k
//
// One wave per token.  Experts are ranked by logit, best first; equal logits go to the lower
// expert index.  Weights: softmax over the k selected logits, or sigmoid scores normalised by
// their sum.  A NaN logit ranks as -inf, so every token still selects k distinct valid experts
// (the ranking is total); a non-finite logit also sets MOE_DEV_NONFINITE_LOGIT in the status word.

constexpr int kMaxPerLane = 8;  // E <= 512
constexpr int32_t kDevNonfiniteLogit = 2;  // MOE_DEV_NONFINITE_LOGIT

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ L, int T, int E, int k, int score,
                                              int32_t* __restrict__ idx, float* __restrict__ w,
                                              int32_t* __restrict__ status) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int l = lane_id();
  float v[kMaxPerLane];
  const int nper = (E + 63) / 64;
  bool nonfinite = false;
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    int e = l + 64 * q;
    float x = (q < nper && e < E) ? L[(size_t)t * E + e] : -INFINITY;
    if (q < nper && e < E && !isfinite(x)) nonfinite = true;
    v[q] = x == x ? x : -INFINITY;  // NaN ranks as -inf
  }
  if (__any(nonfinite) && l == 0) __hip_atomic_store(status, kDevNonfiniteLogit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t taken = 0;
  float sel_v[16];
  int sel_e[16];
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q) {
      int e = l + 64 * q;
      bool ok = q < nper && e < E && !((taken >> q) & 1u);
      if (ok && (v[q] > bv || (v[q] == bv && e < be))) {
        bv = v[q];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o);
      int oe = __shfl_xor(be, o);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be != 0x7FFFFFFF && (be & 63) == l) taken |= 1u << (be >> 6);
    sel_v[j] = bv;
    sel_e[j] = be;
  }
  float wsum = 0.0f, wj[16];
  for (int j = 0; j < k; ++j) {
    float z = score == 0 ? expf(sel_v[j] - sel_v[0]) : 1.0f / (1.0f + expf(-sel_v[j]));
    wj[j] = z;
    wsum += z;
  }
  for (int j = 0; j < k; ++j) {
    if (l == j) {
      idx[(size_t)t * k + j] = sel_e[j];
      w[(size_t)t * k + j] = wj[j] / wsum;
    }
  }
}

// ----------------------------------------------------------------------------- schedule
//
// Expert-major stable permutation of the T*k routed slots in four passes: per 64-token block
// counts; a wavefront scan of each expert's counts over the blocks (one wave per expert); a
// workgroup scan of the per-expert totals into the offset tables; and a scatter in which one
// thread per expert walks its block's tokens in order.  Shared experts own the rows after the
// routed ones (all T tokens, in order).

constexpr int kBlkTok = kSchedBlockTokens;

__global__ __launch_bounds__(256) void k_sched_hist(SchedBuild p) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kBlkTok;
  const int n = min(kBlkTok, p.T - t0) * p.k;  // the block's (token, slot) entries
  for (int q = threadIdx.x; q < n; q += blockDim.x) atomicAdd(&cnt[p.idx[(size_t)t0 * p.k + q]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) p.blkcnt[(size_t)blockIdx.x * p.E + e] = cnt[e];
}

// Inclusive prefix sum over the 64 lanes of a wave (wavefront scan: log2(64) shifted adds).
template <class T>
MOE_DEV T wave_incl_scan(T v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T u = __shfl_up(v, o);
    if (l >= o) v += u;
  }
  return v;
}

// One wave per expert: the expert's per-block counts (a column of blkcnt) are replaced by their
// exclusive prefix over blocks, 64 blocks per wavefront scan, and the total is the expert's
// row count.
__global__ __launch_bounds__(64) void k_sched_colscan(SchedBuild p, int nblk) {
  const int e = blockIdx.x, l = lane_id();
  int run = 0;
  for (int b0 = 0; b0 < nblk; b0 += 64) {
    const int b = b0 + l;
    const int c = b < nblk ? p.blkcnt[(size_t)b * p.E + e] : 0;
    const int incl = wave_incl_scan(c);
    if (b < nblk) p.blkcnt[(size_t)b * p.E + e] = run + incl - c;
    run += __shfl(incl, 63);
  }
  if (l == 0) p.counts[e] = run;
}

// One workgroup: exclusive prefixes over the experts (routed, then shared with T rows each) of
// the counts, the counts rounded up to 32 and to 128, the GEMM row tiles (of up to tile_rows
// rows) and the 64-token tiles, by wavefront scans within waves and one scan of the wave totals.
__global__ __launch_bounds__(1024) void k_sched_offsets(SchedBuild p) {
  __shared__ int64_t wsum[16][5];
  const int n_exp = p.E + p.S;
  const int i = threadIdx.x, l = lane_id(), w = i >> 6;
  int c = 0;
  if (i < p.E) c = p.counts[i];
  else if (i < n_exp) c = p.T;
  int64_t v[5] = {c, (c + 31) / 32 * 32, (c + 127) / 128 * 128, (c + p.tile_rows - 1) / p.tile_rows,
                  (c + 127) / 128 * 2};
  int64_t incl[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    incl[q] = wave_incl_scan(v[q]);
    if (l == 63) wsum[w][q] = incl[q];
  }
  __syncthreads();
  if (w == 0) {  // exclusive scan of the 16 wave totals, by lanes 0 .. 15
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int64_t t = l < 16 ? wsum[l][q] : 0;
      const int64_t in = wave_incl_scan(t);
      if (l < 16) wsum[l][q] = in - t;
    }
  }
  __syncthreads();
  int64_t ex[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) ex[q] = wsum[w][q] + incl[q] - v[q];
  if (i >= p.E && i < n_exp) p.counts[i] = c;
  if (i <= n_exp) {  // thread n_exp writes the totals (its own values are zero)
    p.offsets[i] = (int32_t)ex[0];
    p.poffsets[i] = (int32_t)ex[1];
    p.tok_off[i] = ex[2];
    p.tile_start[i] = (int32_t)ex[3];
    p.tile64[i] = (int32_t)ex[4];
  }
}

__global__ __launch_bounds__(256) void k_sched_scatter(SchedBuild p) {
  extern __shared__ int32_t sidx[];
  const int t0 = blockIdx.x * kBlkTok;
  const int ntok = min(kBlkTok, p.T - t0);
  for (int q = threadIdx.x; q < ntok * p.k; q += blockDim.x) sidx[q] = p.idx[(size_t)t0 * p.k + q];
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) {
    int row = p.offsets[e] + p.blkcnt[(size_t)blockIdx.x * p.E + e];
    for (int tl = 0; tl < ntok; ++tl) {
      for (int j = 0; j < p.k; ++j) {
        if (sidx[tl * p.k + j] == e) {
          int sid = (t0 + tl) * p.k + j;
          p.perm[row] = sid;
          p.pos[sid] = row;
          ++row;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_r, const float* bias, float* logits, int T,
                                int d, int E, hipStream_t st) {
  dim3 grid((T + 63) / 64, (E + 63) / 64);
  hipLaunchKernelGGL(k_router_logits, grid, dim3(256), 0, st, x, w_r, bias, logits, T, d, E);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int score, int32_t* idx, float* w,
                       int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, k, score, idx, w, status);
  return hipGetLastError();
}

hipError_t launch_schedule(const SchedBuild& p, hipStream_t st) {
  const int nblk = (p.T + kBlkTok - 1) / kBlkTok;
  hipLaunchKernelGGL(k_sched_hist, dim3(nblk), dim3(256), p.E * sizeof(int32_t), st, p);
  hipLaunchKernelGGL(k_sched_colscan, dim3(p.E), dim3(64), 0, st, p, nblk);
  hipLaunchKernelGGL(k_sched_offsets, dim3(1), dim3(1024), 0, st, p);
  hipLaunchKernelGGL(k_sched_scatter, dim3(nblk), dim3(256), kBlkTok * p.k * sizeof(int32_t), st, p);
  return hipGetLastError();
}

}  // namespace moe
