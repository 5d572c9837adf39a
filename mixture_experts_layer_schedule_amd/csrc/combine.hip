// Deterministic combine and the backward reductions around the experts.
//
// Expert results are pushed into one fixed slot per (token, selection) (push combine and push
// reverse-dispatch: knowledge card "Mixture-of-Kittens——面向NVL72的开源MoE训练megakernel",
// 方法/产品要点), so every sum here gathers a token's slots in the fixed order j = 0..k-1, then
// the shared experts: no atomics, bitwise identical on every run (一句话结论: deterministic).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// y[t, n] = sum_j w[t, j] Yslot[t, j, n] + sum_s Yslot[t, k + s, n]; 4 columns per thread.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ yslot, const float* __restrict__ w, int T,
                                                 int k, int S, int d, uint16_t* __restrict__ ybf,
                                                 float* __restrict__ yf) {
  const int64_t n4 = (int64_t)T * d / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n4; g += stride) {
    const int64_t t = g / (d / 4);
    const int64_t c = (g - t * (d / 4)) * 4;
    const float* base = yslot + t * (k + S) * d + c;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      float wj = w[t * k + j];
      v4f y = *(const v4f*)(base + (int64_t)j * d);
      acc[0] += wj * y[0]; acc[1] += wj * y[1]; acc[2] += wj * y[2]; acc[3] += wj * y[3];
    }
    for (int s = 0; s < S; ++s) {
      v4f y = *(const v4f*)(base + (int64_t)(k + s) * d);
      acc[0] += y[0]; acc[1] += y[1]; acc[2] += y[2]; acc[3] += y[3];
    }
    if (yf) *(v4f*)(yf + t * d + c) = acc;
    v2i o;
    o[0] = (int)((uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16));
    o[1] = (int)((uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16));
    *(v2i*)(ybf + t * d + c) = o;
  }
}

// Identity experts (a check of the dispatch-free combine path): every slot row of token t holds
// x[t] widened to float32 (exact); 4 columns per thread.
__global__ __launch_bounds__(256) void k_identity_slots(const uint16_t* __restrict__ x, int T, int slots, int d,
                                                        float* __restrict__ yslot) {
  const int64_t n4 = (int64_t)T * slots * (d / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n4; g += stride) {
    const int64_t row = g / (d / 4);  // t * slots + j
    const int64_t c = (g - row * (d / 4)) * 4;
    const int64_t t = row / slots;
    const v2i b = *(const v2i*)(x + t * d + c);
    v4f y;
    y[0] = __uint_as_float((uint32_t)b[0] << 16);
    y[1] = __uint_as_float((uint32_t)b[0] & 0xFFFF0000u);
    y[2] = __uint_as_float((uint32_t)b[1] << 16);
    y[3] = __uint_as_float((uint32_t)b[1] & 0xFFFF0000u);
    *(v4f*)(yslot + row * d + c) = y;
  }
}

// Per token: dw[t, j] = <dy[t], Yslot[t, j]> (reverse-combine of the weights), then the
// gradient of the selected logits.  One 256-thread workgroup per token: thread i holds dy at
// columns 4(i + 256m) in registers and reads each slot row with 16-byte loads, so a token's
// k + 1 rows stream at full width; the partial sums reduce in a fixed tree.
constexpr int kRbQuads = 8;  // column quads per thread and pass (d <= 8192 in one pass)

__global__ __launch_bounds__(256) void k_router_bwd(const uint16_t* __restrict__ dy, const float* __restrict__ yslot,
                                                    const float* __restrict__ L, const int32_t* __restrict__ idx,
                                                    const float* __restrict__ w, int E, int k, int S, int d, int score,
                                                    float* __restrict__ dw_out, float* __restrict__ dl_out) {
  __shared__ float part[16][4];
  __shared__ float dws[16];
  const int t = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int nq = d / 4;
  const uint16_t* dyr = dy + (size_t)t * d;
  const float* ys = yslot + (size_t)t * (k + S) * d;
  float acc[16];
  static_for<16>([&]<int j>() { acc[j] = 0.0f; });
  for (int q0 = 0; q0 < nq; q0 += 256 * kRbQuads) {
    v4f dv[kRbQuads];
    static_for<kRbQuads>([&]<int m>() {
      const int q = q0 + (int)threadIdx.x + 256 * m;
      dv[m] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
      if (q < nq) {
        const v2i b = *(const v2i*)(dyr + 4 * q);
        dv[m] = (v4f){__uint_as_float((uint32_t)b[0] << 16), __uint_as_float((uint32_t)b[0] & 0xFFFF0000u),
                      __uint_as_float((uint32_t)b[1] << 16), __uint_as_float((uint32_t)b[1] & 0xFFFF0000u)};
      }
    });
    static_for<16>([&]<int j>() {
      if (j < k) {
        v4f y[kRbQuads];
        static_for<kRbQuads>([&]<int m>() {
          const int q = q0 + (int)threadIdx.x + 256 * m;
          y[m] = q < nq ? *(const v4f*)(ys + (size_t)j * d + 4 * q) : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
        });
        static_for<kRbQuads>([&]<int m>() {
          acc[j] += dv[m][0] * y[m][0] + dv[m][1] * y[m][1] + dv[m][2] * y[m][2] + dv[m][3] * y[m][3];
        });
      }
    });
  }
  static_for<16>([&]<int j>() {
    if (j < k) {
      const float v = group_sum<64>(acc[j]);
      if (lane_id() == 0) part[j][wave] = v;
    }
  });
  __syncthreads();
  if ((int)threadIdx.x < k) {
    int j = threadIdx.x;
    dws[j] = (part[j][0] + part[j][1]) + (part[j][2] + part[j][3]);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float inner = 0.0f, ssum = 0.0f;
    for (int j = 0; j < k; ++j) inner += w[(size_t)t * k + j] * dws[j];
    if (score == 1)
      for (int j = 0; j < k; ++j) ssum += 1.0f / (1.0f + expf(-L[(size_t)t * E + idx[(size_t)t * k + j]]));
    for (int j = 0; j < k; ++j) {
      float wj = w[(size_t)t * k + j];
      float g;
      if (score == 0) {
        g = wj * (dws[j] - inner);
      } else {
        float sj = 1.0f / (1.0f + expf(-L[(size_t)t * E + idx[(size_t)t * k + j]]));
        g = sj * (1.0f - sj) * (dws[j] - inner) / ssum;
      }
      dw_out[(size_t)t * k + j] = dws[j];
      dl_out[(size_t)t * k + j] = g;
    }
  }
}

// dW_r[e, n] = sum over the expert's routed rows (increasing token order) of dL * x[t, n].  A
// thread owns 8 consecutive columns, so each routed row is one 16-byte load of x; the rows'
// indices and values are loaded 8 at a time ahead of the (in-order) accumulation.
__global__ __launch_bounds__(128) void k_router_wgrad(SchedView s, const float* __restrict__ dl,
                                                      const uint16_t* __restrict__ x, int d, float* __restrict__ dwr) {
  const int e = blockIdx.y;
  const int c8 = blockIdx.x * blockDim.x + threadIdx.x;  // columns [8 c8, 8 c8 + 8)
  if (c8 * 8 >= d) return;
  float acc[8];
  static_for<8>([&]<int c>() { acc[c] = 0.0f; });
  const int r0 = s.offsets[e], r1 = s.offsets[e + 1];
  for (int r = r0; r < r1; r += 8) {
    int sid[8];
    float dv[8];
    v4i xv[8];
    static_for<8>([&]<int u>() { sid[u] = r + u < r1 ? s.perm[r + u] : s.perm[r]; });
    static_for<8>([&]<int u>() {
      dv[u] = dl[sid[u]];
      xv[u] = *(const v4i*)(x + (size_t)(sid[u] / s.k) * d + 8 * c8);
    });
    static_for<8>([&]<int u>() {
      if (r + u < r1) {
        static_for<8>([&]<int c>() {
          const uint32_t wd = (uint32_t)xv[u][c >> 1];
          const float xf = __uint_as_float((c & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
          acc[c] += dv[u] * xf;
        });
      }
    });
  }
  float* o = dwr + (size_t)e * d + 8 * c8;
  *(v4f*)o = (v4f){acc[0], acc[1], acc[2], acc[3]};
  *(v4f*)(o + 4) = (v4f){acc[4], acc[5], acc[6], acc[7]};
}

// dx[t, n] = sum_j dXslot[t, j, n] + sum_s dXslot[t, k + s, n] + sum_j dL[t, j] W_r[idx[t, j], n].
__global__ __launch_bounds__(256) void k_dx_reduce(const float* __restrict__ dxslot, const float* __restrict__ dl,
                                                   const int32_t* __restrict__ idx, const uint16_t* __restrict__ wr,
                                                   int T, int k, int S, int d, uint16_t* __restrict__ dxbf,
                                                   float* __restrict__ dxf) {
  const int64_t n4 = (int64_t)T * d / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n4; g += stride) {
    const int64_t t = g / (d / 4);
    const int64_t c = (g - t * (d / 4)) * 4;
    const float* base = dxslot + t * (k + S) * d + c;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k + S; ++j) {
      v4f v = *(const v4f*)(base + (int64_t)j * d);
      acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
    }
    for (int j = 0; j < k; ++j) {
      float g2 = dl[t * k + j];
      const uint16_t* wrow = wr + (int64_t)idx[t * k + j] * d + c;
      v2i wv = *(const v2i*)wrow;
      acc[0] += g2 * __uint_as_float((uint32_t)wv[0] << 16);
      acc[1] += g2 * __uint_as_float((uint32_t)wv[0] & 0xFFFF0000u);
      acc[2] += g2 * __uint_as_float((uint32_t)wv[1] << 16);
      acc[3] += g2 * __uint_as_float((uint32_t)wv[1] & 0xFFFF0000u);
    }
    if (dxf) *(v4f*)(dxf + t * d + c) = acc;
    v2i o;
    o[0] = (int)((uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16));
    o[1] = (int)((uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16));
    *(v2i*)(dxbf + t * d + c) = o;
  }
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b > 256 * 64 ? 256 * 64 : (b < 1 ? 1 : b));
}

}  // namespace

hipError_t launch_identity_slots(const uint16_t* x, int T, int slots, int d, float* yslot, hipStream_t st) {
  hipLaunchKernelGGL(k_identity_slots, dim3(grid_for((int64_t)T * slots * d / 4)), dim3(256), 0, st, x, T, slots, d,
                     yslot);
  return hipGetLastError();
}

hipError_t launch_combine(const float* yslot, const float* w, int T, int k, int S, int d, uint16_t* y_bf16,
                          float* y_f32, hipStream_t st) {
  hipLaunchKernelGGL(k_combine, dim3(grid_for((int64_t)T * d / 4)), dim3(256), 0, st, yslot, w, T, k, S, d, y_bf16,
                     y_f32);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const uint16_t* dy, const float* yslot, const float* logits, const int32_t* idx,
                             const float* w, int T, int E, int k, int S, int d, int score, float* dw_out,
                             float* dl_out, hipStream_t st) {
  hipLaunchKernelGGL(k_router_bwd, dim3(T), dim3(256), 0, st, dy, yslot, logits, idx, w, E, k, S, d, score, dw_out,
                     dl_out);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const SchedView& s, const float* dl, const uint16_t* x, int d, int E, float* dw_r,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_router_wgrad, dim3((d / 8 + 127) / 128, E), dim3(128), 0, st, s, dl, x, d, dw_r);
  return hipGetLastError();
}

hipError_t launch_dx_reduce(const float* dxslot, const float* dl, const int32_t* idx, const uint16_t* w_r, int T,
                            int k, int S, int d, uint16_t* dx_bf16, float* dx_f32, hipStream_t st) {
  hipLaunchKernelGGL(k_dx_reduce, dim3(grid_for((int64_t)T * d / 4)), dim3(256), 0, st, dxslot, dl, idx, w_r, T, k, S,
                     d, dx_bf16, dx_f32);
  return hipGetLastError();
}

}  // namespace moe
