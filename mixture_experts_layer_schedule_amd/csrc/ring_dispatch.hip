// Ring token buffers for the pull dispatch (MOE_F_RING_DISPATCH), with streams and events.
//
// The pages' dispatch pulls the rows each expert needs into fixed-capacity ring buffers that are
// reused cyclically, with part of the GPU moving data while the rest runs the expert GEMMs and
// no CPU sizing buffers (knowledge card "Mixture-of-Kittens——面向NVL72的开源MoE训练megakernel",
// 方法/产品要点; article "Cursor 為 Composer 改造 MoE 訓練：MoK 點樣拆走跨 GPU 樽頸", section "MoK 將運算
// 同通訊塞入同一個核心").  Here the unit of the ring is a chunk, one GEMM row tile (up to
// chunk_rows rows of one expert), and a slot holds one chunk: chunk c lives in slot c % nslots.
// The chunks go in rounds of H consecutive chunks; for each round
//  * producer workgroups (producer_wgs of them, on a second stream) gather the round's rows of
//    xq / xs through the schedule into their slots (this file), and
//  * the gate/up GEMM (on the caller's stream) runs the round's chunks straight from the slots,
// ordered by events: a round's GEMM waits for its gather, and a round's gather waits for the
// GEMM of the last round that used the same slots.  With H = nslots / 2 one half of the ring
// fills while the GEMM reads the other.  Every kernel runs to completion on its own; nothing
// waits on the device and nothing is dropped at any capacity: every chunk has its round.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {

namespace {

// Round [chunk0, chunk0 + nchunks) of the chunks (those that exist: the schedule's row tiles):
// row r of chunk c <- xq row of its token, into slot c % nslots.  A wave takes kBatch
// consecutive (chunk, row) pairs at a time; its lanes look the batch's tokens up together (the
// tile-table search and perm are a chain of dependent loads, paid once per batch rather than
// once per row), then the wave copies the rows kRows at a time, each lane holding up to eight
// 16-byte pieces of each row in flight (a wave reads 1 KB of a row per instruction).  Pairs
// past a chunk's rows are skipped.
constexpr int kBatch = 16, kRows = 4, kPieces = 8;

__global__ __launch_bounds__(256) void k_ring_gather(SchedView s, const uint8_t* __restrict__ xq,
                                                     const uint8_t* __restrict__ xs, int d, uint8_t* __restrict__ ring,
                                                     uint8_t* __restrict__ ring_s, int slot_rows, int nslots,
                                                     int chunk0, int nchunks) {
  const int c1 = min(chunk0 + nchunks, s.tile_start[s.n_exp]);
  const int pairs = (c1 - chunk0) * slot_rows;
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * 4, wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n16 = d / 16, nsw = d / 128;  // 16-byte pieces and 4-byte scale words per row
  for (int q0 = wave * kBatch; q0 < pairs; q0 += nwaves * kBatch) {
    int tok = -1, dst = 0;  // lane j < kBatch: pair q0 + j
    if (lane < kBatch && q0 + lane < pairs) {
      const int q = q0 + lane, c = chunk0 + q / slot_rows, r = q - (q / slot_rows) * slot_rows;
      const RowTile rt = row_tile(s, c);
      if (r < rt.rows) {
        tok = row_token(s, rt.r0 + r);
        dst = (c % nslots) * slot_rows + r;
      }
    }
    for (int j0 = 0; j0 < kBatch; j0 += kRows) {
      int t[kRows], o[kRows];
      bool any = false;
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        t[u] = __builtin_amdgcn_readlane(tok, j0 + u);
        o[u] = __builtin_amdgcn_readlane(dst, j0 + u);
        any |= t[u] >= 0;
      }
      if (!any) continue;  // wave-uniform
      for (int i0 = 0; i0 < n16; i0 += 64 * kPieces) {
        v4i v[kRows][kPieces];
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
          const v4i* src = (const v4i*)(xq + (size_t)max(t[u], 0) * d);
#pragma unroll
          for (int p = 0; p < kPieces; ++p) {
            const int i = i0 + p * 64 + lane;
            if (t[u] >= 0 && i < n16) v[u][p] = src[i];
          }
        }
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
          v4i* dstp = (v4i*)(ring + (size_t)o[u] * d);
#pragma unroll
          for (int p = 0; p < kPieces; ++p) {
            const int i = i0 + p * 64 + lane;
            if (t[u] >= 0 && i < n16) dstp[i] = v[u][p];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        if (t[u] < 0) continue;
        const uint32_t* ss = (const uint32_t*)(xs + (size_t)t[u] * (d / 32));
        uint32_t* ds = (uint32_t*)(ring_s + (size_t)o[u] * (d / 32));
        for (int i = lane; i < nsw; i += 64) ds[i] = ss[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_ring_gather(const SchedView& s, const uint8_t* xq, const uint8_t* xs, int d, uint8_t* ring,
                              uint8_t* ring_s, int slot_rows, int nslots, int chunk0, int nchunks, int producers,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_ring_gather, dim3(producers), dim3(256), 0, st, s, xq, xs, d, ring, ring_s, slot_rows, nslots,
                     chunk0, nchunks);
  return hipGetLastError();
}

}  // namespace moe
