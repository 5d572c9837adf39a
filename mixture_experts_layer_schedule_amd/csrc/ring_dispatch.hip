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
// row r of chunk c <- xq row of its token, into slot c % nslots.  The (chunk, row) pairs are
// dealt to the workgroups in turn; a pair past the chunk's rows is skipped.
__global__ __launch_bounds__(256) void k_ring_gather(SchedView s, const uint8_t* __restrict__ xq,
                                                     const uint8_t* __restrict__ xs, int d, uint8_t* __restrict__ ring,
                                                     uint8_t* __restrict__ ring_s, int slot_rows, int nslots,
                                                     int chunk0, int nchunks) {
  const int c1 = min(chunk0 + nchunks, s.tile_start[s.n_exp]);
  const int pairs = (c1 - chunk0) * slot_rows;
  for (int q = blockIdx.x; q < pairs; q += gridDim.x) {
    const int c = chunk0 + q / slot_rows, r = q - (q / slot_rows) * slot_rows;
    const RowTile rt = row_tile(s, c);
    if (r >= rt.rows) continue;  // workgroup-uniform
    const int tok = row_token(s, rt.r0 + r);
    const size_t dst_row = (size_t)(c % nslots) * slot_rows + r;
    const v4i* src = (const v4i*)(xq + (size_t)tok * d);
    v4i* dst = (v4i*)(ring + dst_row * d);
    for (int i = threadIdx.x; i < d / 16; i += blockDim.x) dst[i] = src[i];
    const uint32_t* ss = (const uint32_t*)(xs + (size_t)tok * (d / 32));
    uint32_t* ds = (uint32_t*)(ring_s + dst_row * (d / 32));
    for (int i = threadIdx.x; i < d / 128; i += blockDim.x) ds[i] = ss[i];
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
