// Persistent dispatch + gate/up kernel fed through fixed-capacity ring token buffers.
//
// The pages' megakernel splits its SMs between data movement and matrix work, pulls the tokens
// each expert needs (pull-based dispatch), and stages them in fixed-capacity ring buffers that
// are reused cyclically, so no CPU sizes buffers per round and no token is dropped (knowledge
// card "Mixture-of-Kittens——面向NVL72的开源MoE训练megakernel", 方法/产品要点; article "Cursor 為
// Composer 改造 MoE 訓練…", section "MoK 將運算同通訊塞入同一個核心"; commentary "Cursor 开源
// MoK…", section 通信压到18微秒).  On one MI355X the same structure is:
//
//  * producer workgroups gather the quantised rows of each chunk (one GEMM row tile: up to 256
//    of one expert's rows in schedule order) from xq into a ring slot, release them at device
//    scope and publish the slot's lap number;
//  * consumer workgroups run the MXFP8 gate/up GEMM tiles of each chunk straight out of the ring
//    slot (same tile code as the direct kernel, with device-coherent loads of the slot, so no
//    cache has to be invalidated) and count finished work units per slot;
//  * a producer reuses a slot only when every work unit of the chunk it held has been counted.
//
// Chunks are produced in order and each role walks its work in increasing order, so with every
// workgroup co-resident (the grid never exceeds the device's resident capacity) the pipeline
// cannot deadlock.  Every wait is bounded: past `spin_limit` polls the kernel records a status
// code and all workgroups leave their loops.  Results are bitwise those of the direct kernel.
//
// Status: not launched.  The first device run of this consumer (tile code out of line in
// consume_tile) ended in a memory fault whose cause has not been identified; a host build of the
// kernel finds every access in bounds.  MOE_F_RING_DISPATCH runs the stream-ordered ring of
// ring_dispatch.hip instead (producer and consumer kernels ordered by events, no device waits).
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCopyUnroll = 8;
constexpr int kTilesPerUnit = 4;  // consecutive 128-column tiles of one chunk per consumer work unit

// Polls with relaxed device-coherent loads (an acquire per poll would invalidate the cache
// hierarchy on every iteration).
MOE_DEV bool wait_ge(int32_t* p, int32_t target, int32_t* abort_flag, int32_t* status, int spin_limit) {
  int it = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    __builtin_amdgcn_s_sleep(2);
    if (++it > spin_limit) {
      __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  return true;
}

__global__ void k_zero_flags(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Consumer tile: rows of one chunk straight out of its ring slot (device-coherent loads, cache
// policy sc1), 128 I columns of gate and up, SwiGLU + quantisation epilogue.
template <int F>
MOE_DEV void ring_tile(const RingArgs& p, uint8_t* lds, const uint8_t* ring, const uint8_t* rings,
                       const RowTile& rt, int n0) {
  const int d = p.d, I = p.I;
  const uint8_t* w1 = p.w1q + (size_t)rt.e * 2 * I * d;
  const uint8_t* w1s = p.w1s + (size_t)rt.e * 2 * I * (d / 32);
  const int last = rt.rows - 1;
  TileLoads<F> L;
  L.init(ring, [&](int r) { return ring + (size_t)min(r, last) * d; },
         w1, [&](int r) { return w1 + (size_t)gateup_brow(r, n0, I) * d; },
         rings, [&](int r) { return rings + (size_t)min(r, last) * (d / 32); },
         w1s, [&](int r) { return w1s + (size_t)gateup_brow(r, n0, I) * (d / 32); });
  v16f acc[F][2];
  mainloop<F, 2, 16>(lds, L, d / KS, acc);
  gateup_epilogue<F>(acc, rt.r0, rt.rows, n0, I, p.g, p.u, p.hq, p.hs);
}

// One consumer tile, kept out of line: inlined into the persistent loop, its per-lane address
// arithmetic for every row-fragment count would be hoisted out of the loop and spilled.
__device__ __attribute__((noinline)) void consume_tile(const RingArgs& p, uint8_t* lds, const uint8_t* ring,
                                                       const uint8_t* rings, RowTile rt, int n0) {
  switch ((rt.rows + 31) >> 5) {
    case 1: ring_tile<1>(p, lds, ring, rings, rt, n0); break;
    case 2: ring_tile<2>(p, lds, ring, rings, rt, n0); break;
    case 3: ring_tile<3>(p, lds, ring, rings, rt, n0); break;
    case 4: ring_tile<4>(p, lds, ring, rings, rt, n0); break;
    case 5: ring_tile<5>(p, lds, ring, rings, rt, n0); break;
    case 6: ring_tile<6>(p, lds, ring, rings, rt, n0); break;
    case 7: ring_tile<7>(p, lds, ring, rings, rt, n0); break;
    default: ring_tile<8>(p, lds, ring, rings, rt, n0); break;
  }
}

__global__ __launch_bounds__(256, 1) void k_ring_gateup(RingArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_ok;
  const SchedView& s = p.s;
  const int n_chunks = s.tile_start[s.n_exp];  // one chunk per row tile
  const int NT = p.I / 128;
  const int units = (NT + kTilesPerUnit - 1) / kTilesPerUnit;  // consumer work units per chunk
  const int d = p.d;
  const size_t slot_bytes = (size_t)TM * d;
  const size_t slot_sbytes = (size_t)TM * (d / 32);

  if ((int)blockIdx.x < p.producers) {
    // ------------------------------------------------------------------ producer
    for (int i = blockIdx.x; i < n_chunks; i += p.producers) {
      const int slot = i % p.nslots, lap = i / p.nslots;
      if (threadIdx.x == 0) s_ok = lap == 0 || wait_ge(p.done + slot, lap * units, p.abort_flag, p.status, p.spin_limit);
      __syncthreads();
      if (!s_ok) return;
      // the slot's previous readers are done (their loads completed before they counted)
      const RowTile rt = row_tile(s, i);
      const int rows = max(rt.rows, 0);
      uint8_t* dst = p.ring + (size_t)slot * slot_bytes;
      uint8_t* dsts = p.ring_s + (size_t)slot * slot_sbytes;
      // 16-byte pieces, kCopyUnroll loads in flight per lane before their stores
      const int c16 = d / 16;
      const int n16 = rows * c16;
      for (int base = threadIdx.x; base < n16; base += blockDim.x * kCopyUnroll) {
        v4i buf[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
          const int c = base + u * blockDim.x;
          if (c < n16) {
            const int row = c / c16, col = c - row * c16;
            buf[u] = *(const v4i*)(p.xq + (size_t)row_token(s, rt.r0 + row) * d + col * 16);
          }
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
          const int c = base + u * blockDim.x;
          if (c < n16) {
            const int row = c / c16, col = c - row * c16;
            *(v4i*)(dst + (size_t)row * d + col * 16) = buf[u];
          }
        }
      }
      const int c4 = d / 128;  // 4-byte words of one row's scales
      for (int c = threadIdx.x; c < rows * c4; c += blockDim.x) {
        const int row = c / c4, col = c - row * c4;
        const uint32_t* src = (const uint32_t*)(p.xs + (size_t)row_token(s, rt.r0 + row) * (d / 32));
        ((uint32_t*)(dsts + (size_t)row * (d / 32)))[col] = src[col];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(p.ready + slot, lap + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // -------------------------------------------------------------------- consumer
  const int cid = blockIdx.x - p.producers;
  const int n_cons = gridDim.x - p.producers;
  // work unit = (chunk, group of up to kTilesPerUnit consecutive 128-column tiles)
  for (int tau = cid; tau < n_chunks * units; tau += n_cons) {
    const int i = tau / units, ug = tau - i * units;
    const int slot = i % p.nslots, lap = i / p.nslots;
    __syncthreads();  // every wave is done with the LDS buffers and s_ok of the previous unit
    if (threadIdx.x == 0) s_ok = wait_ge(p.ready + slot, lap + 1, p.abort_flag, p.status, p.spin_limit);
    __syncthreads();
    if (!s_ok) return;
    // no cache invalidation: the slot is read below with device-coherent loads only
    const RowTile rt = row_tile(s, i);
    const uint8_t* ring = p.ring + (size_t)slot * slot_bytes;
    const uint8_t* rings = p.ring_s + (size_t)slot * slot_sbytes;
    if (rt.rows > 0) {
      for (int nt = ug * kTilesPerUnit; nt < min(NT, (ug + 1) * kTilesPerUnit); ++nt) {
        if (nt > ug * kTilesPerUnit) __syncthreads();  // previous tile's LDS reads are done
        consume_tile(p, lds, ring, rings, rt, nt * 128);
      }
    }
    // relaxed: the count only has to follow this unit's reads of the slot, which have completed
    if (threadIdx.x == 0) __hip_atomic_fetch_add(p.done + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct RingLaunch {
  int max_resident = 0;
};
RingLaunch g_ring;

}  // namespace

hipError_t ring_init() {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev))) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev))) return e;
  const int bytes = (int)gemm_lds_bytes();
  if ((e = hipFuncSetAttribute((const void*)k_ring_gateup, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)))
    return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_ring_gateup, 256, bytes))) return e;
  g_ring.max_resident = cus * per_cu;
  return hipSuccess;
}

int ring_max_resident() { return g_ring.max_resident; }

hipError_t launch_ring_gateup(const RingArgs& a, hipStream_t st) {
  const int grid = g_ring.max_resident;
  if (grid <= a.producers) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_zero_flags, dim3(1), dim3(256), 0, st, a.flags, a.n_flags);
  hipLaunchKernelGGL(k_ring_gateup, dim3(grid), dim3(256), gemm_lds_bytes(), st, a);
  return hipGetLastError();
}

}  // namespace moe
