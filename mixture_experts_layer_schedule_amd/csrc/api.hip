// Host side of the C ABI: validation, buffer layout, kernel sequence.  Nothing here blocks the
// host or allocates device memory; every launch goes to the caller's stream.
#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Dims {
  int64_t T, d, E, k, I, S, NX, R, RS, nblk, ld_tok, tiles_bound, tile64_bound;
  int64_t ring_rows, nslots, producers;
  int64_t tile_rows;  // rows per GEMM row tile at most (chunk_rows)
  bool unfused;
};

constexpr int kChunkRows = 256;      // rows per ring slot: one GEMM row tile at most
constexpr int kDefaultRingRows = 16384;
constexpr int kDefaultProducers = 128;

Dims dims(const moe_config& c) {
  Dims m;
  m.T = c.T; m.d = c.d; m.E = c.E; m.k = c.k; m.I = c.inter; m.S = c.n_shared;
  m.NX = m.E + m.S;
  m.R = m.T * m.k;
  m.RS = m.R + m.S * m.T;
  m.nblk = (m.T + kSchedBlockTokens - 1) / kSchedBlockTokens;
  m.ld_tok = (int64_t)up((size_t)(m.RS + 127 * m.NX), 128);
  m.tile_rows = c.chunk_rows ? c.chunk_rows : kChunkRows;
  m.tiles_bound = m.RS / m.tile_rows + m.NX + 1;  // sum over experts of ceil(count / tile_rows)
  m.tile64_bound = m.ld_tok / 64;
  // the ring buffer exists only for the ring dispatch
  const int64_t ring_rows = !(c.flags & MOE_F_RING_DISPATCH) ? 0 : c.ring_rows ? c.ring_rows : kDefaultRingRows;
  m.ring_rows = ring_rows;
  m.nslots = ring_rows / m.tile_rows;  // a slot holds one chunk: one row tile
  m.producers = c.producer_wgs ? c.producer_wgs : kDefaultProducers;
  m.unfused = (c.flags & MOE_F_UNFUSED) != 0;
  return m;
}

constexpr uint32_t kKnownFlags =
    MOE_F_DIRECT_GATHER | MOE_F_RING_DISPATCH | MOE_F_SERIAL_BWD | MOE_F_IDENTITY_EXPERTS | MOE_F_FORWARD_ONLY |
    MOE_F_UNFUSED | MOE_F_DW_BF16;

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_EINVAL;
  if (c->T < 1 || c->d < 128 || c->d % 128 || c->inter < 128 || c->inter % 128) return MOE_ESHAPE;
  if (c->k < 1 || c->k > 16 || c->E < c->k || c->E > 512) return MOE_ESHAPE;
  if (c->n_shared < 0 || c->n_shared > 1) return MOE_ESHAPE;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (c->flags & ~kKnownFlags) return MOE_EINVAL;
  if ((c->flags & MOE_F_DIRECT_GATHER) && (c->flags & MOE_F_RING_DISPATCH)) return MOE_EINVAL;
  // ring capacity and producer workgroups act on the ring dispatch only
  if (!(c->flags & MOE_F_RING_DISPATCH) && (c->ring_rows || c->producer_wgs)) return MOE_EINVAL;
  if (c->ring_rows < 0 || c->producer_wgs < 0 || c->producer_wgs > 128) return MOE_ESHAPE;
  // rows per GEMM row tile (every path; a ring slot holds one tile)
  if (c->chunk_rows < 0 || c->chunk_rows > kChunkRows || c->chunk_rows % 32) return MOE_ESHAPE;
  const int64_t slot_rows = c->chunk_rows ? c->chunk_rows : kChunkRows;
  if (c->ring_rows && (c->ring_rows < slot_rows || c->ring_rows % slot_rows)) return MOE_ESHAPE;
  const int64_t RS = (int64_t)c->T * c->k + (int64_t)c->n_shared * c->T;
  if (RS >= (1ll << 30)) return MOE_ESHAPE;
  // operands addressed with 32-bit byte offsets from one base: the gathered activations
  // (xq, dyq: T*d), one expert's weights (2I*d) and the token-axis operands of the weight
  // gradients (up to 256 rows of stride ld_tok)
  if ((int64_t)c->T * c->d >= (1ll << 32)) return MOE_ESHAPE;
  if (2 * (int64_t)c->inter * c->d >= (1ll << 32)) return MOE_ESHAPE;
  if (dims(*c).ld_tok >= (1ll << 24)) return MOE_ESHAPE;
  if (c->flags & MOE_F_UNFUSED) {
    // the forward baseline only (no transposed weights for a backward pass), with real experts
    if (!(c->flags & MOE_F_FORWARD_ONLY) || (c->flags & MOE_F_IDENTITY_EXPERTS)) return MOE_EINVAL;
    if (RS * c->d >= (1ll << 32)) return MOE_ESHAPE;  // the permuted rows, one 32-bit offset base
  }
  return MOE_OK;
}

// Sequential layout builder.
struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = up(off + bytes, kAlign);
    return o;
  }
};

moe_saved_layout saved_layout(const Dims& m, uint32_t flags) {
  moe_saved_layout s{};
  Layout L;
  s.logits = L.take(4 * m.T * m.E);
  s.idx = L.take(4 * m.T * m.k);
  s.w = L.take(4 * m.T * m.k);
  s.counts = L.take(4 * m.NX);
  s.offsets = L.take(4 * (m.NX + 1));
  s.poffsets = L.take(4 * (m.NX + 1));
  s.tok_off = L.take(8 * (m.NX + 1));
  s.tile_start = L.take(4 * (m.NX + 1));
  s.tile64 = L.take(4 * (m.NX + 1));
  s.perm = L.take(4 * m.R);
  s.pos = L.take(4 * m.R);
  s.xq = L.take(m.T * m.d);
  s.xs = L.take(m.T * m.d / 32);
  s.g = L.take(4 * m.RS * m.I);
  s.u = L.take(4 * m.RS * m.I);
  s.hq = L.take(m.RS * m.I);
  s.hs = L.take(m.RS * m.I / 32);
  s.yslot = L.take(4 * m.T * (m.k + m.S) * m.d);
  const bool wt = !(flags & (MOE_F_FORWARD_ONLY | MOE_F_IDENTITY_EXPERTS));
  const size_t wbytes = wt ? (size_t)(m.NX * 2 * m.I * m.d) : 0;
  s.w1t = L.take(wbytes);
  s.w1ts = L.take(wbytes / 32);
  s.w2t = L.take(wbytes / 2);
  s.w2ts = L.take(wbytes / 64);
  s.total = L.off;
  return s;
}

moe_workspace_layout work_layout(const Dims& m) {
  moe_workspace_layout w{};
  Layout L;
  w.status = L.take(64);
  // sized by the capacity alone (the most slots any row-tile height gives for the flags), so
  // that one workspace serves every chunk_rows
  w.ring = L.take(m.ring_rows * m.d);
  w.ring_s = L.take(m.ring_rows * m.d / 32);
  w.ring_flags = L.take(4 * (2 * (m.ring_rows / 32) + 1));
  w.blkcnt = L.take(4 * m.nblk * m.E);
  w.dyq = L.take(m.T * m.d);
  w.dys = L.take(m.T * m.d / 32);
  w.dw = L.take(4 * m.T * m.k);
  w.dl = L.take(4 * m.T * m.k);
  w.dguq = L.take(m.RS * 2 * m.I);
  w.dgus = L.take(m.RS * 2 * m.I / 32);
  w.dxslot = L.take(4 * m.T * (m.k + m.S) * m.d);
  w.xt = L.take(m.d * m.ld_tok);
  w.xts = L.take(m.d * m.ld_tok / 32);
  w.ht = L.take(m.I * m.ld_tok);
  w.hts = L.take(m.I * m.ld_tok / 32);
  w.dyt = L.take(m.d * m.ld_tok);
  w.dyts = L.take(m.d * m.ld_tok / 32);
  w.dgut = L.take(2 * m.I * m.ld_tok);
  w.dguts = L.take(2 * m.I * m.ld_tok / 32);
  w.xp = L.take(m.unfused ? m.RS * m.d : 0);
  w.xps = L.take(m.unfused ? m.RS * m.d / 32 : 0);
  w.yrows = L.take(m.unfused ? 4 * m.RS * m.d : 0);
  w.tok_stride = (size_t)m.ld_tok;
  w.total = L.off;
  return w;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

template <class T>
T* at(void* base, size_t off) { return (T*)((char*)base + off); }
template <class T>
const T* at(const void* base, size_t off) { return (const T*)((const char*)base + off); }

// Optional phase timing (measurement only): events recorded after each phase.
hipEvent_t* g_events = nullptr;
int g_n_events = 0;

inline void mark(hipStream_t st, int phase) {
  if (g_events && phase < g_n_events) hipEventRecord(g_events[phase], st);
}

std::once_flag g_init_once;
hipError_t g_init_err = hipSuccess;

moe_status ensure_init() {
  std::call_once(g_init_once, [] {
    g_init_err = gemm_init();
    if (g_init_err == hipSuccess) g_init_err = ring_init();
  });
  return g_init_err == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

// Extra streams of each device, with fork / join events around their work: kBranchStream runs
// the backward's independent branch, kRingStream the ring dispatch's producers (its own, so the
// backward's producers never queue behind that branch), kRingConsumerStream every other round
// of the ring's GEMM.  One set per host thread and device (created on first use, default
// priority, kept until the process ends), so calls from different threads never share events.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ok = false, tried = false;
};
constexpr int kMaxDevices = 64;
constexpr int kBranchStream = 0, kRingStream = 1, kRingConsumerStream = 2;
thread_local SideStream t_side[kMaxDevices][3];

// Events that order the ring dispatch's rounds, per host thread and device (created on first
// use, kept until the process ends).
struct RingEvents {
  std::vector<hipEvent_t> prod, cons;
  bool ensure(size_t n) {
    while (prod.size() < n) {
      hipEvent_t a = nullptr, b = nullptr;
      if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess) return false;
      if (hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
        hipEventDestroy(a);
        return false;
      }
      prod.push_back(a);
      cons.push_back(b);
    }
    return true;
  }
};
thread_local RingEvents t_ring_events[kMaxDevices];

SideStream* side_stream(int which) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& s = t_side[dev][which];
  if (!s.tried) {
    s.tried = true;
    s.ok = hipStreamCreateWithFlags(&s.st, hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&s.join, hipEventDisableTiming) == hipSuccess;
  }
  return s.ok ? &s : nullptr;
}

#define MOE_TRY(expr)                      \
  do {                                     \
    if ((expr) != hipSuccess) return MOE_ELAUNCH; \
  } while (0)

SchedView sched_view(const void* saved, const moe_saved_layout& sl, const Dims& m) {
  SchedView v;
  v.perm = at<int32_t>(saved, sl.perm);
  v.offsets = at<int32_t>(saved, sl.offsets);
  v.tile_start = at<int32_t>(saved, sl.tile_start);
  v.n_exp = (int)m.NX;
  v.R = (int)m.R;
  v.T = (int)m.T;
  v.k = (int)m.k;
  v.S = (int)m.S;
  return v;
}

// Static scratch of moe_fwd_noalloc: the status word and the schedule's per-block expert counts,
// in a file-scope device array (each GPU the library runs on holds its own copy until the
// process ends).  Host code never uses the array's name as an address: the address of each
// device's copy comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t noalloc_scratch_bytes(const Dims& m) { return kAlign + (size_t)4 * m.nblk * m.E; }

uint8_t* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

moe_status device_scratch(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ELAUNCH;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ELAUNCH;
    g_scratch_ptr[dev] = (uint8_t*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The forward pass over the caller's buffers and a scratch descriptor (the workspace's, or the
// library's static scratch for moe_fwd_noalloc).
struct FwdScratch {
  int32_t* status;      // device status word
  int32_t* blkcnt;      // [ceil(T/64), E] per-block expert counts
  uint8_t *ring, *ring_s;
  int32_t* ring_flags;
  uint8_t *xp = nullptr, *xps = nullptr;  // unfused forward: rows in expert order
  float* yrows = nullptr;
};

// Ring dispatch of the rows one grouped GEMM pulls (forward gate/up: xq; backward dgrad-down:
// dYq).  Chunks (row tiles) go in rounds of H = nslots / 2, chunk c in slot c % nslots.  Round
// r's gather (producers on the ring stream) waits for the GEMM of round r - lag, the last round
// whose chunks used its slots (lag = nslots / H, so the rounds in between use others); round r's
// GEMM, launched by consume(chunk0, nchunks, stream), waits for its gather.  With lag >= 2 the
// GEMM rounds alternate between the caller's stream and a consumer stream of the library's, so
// that two rounds' GEMMs (on disjoint slots) share the GPU; the caller's stream waits for the
// consumer stream's last round at the end.  While the caller's stream is being captured into a
// graph the GEMM rounds all stay on the caller's stream: the capture of a step whose rounds used
// both consumer streams ended the process (DeepSeek-V3 shape; cause not found), and the
// one-consumer schedule captures and replays bit for bit.  The host bounds the chunk count by
// tiles_bound; rounds past the schedule's real count find no chunks and return.  Without
// overlap (or without the ring stream) everything runs in launch order on the caller's stream.
template <class Consume>
moe_status ring_rounds(const Dims& m, const SchedView& sv, const uint8_t* q, const uint8_t* qs, uint8_t* ring,
                       uint8_t* ring_s, bool overlap, hipStream_t stream, Consume consume) {
  const int nslots = (int)m.nslots, H = std::max(1, nslots / 2);
  const int lag = nslots / H;
  const int rounds = (int)((m.tiles_bound + H - 1) / H);
  SideStream* side = overlap ? side_stream(kRingStream) : nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  bool capturing = true;  // when the query fails: the schedule that is known to capture
  if (hipStreamIsCapturing(stream, &cap) == hipSuccess) capturing = cap != hipStreamCaptureStatusNone;
  else (void)hipGetLastError();  // leave no error behind for the launch checks
  SideStream* cons2 = side && lag >= 2 && !capturing ? side_stream(kRingConsumerStream) : nullptr;
  int dev = 0;
  MOE_TRY(hipGetDevice(&dev));
  RingEvents& ev = t_ring_events[dev % kMaxDevices];
  const size_t K = (size_t)lag + 2;  // event r % K is recorded again only after round r - lag's wait
  if (side && !ev.ensure(K)) return MOE_ELAUNCH;
  hipStream_t ps = side ? side->st : stream;
  const hipStream_t cs[2] = {stream, cons2 ? cons2->st : stream};
  if (side) {
    MOE_TRY(hipEventRecord(side->fork, stream));  // the pulled rows and the schedule are ready
    MOE_TRY(hipStreamWaitEvent(ps, side->fork, 0));
    if (cons2) MOE_TRY(hipStreamWaitEvent(cs[1], side->fork, 0));
  }
  for (int r = 0; r < rounds; ++r) {
    const hipStream_t c = cs[r & 1];
    if (side && r >= lag) MOE_TRY(hipStreamWaitEvent(ps, ev.cons[(r - lag) % K], 0));
    MOE_TRY(launch_ring_gather(sv, q, qs, (int)m.d, ring, ring_s, (int)m.tile_rows, nslots, r * H, H,
                               (int)m.producers, ps));
    if (side) {
      MOE_TRY(hipEventRecord(ev.prod[r % K], ps));
      MOE_TRY(hipStreamWaitEvent(c, ev.prod[r % K], 0));
    }
    MOE_TRY(consume(r * H, H, c));
    if (side) MOE_TRY(hipEventRecord(ev.cons[r % K], c));
  }
  if (cons2) {  // the consumer stream's rounds are all done before the caller's next kernel
    MOE_TRY(hipEventRecord(cons2->join, cs[1]));
    MOE_TRY(hipStreamWaitEvent(stream, cons2->join, 0));
  }
  return MOE_OK;
}

moe_status forward_impl(const moe_config* cfg, const Dims& m, const moe_saved_layout& sl, const void* x,
                        const void* w_router, const float* router_bias, const uint8_t* w1q, const uint8_t* w1s,
                        const uint8_t* w2q, const uint8_t* w2s, void* y_bf16, float* y_f32, void* saved,
                        const FwdScratch& sc, hipStream_t stream) {
  const int d = (int)m.d, I = (int)m.I;
  const bool want_wt = !(cfg->flags & MOE_F_FORWARD_ONLY);

  uint8_t* xq = at<uint8_t>(saved, sl.xq);
  uint8_t* xs = at<uint8_t>(saved, sl.xs);
  float* logits = at<float>(saved, sl.logits);
  int32_t* idx = at<int32_t>(saved, sl.idx);
  float* w = at<float>(saved, sl.w);
  int32_t* status = sc.status;

  mark(stream, MOE_PH_FWD_BEGIN);
  MOE_TRY(launch_quant_rows(x, 0, m.T, m.d, xq, xs, stream));
  mark(stream, MOE_PH_QUANT_X);
  MOE_TRY(launch_router_logits((const uint16_t*)x, (const uint16_t*)w_router, router_bias, logits, (int)m.T, d,
                               (int)m.E, stream));
  mark(stream, MOE_PH_ROUTER);
  MOE_TRY(launch_topk(logits, (int)m.T, (int)m.E, (int)m.k, cfg->score_fn, idx, w, status, stream));

  SchedBuild sb;
  sb.idx = idx;
  sb.blkcnt = sc.blkcnt;
  sb.counts = at<int32_t>(saved, sl.counts);
  sb.offsets = at<int32_t>(saved, sl.offsets);
  sb.poffsets = at<int32_t>(saved, sl.poffsets);
  sb.tok_off = at<int64_t>(saved, sl.tok_off);
  sb.tile_start = at<int32_t>(saved, sl.tile_start);
  sb.tile64 = at<int32_t>(saved, sl.tile64);
  sb.perm = at<int32_t>(saved, sl.perm);
  sb.pos = at<int32_t>(saved, sl.pos);
  sb.T = (int)m.T;
  sb.E = (int)m.E;
  sb.k = (int)m.k;
  sb.S = (int)m.S;
  sb.tile_rows = (int)m.tile_rows;
  mark(stream, MOE_PH_TOPK);
  MOE_TRY(launch_schedule(sb, stream));
  mark(stream, MOE_PH_SCHEDULE);

  if (cfg->flags & MOE_F_IDENTITY_EXPERTS) {  // combine check: x in every slot row, then the combine
    float* yslot = at<float>(saved, sl.yslot);
    MOE_TRY(launch_identity_slots((const uint16_t*)x, (int)m.T, (int)(m.k + m.S), d, yslot, stream));
    mark(stream, MOE_PH_GATEUP);
    mark(stream, MOE_PH_DOWN);
    MOE_TRY(launch_combine(yslot, w, (int)m.T, (int)m.k, (int)m.S, d, (uint16_t*)y_bf16, y_f32, stream));
    mark(stream, MOE_PH_COMBINE);
    return MOE_OK;
  }

  const SchedView sv = sched_view(saved, sl, m);
  if (m.unfused) {
    // the conventional pipeline: permute, gate/up GEMM (G, U), SwiGLU + quantisation, down GEMM
    // (rows in expert order), unpermute, combine; every boundary through HBM
    MOE_TRY(launch_permute_rows(sv, xq, xs, d, (int)m.RS, sc.xp, sc.xps, stream));
    GateUpArgs ga{};
    ga.s = sv;
    ga.xq = sc.xp;
    ga.xs = sc.xps;
    ga.contiguous = 1;
    ga.w1q = w1q;
    ga.w1s = w1s;
    ga.g = at<float>(saved, sl.g);
    ga.u = at<float>(saved, sl.u);
    ga.d = d;
    ga.I = I;
    MOE_TRY(launch_gemm_gateup(ga, (int)m.tiles_bound, stream));
    mark(stream, MOE_PH_GATEUP);
    uint8_t* hq = at<uint8_t>(saved, sl.hq);
    uint8_t* hs = at<uint8_t>(saved, sl.hs);
    MOE_TRY(launch_swiglu_quant(ga.g, ga.u, (int)m.RS, I, hq, hs, stream));
    DownArgs da{};
    da.s = sv;
    da.hq = hq;
    da.hs = hs;
    da.w2q = w2q;
    da.w2s = w2s;
    da.yrows = sc.yrows;
    da.d = d;
    da.I = I;
    MOE_TRY(launch_gemm_down(da, (int)m.tiles_bound, stream));
    float* yslot = at<float>(saved, sl.yslot);
    MOE_TRY(launch_unpermute_rows(sv, sc.yrows, (int)m.RS, d, yslot, stream));
    mark(stream, MOE_PH_DOWN);
    MOE_TRY(launch_combine(yslot, w, (int)m.T, (int)m.k, (int)m.S, d, (uint16_t*)y_bf16, y_f32, stream));
    mark(stream, MOE_PH_COMBINE);
    return MOE_OK;
  }
  GateUpArgs ga{};
  ga.s = sv;
  ga.xq = xq;
  ga.xs = xs;
  ga.w1q = w1q;
  ga.w1s = w1s;
  ga.g = at<float>(saved, sl.g);
  ga.u = at<float>(saved, sl.u);
  ga.hq = at<uint8_t>(saved, sl.hq);
  ga.hs = at<uint8_t>(saved, sl.hs);
  ga.w1t = want_wt ? at<uint8_t>(saved, sl.w1t) : nullptr;
  ga.w1ts = want_wt ? at<uint8_t>(saved, sl.w1ts) : nullptr;
  ga.d = d;
  ga.I = I;
  if (!(cfg->flags & MOE_F_RING_DISPATCH)) {
    MOE_TRY(launch_gemm_gateup(ga, (int)m.tiles_bound, stream));
  } else {
    ga.ring = sc.ring;
    ga.ring_s = sc.ring_s;
    ga.nslots = (int)m.nslots;
    ga.slot_rows = (int)m.tile_rows;
    moe_status st;
    if ((st = ring_rounds(m, sv, xq, xs, sc.ring, sc.ring_s, true, stream,
                          [&](int chunk0, int nchunks, hipStream_t cst) {
                            ga.chunk0 = chunk0;
                            ga.nchunks = nchunks;
                            return launch_gemm_gateup(ga, nchunks, cst);
                          })) != MOE_OK)
      return st;
  }
  mark(stream, MOE_PH_GATEUP);

  DownArgs da{};
  da.s = sv;
  da.hq = ga.hq;
  da.hs = ga.hs;
  da.w2q = w2q;
  da.w2s = w2s;
  da.yslot = at<float>(saved, sl.yslot);
  da.w2t = want_wt ? at<uint8_t>(saved, sl.w2t) : nullptr;
  da.w2ts = want_wt ? at<uint8_t>(saved, sl.w2ts) : nullptr;
  da.d = d;
  da.I = I;
  MOE_TRY(launch_gemm_down(da, (int)m.tiles_bound, stream));
  mark(stream, MOE_PH_DOWN);

  MOE_TRY(launch_combine(da.yslot, w, (int)m.T, (int)m.k, (int)m.S, d, (uint16_t*)y_bf16, y_f32, stream));
  mark(stream, MOE_PH_COMBINE);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_query(const moe_config* cfg, size_t* workspace_bytes, moe_saved_layout* saved,
                     moe_workspace_layout* work) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  Dims m = dims(*cfg);
  const moe_workspace_layout wl = work_layout(m);
  if (workspace_bytes) *workspace_bytes = wl.total;
  if (saved) *saved = saved_layout(m, cfg->flags);
  if (work) *work = wl;
  return MOE_OK;
}

moe_status moe_quantize_mxfp8(const void* src, int src_is_f32, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* scales, hipStream_t stream) {
  if (!src || !q || !scales) return MOE_EINVAL;
  if (rows < 0 || cols < 0 || cols % 32) return MOE_ESHAPE;
  if (!aligned(src, 16) || !aligned(q, 16)) return MOE_EALIGN;
  return launch_quant_rows(src, src_is_f32 ? 1 : 0, rows, cols, q, scales, stream) == hipSuccess ? MOE_OK
                                                                                                : MOE_ELAUNCH;
}

moe_status moe_requant_transpose(const uint8_t* q, const uint8_t* scales, int64_t batch, int64_t rows, int64_t cols,
                                 uint8_t* qt, uint8_t* st, hipStream_t stream) {
  if (!q || !scales || !qt || !st) return MOE_EINVAL;
  if (batch < 0 || rows < 0 || cols < 0 || rows % 64 || cols % 64) return MOE_ESHAPE;
  if (!aligned(q, 16) || !aligned(qt, 16)) return MOE_EALIGN;
  return launch_requant_t(q, scales, batch, rows, cols, qt, st, stream) == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

moe_status moe_fwd(const moe_config* cfg, const void* x, const void* w_router, const float* router_bias,
                   const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q, const uint8_t* w2s, void* y_bf16,
                   float* y_f32, void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !w1q || !w1s || !w2q || !w2s || !y_bf16 || !saved || !workspace) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(w1q, 16) || !aligned(w2q, 16) || !aligned(y_bf16, 16) ||
      (y_f32 && !aligned(y_f32, 16)) || !aligned(saved, kAlign) || !aligned(workspace, kAlign))
    return MOE_EALIGN;
  const Dims m = dims(*cfg);
  const moe_saved_layout sl = saved_layout(m, cfg->flags);
  const moe_workspace_layout wl = work_layout(m);
  if (saved_bytes < sl.total || workspace_bytes < wl.total) return MOE_EWORKSPACE;
  if ((st = ensure_init()) != MOE_OK) return st;
  FwdScratch sc;
  sc.status = at<int32_t>(workspace, wl.status);
  sc.blkcnt = at<int32_t>(workspace, wl.blkcnt);
  sc.ring = at<uint8_t>(workspace, wl.ring);
  sc.ring_s = at<uint8_t>(workspace, wl.ring_s);
  sc.ring_flags = at<int32_t>(workspace, wl.ring_flags);
  if (m.unfused) {
    sc.xp = at<uint8_t>(workspace, wl.xp);
    sc.xps = at<uint8_t>(workspace, wl.xps);
    sc.yrows = at<float>(workspace, wl.yrows);
  }
  return forward_impl(cfg, m, sl, x, w_router, router_bias, w1q, w1s, w2q, w2s, y_bf16, y_f32, saved, sc, stream);
}

moe_status moe_fwd_noalloc(const moe_config* cfg, const void* x, const void* w_router, const float* router_bias,
                           const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q, const uint8_t* w2s,
                           void* y_bf16, float* y_f32, void* saved, size_t saved_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  // the ring buffer and the unfused forward's permuted rows live in a workspace
  if (cfg->flags & (MOE_F_RING_DISPATCH | MOE_F_UNFUSED)) return MOE_EINVAL;
  if (!x || !w_router || !w1q || !w1s || !w2q || !w2s || !y_bf16 || !saved) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(w1q, 16) || !aligned(w2q, 16) || !aligned(y_bf16, 16) ||
      (y_f32 && !aligned(y_f32, 16)) || !aligned(saved, kAlign))
    return MOE_EALIGN;
  const Dims m = dims(*cfg);
  const moe_saved_layout sl = saved_layout(m, cfg->flags);
  if (saved_bytes < sl.total) return MOE_EWORKSPACE;
  if (noalloc_scratch_bytes(m) > kScratchBytes) return MOE_EWORKSPACE;  // beyond the static scratch
  if ((st = ensure_init()) != MOE_OK) return st;
  uint8_t* base = nullptr;
  if ((st = device_scratch(&base)) != MOE_OK) return st;
  FwdScratch sc;
  sc.status = (int32_t*)base;
  sc.blkcnt = (int32_t*)(base + kAlign);
  sc.ring = nullptr;
  sc.ring_s = nullptr;
  sc.ring_flags = nullptr;
  return forward_impl(cfg, m, sl, x, w_router, router_bias, w1q, w1s, w2q, w2s, y_bf16, y_f32, saved, sc, stream);
}

moe_status moe_bwd(const moe_config* cfg, const void* dy, const void* x, const void* w_router, const void* saved,
                   size_t saved_bytes, void* dx_bf16, float* dx_f32, float* dw_router, void* dw1, void* dw2,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  // forward-only check mode / forward-only layout: there is no saved state to differentiate
  if (cfg->flags & (MOE_F_IDENTITY_EXPERTS | MOE_F_FORWARD_ONLY)) return MOE_EINVAL;
  if (!dy || !x || !w_router || !saved || !dx_bf16 || !dw_router || !dw1 || !dw2 || !workspace) return MOE_EINVAL;
  if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(w_router, 16) || !aligned(dx_bf16, 16) ||
      (dx_f32 && !aligned(dx_f32, 16)) || !aligned(dw_router, 16) || !aligned(dw1, 16) || !aligned(dw2, 16) ||
      !aligned(saved, kAlign) || !aligned(workspace, kAlign))
    return MOE_EALIGN;
  const Dims m = dims(*cfg);
  const moe_saved_layout sl = saved_layout(m, cfg->flags);
  const moe_workspace_layout wl = work_layout(m);
  if (saved_bytes < sl.total || workspace_bytes < wl.total) return MOE_EWORKSPACE;
  if ((st = ensure_init()) != MOE_OK) return st;
  const int d = (int)m.d, I = (int)m.I;
  const SchedView sv = sched_view(saved, sl, m);
  const float* w = at<float>(saved, sl.w);
  const int32_t* idx = at<int32_t>(saved, sl.idx);
  const int64_t* tok_off = at<int64_t>(saved, sl.tok_off);
  const int32_t* tile64 = at<int32_t>(saved, sl.tile64);

  uint8_t* dyq = at<uint8_t>(workspace, wl.dyq);
  uint8_t* dys = at<uint8_t>(workspace, wl.dys);
  float* dwv = at<float>(workspace, wl.dw);
  float* dl = at<float>(workspace, wl.dl);
  mark(stream, MOE_PH_BWD_BEGIN);
  MOE_TRY(launch_quant_rows(dy, 0, m.T, m.d, dyq, dys, stream));
  mark(stream, MOE_PH_QUANT_DY);

  // Token-axis requantisation of the weight-gradient operands, and dW2[e] [d, I] = dYw^T H, depend
  // only on the forward's saved rows and on dy: they run on the device's second stream, beside
  // the router backward and the dgrad chain (whose buffers they do not touch), and are joined
  // before dW1.  MOE_F_SERIAL_BWD (or no second stream) keeps everything in launch order.
  SideStream* side = (cfg->flags & MOE_F_SERIAL_BWD) ? nullptr : side_stream(kBranchStream);
  hipStream_t sst = side ? side->st : stream;
  TokArgs ta{};
  ta.s = sv;
  ta.w = w;
  ta.tok_off = tok_off;
  ta.tile64 = tile64;
  ta.ld = m.ld_tok;
  const int tb = (int)m.tile64_bound;
  WgradArgs wa{};
  wa.tok_off = tok_off;
  wa.dw_bf16 = (cfg->flags & MOE_F_DW_BF16) ? 1 : 0;
  wa.ld = m.ld_tok;
  auto side_branch = [&]() -> moe_status {
    ta.q = at<uint8_t>(saved, sl.xq); ta.qs = at<uint8_t>(saved, sl.xs); ta.cols = d; ta.src = TOK_X;
    ta.out = at<uint8_t>(workspace, wl.xt); ta.outs = at<uint8_t>(workspace, wl.xts);
    MOE_TRY(launch_token_requant(ta, tb, sst));
    ta.q = at<uint8_t>(saved, sl.hq); ta.qs = at<uint8_t>(saved, sl.hs); ta.cols = I; ta.src = TOK_H;
    ta.out = at<uint8_t>(workspace, wl.ht); ta.outs = at<uint8_t>(workspace, wl.hts);
    MOE_TRY(launch_token_requant(ta, tb, sst));
    ta.q = dyq; ta.qs = dys; ta.cols = d; ta.src = TOK_DYW;
    ta.out = at<uint8_t>(workspace, wl.dyt); ta.outs = at<uint8_t>(workspace, wl.dyts);
    MOE_TRY(launch_token_requant(ta, tb, sst));
    return MOE_OK;
  };
  auto wgrad_down = [&]() -> moe_status {
    WgradArgs a2 = wa;
    a2.at = at<uint8_t>(workspace, wl.dyt); a2.ats = at<uint8_t>(workspace, wl.dyts);
    a2.bt = at<uint8_t>(workspace, wl.ht); a2.bts = at<uint8_t>(workspace, wl.hts);
    a2.dw = dw2; a2.M = d; a2.N = I; a2.n_exp = (int)m.NX;
    MOE_TRY(launch_gemm_wgrad(a2, 0, sst));
    return MOE_OK;
  };
  if (side) {
    MOE_TRY(hipEventRecord(side->fork, stream));
    MOE_TRY(hipStreamWaitEvent(side->st, side->fork, 0));
    if ((st = side_branch()) != MOE_OK) return st;
    if ((st = wgrad_down()) != MOE_OK) return st;
    MOE_TRY(hipEventRecord(side->join, side->st));
  }

  MOE_TRY(launch_router_bwd((const uint16_t*)dy, at<float>(saved, sl.yslot), at<float>(saved, sl.logits), idx, w,
                            (int)m.T, (int)m.E, (int)m.k, (int)m.S, d, cfg->score_fn, dwv, dl, stream));
  mark(stream, MOE_PH_ROUTER_BWD);
  MOE_TRY(launch_router_wgrad(sv, dl, (const uint16_t*)x, d, (int)m.E, dw_router, stream));
  mark(stream, MOE_PH_ROUTER_WGRAD);

  // The transposed requantisation of the expert weights (W1 along 2I, W2 along d) was done by
  // the forward GEMMs from the weight slices they streamed (saved w1t / w2t): the phase below
  // is empty.
  mark(stream, MOE_PH_REQUANT_W);

  DgradDownArgs dd{};
  dd.s = sv;
  dd.dyq = dyq;
  dd.dys = dys;
  dd.w2t = at<uint8_t>(saved, sl.w2t);
  dd.w2ts = at<uint8_t>(saved, sl.w2ts);
  dd.w = w;
  dd.g = at<float>(saved, sl.g);
  dd.u = at<float>(saved, sl.u);
  dd.dguq = at<uint8_t>(workspace, wl.dguq);
  dd.dgus = at<uint8_t>(workspace, wl.dgus);
  dd.d = d;
  dd.I = I;
  if (!(cfg->flags & MOE_F_RING_DISPATCH)) {
    MOE_TRY(launch_gemm_dgrad_down(dd, (int)m.tiles_bound, stream));
  } else {
    // pull reverse-combine through the ring: the dY rows each expert needs, staged in its slots
    // (the forward's GEMM rounds that read the ring are all ahead of this call on the stream)
    dd.ring = at<uint8_t>(workspace, wl.ring);
    dd.ring_s = at<uint8_t>(workspace, wl.ring_s);
    dd.nslots = (int)m.nslots;
    dd.slot_rows = (int)m.tile_rows;
    if ((st = ring_rounds(m, sv, dyq, dys, at<uint8_t>(workspace, wl.ring), at<uint8_t>(workspace, wl.ring_s),
                          !(cfg->flags & MOE_F_SERIAL_BWD), stream,
                          [&](int chunk0, int nchunks, hipStream_t cst) {
                            dd.chunk0 = chunk0;
                            dd.nchunks = nchunks;
                            return launch_gemm_dgrad_down(dd, nchunks, cst);
                          })) != MOE_OK)
      return st;
  }
  mark(stream, MOE_PH_DGRAD_DOWN);

  DgradGateUpArgs dg{};
  dg.s = sv;
  dg.dguq = dd.dguq;
  dg.dgus = dd.dgus;
  dg.w1t = at<uint8_t>(saved, sl.w1t);
  dg.w1ts = at<uint8_t>(saved, sl.w1ts);
  dg.dxslot = at<float>(workspace, wl.dxslot);
  dg.d = d;
  dg.I = I;
  MOE_TRY(launch_gemm_dgrad_gateup(dg, (int)m.tiles_bound, stream));
  mark(stream, MOE_PH_DGRAD_GATEUP);
  MOE_TRY(launch_dx_reduce(dg.dxslot, dl, idx, (const uint16_t*)w_router, (int)m.T, (int)m.k, (int)m.S, d,
                           (uint16_t*)dx_bf16, dx_f32, stream));
  mark(stream, MOE_PH_DX_REDUCE);

  if (!side && (st = side_branch()) != MOE_OK) return st;
  ta.q = dd.dguq; ta.qs = dd.dgus; ta.cols = 2 * I; ta.src = TOK_DGU;
  ta.out = at<uint8_t>(workspace, wl.dgut); ta.outs = at<uint8_t>(workspace, wl.dguts);
  MOE_TRY(launch_token_requant(ta, tb, stream));
  mark(stream, MOE_PH_TOKEN_REQUANT);
  if (!side && (st = wgrad_down()) != MOE_OK) return st;
  if (side) MOE_TRY(hipStreamWaitEvent(stream, side->join, 0));
  mark(stream, MOE_PH_WGRAD_DOWN);
  // dW1[e] [2I, d] = dGU^T X
  wa.at = at<uint8_t>(workspace, wl.dgut); wa.ats = at<uint8_t>(workspace, wl.dguts);
  wa.bt = at<uint8_t>(workspace, wl.xt); wa.bts = at<uint8_t>(workspace, wl.xts);
  wa.dw = dw1; wa.M = 2 * I; wa.N = d; wa.n_exp = (int)m.NX;
  MOE_TRY(launch_gemm_wgrad(wa, 1, stream));
  mark(stream, MOE_PH_WGRAD_GATEUP);
  return MOE_OK;
}

moe_status moe_set_phase_events(hipEvent_t* events, int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && !events)) return MOE_EINVAL;
  g_events = n_events ? events : nullptr;
  g_n_events = n_events;
  return MOE_OK;
}

moe_status moe_device_status(const void* workspace, int32_t* device_code) {
  if (!workspace || !device_code) return MOE_EINVAL;
  int32_t code = 0;
  if (hipMemcpy(&code, workspace, sizeof(code), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ELAUNCH;
  *device_code = code;
  return code == 0 ? MOE_OK : MOE_EDEVICE;
}

moe_status moe_probe_mfma(float* sink, size_t sink_bytes, int32_t iters, double* flop, size_t* sink_needed,
                          hipStream_t stream) {
  if (!flop) return MOE_EINVAL;
  *flop = 0.0;
  if (iters < 1) return MOE_EINVAL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ELAUNCH;
  const size_t need = probe_mfma_sink_bytes(cus);
  if (sink_needed) *sink_needed = need;
  if (!sink || sink_bytes < need) return MOE_EWORKSPACE;
  return launch_probe_mfma(sink, cus, iters, flop, stream) == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

const char* moe_strerror(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer or unsupported option)";
    case MOE_ESHAPE: return "unsupported sizes";
    case MOE_EALIGN: return "misaligned pointer";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_ELAUNCH: return "kernel launch failed";
    case MOE_EDEVICE: return "device reported an anomaly";
  }
  return "unknown status";
}

}  // extern "C"
