// api.cpp -- the C ABI of libra.so: host-side validation, status reporting,
// and the ring driver that runs R hops on one GPU with the K/V hand-off on a
// second stream.
//
// Ring structure: highthink.cn Ring Attention article, section "Zig Zag Ring
// Attention 通信和计算重叠" (each rank keeps its Q chunk, computes attention
// with the K/V it holds, sends that K/V to the next rank and receives the
// previous rank's, until every query has met every key; the next block is
// received while the current one is computed).  Folding of the per-hop
// partials: aiunderstanding.org "Sequenzparallelität und Ringaufmerksamkeit",
// "Tiefer Einblick", and its Thai version, technical-insight section.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "ra_internal.h"

namespace ra {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

namespace {

int elt_bytes(int dtype) {
  switch (dtype) {
    case RA_DT_BF16:
    case RA_DT_FP16:
      return 2;
    case RA_DT_FP32:
      return 4;
    default:
      return 0;
  }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

ra_status fail(ra_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

ra_status hip_fail(hipError_t e, const char *what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define RA_HIP(call, what)                     \
  do {                                         \
    hipError_t e_ = (call);                    \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr int64_t kMaxI32 = 2147483647;

// Events with which the ring drivers order their two streams.  A call leases
// a set while it enqueues its work and hands it back when it returns: a
// stream wait binds to the record that precedes it, so the same events can
// serve the next call at once.  Sets are cached per device behind a mutex --
// as many sets as calls ever ran at the same time -- and kept until the
// process ends (destroying them at exit could outlive the HIP runtime).
class EventSets {
 public:
  hipError_t acquire(int dev, size_t n, std::vector<hipEvent_t> *out) {
    {
      std::lock_guard<std::mutex> g(mu_);
      auto &fl = free_[dev];
      if (!fl.empty()) {
        *out = std::move(fl.back());
        fl.pop_back();
      }
    }
    while (out->size() < n) {
      hipEvent_t e;
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
      out->push_back(e);
      std::lock_guard<std::mutex> g(mu_);
      ++created_;
    }
    return hipSuccess;
  }
  void release(int dev, std::vector<hipEvent_t> *ev) {
    if (ev->empty()) return;
    std::lock_guard<std::mutex> g(mu_);
    free_[dev].push_back(std::move(*ev));
    ev->clear();
  }
  size_t created() {
    std::lock_guard<std::mutex> g(mu_);
    return created_;
  }

 private:
  std::mutex mu_;
  std::map<int, std::vector<std::vector<hipEvent_t>>> free_;
  size_t created_ = 0;
};

EventSets &event_sets() {
  static EventSets *sets = new EventSets;  // intentionally never destroyed
  return *sets;
}

// A leased event set, handed back on every exit path of the call.
struct EventLease {
  int dev = 0;
  std::vector<hipEvent_t> ev;
  ~EventLease() { event_sets().release(dev, &ev); }
  hipError_t acquire(size_t n) {
    hipError_t r = hipGetDevice(&dev);
    if (r != hipSuccess) return r;
    return event_sets().acquire(dev, n, &ev);
  }
};

// Debug aid for the stream ordering of the ring drivers: the environment
// variables RA_DEBUG_DELAY_COPY and RA_DEBUG_DELAY_COMPUTE (a step count, at
// most 100000, of about 4 us each) put a bounded sleeping kernel on the copy
// stream before each hand-off, or on the compute stream before each hop's
// kernels.  Results must not change: only the timing of the two streams
// relative to each other does.  Read at every call; unset means no delay.
struct DebugDelay {
  int copy = 0, compute = 0;
};
DebugDelay debug_delay() {
  auto get = [](const char *name) {
    const char *v = std::getenv(name);
    if (!v || !*v) return 0;
    const long x = std::strtol(v, nullptr, 10);
    return (int)std::min<long>(std::max<long>(x, 0), 100000);
  };
  DebugDelay d;
  d.copy = get("RA_DEBUG_DELAY_COPY");
  d.compute = get("RA_DEBUG_DELAY_COMPUTE");
  return d;
}

// Which hand-off copy a ring uses: the thin one, which runs beside the hop's
// kernels without taking their compute units, when the hop's MFMA work (4 d
// flop per allowed (query, key) pair and query head at 1.3 PFLOP/s; a causal
// block has about half its pairs; `work` scales for the backward's kernels)
// lasts at least half as long as moving the hop's bytes at a deliberately low
// 1 TB/s -- the hops of the 1M-token share and of 4096-token blocks (32k
// causal MHA over 8 ranks: 6.6 % shorter steps contiguous, 2 % striped), not
// those of 512-token blocks, which are short and memory-heavy: there the copy
// competes with the hop for HBM and the 64-workgroup copy costs less
// (measured side by side).
bool thin_handoff(double moved_bytes, double pairs_heads, int d, double work) {
  const double t_hop = work * 4.0 * d * pairs_heads / 1.3e15;
  return t_hop > 0.5 * moved_bytes / 1.0e12;
}

struct WsLayout {
  size_t vpack, kbuf[2], vbuf[2], o_acc, m_acc, l_acc, o_blk, m_blk, l_blk, total;
};

// The ring feeds 16-bit V to the block kernel in the packed layout.
bool ring_packs_v(const ra_ring_args *a) { return a->dtype != RA_DT_FP32; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const ra_ring_args *a) {
  WsLayout w{};
  const size_t elt = (size_t)elt_bytes(a->dtype);
  const size_t blk = (size_t)a->B * a->Hkv * a->n * a->d;
  const size_t blkv = ring_packs_v(a) ? (size_t)a->B * a->Hkv * a->d * packed_n(a->n) : blk;
  const size_t k_bytes = (size_t)a->n_ranks * blk * elt;
  const size_t v_bytes = (size_t)a->n_ranks * blkv * elt;
  const size_t rows = (size_t)a->n_ranks * a->B * a->Hq * a->n;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (ring_packs_v(a)) w.vpack = take((size_t)a->R * blkv * elt);
  if (a->handoff != RA_HANDOFF_SWAP && a->R > 1) {
    w.kbuf[0] = take(k_bytes);
    w.kbuf[1] = take(k_bytes);
    w.vbuf[0] = take(v_bytes);
    w.vbuf[1] = take(v_bytes);
  }
  w.o_acc = take(rows * a->d * sizeof(float));
  w.m_acc = take(rows * sizeof(float));
  w.l_acc = take(rows * sizeof(float));
  if (a->merge_mode == RA_MERGE_SEPARATE) {
    w.o_blk = take(rows * a->d * sizeof(float));
    w.m_blk = take(rows * sizeof(float));
    w.l_blk = take(rows * sizeof(float));
  }
  w.total = off;
  return w;
}

bool known_layout(int32_t layout) {
  return layout == RA_LAYOUT_CONTIGUOUS || layout == RA_LAYOUT_STRIPED ||
         layout == RA_LAYOUT_ZIGZAG;
}

// Global token id of local position j of rank `rank` (the maps of
// ra_layout_permute), n tokens per rank.
int64_t layout_gid(int32_t layout, int32_t R, int64_t n, int32_t rank, int64_t j) {
  if (layout == RA_LAYOUT_CONTIGUOUS) return (int64_t)rank * n + j;
  if (layout == RA_LAYOUT_STRIPED) return j * R + rank;
  const int64_t c = n / 2;
  return j < c ? (int64_t)rank * c + j : (2 * (int64_t)R - 1 - rank) * c + (j - c);
}

ra_status check_block_bwd(const ra_block_bwd_args *a) {
  if (!a) return fail(RA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != RA_DT_BF16 && a->dtype != RA_DT_FP16) {
    if (a->dtype == RA_DT_FP32) return fail(RA_ERR_UNSUPPORTED, "backward is for 16-bit inputs");
    return fail(RA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  }
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1) return fail(RA_ERR_SHAPE, "B, Hq, Hkv must be >= 1");
  if (a->Hq % a->Hkv) return fail(RA_ERR_SHAPE, "Hq %% Hkv != 0 (%d, %d)", a->Hq, a->Hkv);
  if (a->d != 64 && a->d != 128) return fail(RA_ERR_SHAPE, "d must be 64 or 128 (got %d)", a->d);
  if (a->n_q < 0 || a->n_k < 0) return fail(RA_ERR_SHAPE, "n_q, n_k must be >= 0");
  if (a->n_q > kMaxPackedKeys || a->n_k > kMaxPackedKeys)
    return fail(RA_ERR_UNSUPPORTED, "n_q, n_k are limited to %lld", (long long)kMaxPackedKeys);
  if (a->q_gid_step < 1 || a->k_gid_step < 1)
    return fail(RA_ERR_INVALID_ARG, "global-id steps must be >= 1");
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(RA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (a->n_q == 0) return RA_OK;
  if (!a->q || !a->o || !a->dout || !a->lse || !a->dq || (a->n_k > 0 && (!a->k || !a->v ||
                                                                        !a->dk || !a->dv)))
    return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(a->q) || !aligned16(a->o) || !aligned16(a->dout) || !aligned16(a->dq) ||
      (a->n_k > 0 && (!aligned16(a->k) || !aligned16(a->v) || !aligned16(a->dk) ||
                      !aligned16(a->dv))))
    return fail(RA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  return RA_OK;
}

struct BwdWs {
  size_t qT, doT, kT, nd, nl, total;
};
BwdWs block_bwd_ws(const ra_block_bwd_args *a) {
  BwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t qbytes = (size_t)a->B * a->Hq * a->d * packed_n(a->n_q) * 2;
  w.qT = take(qbytes);
  w.doT = take(qbytes);
  w.kT = take((size_t)a->B * a->Hkv * a->d * packed_n(a->n_k) * 2);
  w.nd = take((size_t)a->B * a->Hq * a->n_q * 4);
  w.nl = take((size_t)a->B * a->Hq * a->n_q * 4);
  w.total = off;
  return w;
}

ra_status check_ring_bwd(const ra_ring_bwd_args *a) {
  if (!a) return fail(RA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != RA_DT_BF16 && a->dtype != RA_DT_FP16) {
    if (a->dtype == RA_DT_FP32) return fail(RA_ERR_UNSUPPORTED, "backward is for 16-bit inputs");
    return fail(RA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  }
  if (!known_layout(a->layout)) return fail(RA_ERR_INVALID_ARG, "unknown layout %d", a->layout);
  if (a->handoff != RA_HANDOFF_COPY && a->handoff != RA_HANDOFF_SWAP &&
      a->handoff != RA_HANDOFF_FORWARD)
    return fail(RA_ERR_INVALID_ARG, "unknown handoff %d", a->handoff);
  if (a->R < 1) return fail(RA_ERR_SHAPE, "R must be >= 1 (got %d)", a->R);
  if (a->n_ranks < 1 || a->n_ranks > a->R || a->rank0 < 0 || a->rank0 + a->n_ranks > a->R)
    return fail(RA_ERR_SHAPE, "ranks [rank0, rank0+n_ranks) must lie in [0, R)");
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1) return fail(RA_ERR_SHAPE, "B, Hq, Hkv must be >= 1");
  if (a->Hq % a->Hkv) return fail(RA_ERR_SHAPE, "Hq %% Hkv != 0 (%d, %d)", a->Hq, a->Hkv);
  if (a->d != 64 && a->d != 128) return fail(RA_ERR_SHAPE, "d must be 64 or 128 (got %d)", a->d);
  if (a->n < 0) return fail(RA_ERR_SHAPE, "n must be >= 0");
  if (a->layout == RA_LAYOUT_ZIGZAG && a->n % 2)
    return fail(RA_ERR_SHAPE, "zig-zag blocks hold two equal chunks: n must be even");
  if (a->n > kMaxPackedKeys)
    return fail(RA_ERR_UNSUPPORTED, "blocks are limited to %lld tokens", (long long)kMaxPackedKeys);
  if ((int64_t)a->n * a->R > kMaxI32) return fail(RA_ERR_SHAPE, "S = n*R must be < 2^31");
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(RA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (a->n > 0) {
    if (!a->q_sh || !a->k_sh || !a->v_sh || !a->o_sh || !a->dout_sh || !a->lse || !a->dq_sh ||
        !a->dk_sh || !a->dv_sh)
      return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    const void *ptrs[] = {a->q_sh, a->k_sh, a->v_sh, a->o_sh, a->dout_sh, a->dq_sh, a->dk_sh,
                          a->dv_sh};
    for (const void *x : ptrs)
      if (!aligned16(x)) return fail(RA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  }
  return RA_OK;
}

struct RingBwdWs {
  size_t qT, doT, kT, D, nl, dq, dk, dv, total;
  // COPY hand-off: two receive buffers (n_ranks blocks each) for K, V, packed
  // K^T and the fp32 dK, dV accumulators that travel with the block
  size_t kbuf[2], vbuf[2], kTbuf[2], dkbuf[2], dvbuf[2];
};
RingBwdWs ring_bwd_ws(const ra_ring_bwd_args *a) {
  RingBwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t np = (size_t)packed_n(a->n);
  const size_t qrows = (size_t)a->n_ranks * a->B * a->Hq;
  const size_t kblocks = (size_t)a->R * a->B * a->Hkv;
  w.qT = take(qrows * a->d * np * 2);
  w.doT = take(qrows * a->d * np * 2);
  w.kT = take(kblocks * a->d * np * 2);
  w.D = take(qrows * a->n * 4);
  w.nl = take(qrows * a->n * 4);
  w.dq = take(qrows * a->n * a->d * 4);
  w.dk = take(kblocks * a->n * a->d * 4);
  w.dv = take(kblocks * a->n * a->d * 4);
  if (a->handoff != RA_HANDOFF_SWAP && a->R > 1) {
    const size_t rblocks = (size_t)a->n_ranks * a->B * a->Hkv;
    for (int b = 0; b < 2; ++b) {
      w.kbuf[b] = take(rblocks * a->n * a->d * 2);
      w.vbuf[b] = take(rblocks * a->n * a->d * 2);
      w.kTbuf[b] = take(rblocks * a->d * np * 2);
      w.dkbuf[b] = take(rblocks * a->n * a->d * 4);
      w.dvbuf[b] = take(rblocks * a->n * a->d * 4);
    }
  }
  w.total = off;
  return w;
}

ra_status check_decode(const ra_decode_args *a) {
  if (!a) return fail(RA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != RA_DT_BF16 && a->dtype != RA_DT_FP16) {
    if (a->dtype == RA_DT_FP32) return fail(RA_ERR_UNSUPPORTED, "decode reads packed 16-bit V");
    return fail(RA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  }
  if (a->R < 1 || a->R > 512) return fail(RA_ERR_SHAPE, "R must be in [1, 512] (got %d)", a->R);
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1) return fail(RA_ERR_SHAPE, "B, Hq, Hkv must be >= 1");
  if (a->Hq % a->Hkv) return fail(RA_ERR_SHAPE, "Hq %% Hkv != 0 (%d, %d)", a->Hq, a->Hkv);
  if (a->d != 64 && a->d != 128) return fail(RA_ERR_SHAPE, "d must be 64 or 128 (got %d)", a->d);
  if (a->nq < 1 || (int64_t)(a->Hq / a->Hkv) * a->nq > 256)
    return fail(RA_ERR_SHAPE, "need 1 <= nq and (Hq/Hkv)*nq <= 256 (nq=%d)", a->nq);
  if (a->n < 0) return fail(RA_ERR_SHAPE, "n must be >= 0");
  if (a->n > kMaxPackedKeys)
    return fail(RA_ERR_UNSUPPORTED, "cache shards are limited to %lld tokens",
                (long long)kMaxPackedKeys);
  if ((int64_t)a->n * a->R > kMaxI32) return fail(RA_ERR_SHAPE, "R*n must be < 2^31");
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(RA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!a->q || !a->o || !a->lse || (a->n > 0 && (!a->k || !a->v)))
    return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(a->q) || !aligned16(a->o) || (a->n > 0 && (!aligned16(a->k) || !aligned16(a->v))))
    return fail(RA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  return RA_OK;
}

// Work split of a decode call: enough workgroups to fill the GPU, every wave
// a run of keys (a multiple of 32), one partial per workgroup, at most 4096
// partials per row.
DecodeParams decode_plan(const ra_decode_args *a) {
  DecodeParams p{};
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.nq = a->nq;
  p.n = a->n;
  p.d = a->d;
  p.R = a->R;
  p.n_pad = packed_n(a->n);
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.q_gid0 = a->q_gid0;
  p.col_blocks = ((a->Hq / a->Hkv) * a->nq + 31) / 32;
  const int64_t groups = (int64_t)a->R * a->B * a->Hkv * p.col_blocks;
  const int64_t W = kDecodeWaves;
  // each wave streams whole 64-key tiles (one packed V^T tile each)
  const int64_t max_splits = std::max<int64_t>(1, (a->n + W * 64 - 1) / (W * 64));
  // Workgroups: exactly as many as fit at once (a 64-key LDS ring per wave
  // leaves room for one workgroup per CU at d = 128, two at d = 64), so the
  // cache streams in one round with no tail; measured on the 1M-token cache:
  // 256 workgroups 6.95 TB/s, 512 6.66, 1024 6.52.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int64_t want = (int64_t)cus * (a->d == 64 ? 2 : 1);
  int64_t splits = std::min<int64_t>(max_splits, std::max<int64_t>(1, (want + groups - 1) / groups));
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, 4096 / (int64_t)a->R));
  int64_t wk = (a->n + splits * W - 1) / (splits * W);
  wk = std::max<int64_t>(64, (wk + 63) / 64 * 64);
  splits = std::max<int64_t>(1, (a->n + W * wk - 1) / (W * wk));
  p.splits = (int32_t)splits;
  p.wave_keys = (int32_t)wk;
  p.P = (int32_t)(a->R * splits);
  return p;
}

size_t decode_ws_bytes(const DecodeParams &p) {
  const size_t rows = (size_t)p.B * p.Hq * p.nq;
  return align256((size_t)p.P * rows * p.d * 4) + 2 * align256((size_t)p.P * rows * 4);
}

// Decode with its partials at ws (decode_ws_bytes(p) bytes, 256-byte
// aligned).  Every partial is written before it is read, so ws needs no
// clearing.
ra_status run_decode(const ra_decode_args *a, DecodeParams p, char *ws, hipStream_t s) {
  const size_t rows = (size_t)p.B * p.Hq * p.nq;
  p.po = (float *)ws;
  p.pm = (float *)(ws + align256((size_t)p.P * rows * p.d * 4));
  p.pl = (float *)((char *)p.pm + align256((size_t)p.P * rows * 4));
  p.q = a->q;
  p.k = a->n > 0 ? a->k : a->q;  // never read when n == 0
  p.v = a->n > 0 ? a->v : a->q;
  RA_HIP(launch_decode(p, a->dtype, a->o, a->lse, s), "decode kernels");
  return RA_OK;
}

ra_status check_ring(const ra_ring_args *a) {
  if (!a) return fail(RA_ERR_INVALID_ARG, "args is NULL");
  if (!elt_bytes(a->dtype)) return fail(RA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (!known_layout(a->layout)) return fail(RA_ERR_INVALID_ARG, "unknown layout %d", a->layout);
  if (a->handoff != RA_HANDOFF_COPY && a->handoff != RA_HANDOFF_SWAP &&
      a->handoff != RA_HANDOFF_FORWARD)
    return fail(RA_ERR_INVALID_ARG, "unknown handoff %d", a->handoff);
  if (a->merge_mode != RA_MERGE_FUSED && a->merge_mode != RA_MERGE_SEPARATE)
    return fail(RA_ERR_INVALID_ARG, "unknown merge_mode %d", a->merge_mode);
  if (a->R < 1) return fail(RA_ERR_SHAPE, "R must be >= 1 (got %d)", a->R);
  if (a->n_ranks < 1 || a->n_ranks > a->R)
    return fail(RA_ERR_SHAPE, "n_ranks must be in [1, R] (got %d, R=%d)", a->n_ranks, a->R);
  if (a->rank0 < 0 || a->rank0 + a->n_ranks > a->R)
    return fail(RA_ERR_SHAPE, "ranks [rank0, rank0+n_ranks) must lie in [0, R) (rank0=%d)",
                a->rank0);
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1)
    return fail(RA_ERR_SHAPE, "B, Hq, Hkv must be >= 1");
  if (a->Hq % a->Hkv) return fail(RA_ERR_SHAPE, "Hq %% Hkv != 0 (%d, %d)", a->Hq, a->Hkv);
  if (a->d != 64 && a->d != 128) return fail(RA_ERR_SHAPE, "d must be 64 or 128 (got %d)", a->d);
  if (a->n < 0) return fail(RA_ERR_SHAPE, "n must be >= 0");
  if (a->layout == RA_LAYOUT_ZIGZAG && a->n % 2)
    return fail(RA_ERR_SHAPE, "zig-zag blocks hold two equal chunks: n must be even (got %d)",
                a->n);
  if (a->dtype != RA_DT_FP32 && a->n > kMaxPackedKeys)
    return fail(RA_ERR_UNSUPPORTED, "16-bit ring blocks are limited to %lld tokens (got %d)",
                (long long)kMaxPackedKeys, a->n);
  if ((int64_t)a->n * a->R > kMaxI32) return fail(RA_ERR_SHAPE, "S = n*R must be < 2^31");
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(RA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (a->n > 0) {
    if (!a->q_sh || !a->k_sh || !a->v_sh || !a->o || !a->lse)
      return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(a->q_sh) || !aligned16(a->k_sh) || !aligned16(a->v_sh) || !aligned16(a->o))
      return fail(RA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  }
  return RA_OK;
}

ra_status check_block(const ra_block_args *a) {
  if (!a) return fail(RA_ERR_INVALID_ARG, "args is NULL");
  const int elt = elt_bytes(a->dtype);
  if (!elt) return fail(RA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1)
    return fail(RA_ERR_SHAPE, "B, Hq, Hkv must be >= 1");
  if (a->Hq % a->Hkv) return fail(RA_ERR_SHAPE, "Hq %% Hkv != 0 (%d, %d)", a->Hq, a->Hkv);
  if (a->d != 64 && a->d != 128) return fail(RA_ERR_SHAPE, "d must be 64 or 128 (got %d)", a->d);
  if (a->n_q < 0 || a->n_k < 0) return fail(RA_ERR_SHAPE, "n_q, n_k must be >= 0");
  if (a->v_packed != 0 && a->v_packed != 1) return fail(RA_ERR_INVALID_ARG, "v_packed must be 0 or 1");
  if (a->v_packed && a->dtype == RA_DT_FP32)
    return fail(RA_ERR_UNSUPPORTED, "packed V is for bf16/fp16 inputs");
  if (a->q_gid_step < 1 || a->k_gid_step < 1)
    return fail(RA_ERR_INVALID_ARG, "global-id steps must be >= 1");
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(RA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (a->n_q == 0) return RA_OK;
  if (!a->q || !a->o || !a->m || !a->l) return fail(RA_ERR_INVALID_ARG, "null tensor pointer");
  if (a->n_k > 0 && (!a->k || !a->v)) return fail(RA_ERR_INVALID_ARG, "null k/v pointer");
  if (!aligned16(a->q) || !aligned16(a->o) || (a->n_k > 0 && (!aligned16(a->k) || !aligned16(a->v))))
    return fail(RA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  const int64_t vs_chk = a->v_packed ? 0 : 1;
  for (int i = 0; i < 3; ++i) {
    if ((a->q_stride[i] * elt) % 16 || (a->k_stride[i] * elt) % 16 ||
        (vs_chk * a->v_stride[i] * elt) % 16 || (a->o_stride[i] * 4) % 16)
      return fail(RA_ERR_ALIGNMENT, "strides must keep rows 16-byte aligned");
    if (a->q_stride[i] < 0 || a->k_stride[i] < 0 || vs_chk * a->v_stride[i] < 0 ||
        a->o_stride[i] < 0)
      return fail(RA_ERR_SHAPE, "negative stride");
  }
  if (a->v_packed && (a->n_k > kMaxPackedKeys || a->k_stride[2] > kMaxKRowStride))
    return fail(RA_ERR_UNSUPPORTED, "packed V: n_k <= %lld and K token stride <= %lld",
                (long long)kMaxPackedKeys, (long long)kMaxKRowStride);
  if (a->q_stride[2] < a->d || a->o_stride[2] < a->d ||
      (a->n_k > 0 && (a->k_stride[2] < a->d || (!a->v_packed && a->v_stride[2] < a->d))))
    return fail(RA_ERR_SHAPE, "token stride smaller than d");
  return RA_OK;
}

}  // namespace
}  // namespace ra

using namespace ra;

extern "C" {

int ra_version(void) { return 100; }

size_t ra_cached_events(void) { return event_sets().created(); }

const char *ra_status_string(ra_status s) {
  switch (s) {
    case RA_OK:
      return "RA_OK";
    case RA_ERR_INVALID_ARG:
      return "RA_ERR_INVALID_ARG";
    case RA_ERR_SHAPE:
      return "RA_ERR_SHAPE";
    case RA_ERR_DTYPE:
      return "RA_ERR_DTYPE";
    case RA_ERR_ALIGNMENT:
      return "RA_ERR_ALIGNMENT";
    case RA_ERR_WORKSPACE:
      return "RA_ERR_WORKSPACE";
    case RA_ERR_UNSUPPORTED:
      return "RA_ERR_UNSUPPORTED";
    case RA_ERR_HIP:
      return "RA_ERR_HIP";
  }
  return "RA_ERR_UNKNOWN";
}

const char *ra_last_error(void) { return g_err; }

ra_status ra_layout_permute(int32_t layout, int64_t S, int32_t R, int32_t *fwd, int32_t *inv,
                            ra_stream stream) {
  clear_error();
  if (!known_layout(layout)) return fail(RA_ERR_INVALID_ARG, "unknown layout %d", layout);
  if (R < 1 || S < 0 || S % R) return fail(RA_ERR_SHAPE, "need R >= 1, S >= 0, S %% R == 0");
  if (layout == RA_LAYOUT_ZIGZAG && S % (2 * (int64_t)R))
    return fail(RA_ERR_SHAPE, "zig-zag needs S %% 2R == 0");
  if (S > kMaxI32) return fail(RA_ERR_SHAPE, "S must be < 2^31");
  if (S > 0 && !fwd) return fail(RA_ERR_INVALID_ARG, "fwd is NULL");
  RA_HIP(launch_layout_permute(layout, S, R, fwd, inv, (hipStream_t)stream), "layout kernel");
  return RA_OK;
}

static ra_status layout_move(bool gather, const void *src, void *dst, const int32_t *fwd,
                             int32_t elem_bytes, int64_t B, int64_t H, int64_t S, int64_t d,
                             int32_t R, int32_t rank0, int32_t n_ranks, ra_stream stream) {
  clear_error();
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return fail(RA_ERR_INVALID_ARG, "elem_bytes must be 1, 2, 4 or 8");
  if (R < 1 || S < 0 || S % R) return fail(RA_ERR_SHAPE, "need R >= 1, S >= 0, S %% R == 0");
  if (S > kMaxI32) return fail(RA_ERR_SHAPE, "S must be < 2^31");
  if (B < 0 || H < 0 || d < 0) return fail(RA_ERR_SHAPE, "negative size");
  if (rank0 < 0 || n_ranks < 0 || rank0 + n_ranks > R)
    return fail(RA_ERR_SHAPE, "ranks [rank0, rank0+n_ranks) must lie in [0, R)");
  if (B * H * S * d * n_ranks == 0) return RA_OK;
  if (!src || !dst || !fwd) return fail(RA_ERR_INVALID_ARG, "null pointer");
  RA_HIP(launch_layout_move(gather, src, dst, fwd, elem_bytes, B, H, S, d, R, rank0, n_ranks,
                            (hipStream_t)stream),
         "layout move kernel");
  return RA_OK;
}

ra_status ra_layout_gather(const void *x, void *x_sh, const int32_t *fwd, int32_t elem_bytes,
                           int64_t B, int64_t H, int64_t S, int64_t d, int32_t R, int32_t rank0,
                           int32_t n_ranks, ra_stream stream) {
  return layout_move(true, x, x_sh, fwd, elem_bytes, B, H, S, d, R, rank0, n_ranks, stream);
}

ra_status ra_layout_scatter(const void *x_sh, void *x, const int32_t *fwd, int32_t elem_bytes,
                            int64_t B, int64_t H, int64_t S, int64_t d, int32_t R, int32_t rank0,
                            int32_t n_ranks, ra_stream stream) {
  return layout_move(false, x_sh, x, fwd, elem_bytes, B, H, S, d, R, rank0, n_ranks, stream);
}

ra_status ra_block_fwd(const ra_block_args *a, ra_stream stream) {
  clear_error();
  ra_status st = check_block(a);
  if (st != RA_OK) return st;
  if (a->n_q == 0) return RA_OK;
  BatchParams p{};
  p.q = a->q;
  p.k = a->n_k > 0 ? a->k : a->q;  // never read when n_k == 0
  p.v = a->n_k > 0 ? a->v : a->q;
  p.q_zstride = 0;
  p.kv_zstride = 0;
  p.kv_vzstride = 0;
  p.kv_idx0 = 0;
  p.kv_idx_mod = 1;
  p.qs_b = a->q_stride[0];
  p.qs_h = a->q_stride[1];
  p.qs_t = a->q_stride[2];
  p.ks_b = a->k_stride[0];
  p.ks_h = a->k_stride[1];
  p.ks_t = a->k_stride[2];
  p.v_packed = a->v_packed;
  if (a->v_packed) {
    const int64_t np = packed_n(a->n_k);
    p.vs_b = (int64_t)a->Hkv * a->d * np;
    p.vs_h = (int64_t)a->d * np;
    p.vs_t = np;
  } else {
    p.vs_b = a->v_stride[0];
    p.vs_h = a->v_stride[1];
    p.vs_t = a->v_stride[2];
  }
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.nq = a->n_q;
  p.nk = a->n_k;
  p.d = a->d;
  p.nz = 1;
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.qg_add = a->q_gid0;
  p.qg_z = 0;
  p.q_step = a->q_gid_step;
  p.kg_add = a->k_gid0;
  p.kg_mult = 0;
  p.k_step = a->k_gid_step;
  p.kg_s0 = 0;
  p.kg_smod = 1;
  p.o = a->o;
  p.o_zstride = 0;
  p.os_b = a->o_stride[0];
  p.os_h = a->o_stride[1];
  p.os_t = a->o_stride[2];
  p.m = a->m;
  p.l = a->l;
  p.ml_zstride = 0;
  p.accumulate = 0;
  p.exact_m = 1;
  RA_HIP(launch_block_fwd(p, a->dtype, (hipStream_t)stream), "block kernel");
  return RA_OK;
}

size_t ra_packed_v_bytes(int32_t dtype, int32_t B, int32_t H, int32_t n, int32_t d) {
  clear_error();
  if (dtype != RA_DT_BF16 && dtype != RA_DT_FP16) {
    fail(RA_ERR_DTYPE, "packed V is for bf16/fp16");
    return 0;
  }
  if (B < 0 || H < 0 || n < 0 || d < 0) {
    fail(RA_ERR_SHAPE, "negative size");
    return 0;
  }
  return (size_t)B * H * d * packed_n(n) * 2;
}

ra_status ra_pack_v(const void *v, void *vp, int32_t dtype, int32_t B, int32_t H, int32_t n,
                    int32_t d, const int64_t v_stride[3], ra_stream stream) {
  clear_error();
  if (dtype != RA_DT_BF16 && dtype != RA_DT_FP16)
    return fail(RA_ERR_DTYPE, "packed V is for bf16/fp16");
  if (B < 0 || H < 0 || n < 0) return fail(RA_ERR_SHAPE, "negative size");
  if (d != 64 && d != 128) return fail(RA_ERR_SHAPE, "d must be 64 or 128 (got %d)", d);
  if ((int64_t)B * H * n == 0) return RA_OK;
  if (!v || !vp || !v_stride) return fail(RA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(v) || !aligned16(vp)) return fail(RA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (v_stride[i] < 0) return fail(RA_ERR_SHAPE, "negative stride");
    if ((v_stride[i] * 2) % 16) return fail(RA_ERR_ALIGNMENT, "strides must keep rows 16-byte aligned");
  }
  if (v_stride[2] < d) return fail(RA_ERR_SHAPE, "token stride smaller than d");
  RA_HIP(launch_pack_v(v, vp, 2, (int64_t)B * H, H, n, d, v_stride[0], v_stride[1], v_stride[2],
                       (hipStream_t)stream),
         "pack kernel");
  return RA_OK;
}

ra_status ra_handoff_copy(void *dst, const void *src, size_t bytes, int32_t thin,
                          ra_stream stream) {
  clear_error();
  if (thin != 0 && thin != 1) return fail(RA_ERR_INVALID_ARG, "thin must be 0 or 1");
  if (bytes == 0) return RA_OK;
  if (!dst || !src) return fail(RA_ERR_INVALID_ARG, "null pointer");
  RA_HIP(launch_handoff_copy(dst, src, bytes, (hipStream_t)stream, thin != 0), "hand-off copy");
  return RA_OK;
}

int32_t ra_handoff_thin(double moved_bytes, double pairs_heads, int32_t d, double work) {
  return thin_handoff(moved_bytes, pairs_heads, d, work) ? 1 : 0;
}

ra_status ra_merge(float *o_acc, float *m_acc, float *l_acc, const float *o_blk,
                   const float *m_blk, const float *l_blk, int64_t rows, int32_t d,
                   ra_stream stream) {
  clear_error();
  if (rows < 0 || d < 0 || d % 4) return fail(RA_ERR_SHAPE, "rows >= 0 and d %% 4 == 0 required");
  if (rows == 0 || d == 0) return RA_OK;
  if (!o_acc || !m_acc || !l_acc || !o_blk || !m_blk || !l_blk)
    return fail(RA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(o_acc) || !aligned16(o_blk))
    return fail(RA_ERR_ALIGNMENT, "o pointers must be 16-byte aligned");
  RA_HIP(launch_merge(o_acc, m_acc, l_acc, o_blk, m_blk, l_blk, rows, d, (hipStream_t)stream),
         "merge kernel");
  return RA_OK;
}

ra_status ra_finalize(const float *o_acc, const float *m, const float *l, void *out, float *lse,
                      int32_t dtype, int64_t rows, int32_t d, ra_stream stream) {
  clear_error();
  if (!elt_bytes(dtype)) return fail(RA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (rows < 0 || d < 0 || d % 4) return fail(RA_ERR_SHAPE, "rows >= 0 and d %% 4 == 0 required");
  if (rows == 0 || d == 0) return RA_OK;
  if (!o_acc || !m || !l || !out || !lse) return fail(RA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(o_acc)) return fail(RA_ERR_ALIGNMENT, "o_acc must be 16-byte aligned");
  RA_HIP(launch_finalize(o_acc, m, l, out, lse, dtype, rows, d, (hipStream_t)stream),
         "finalize kernel");
  return RA_OK;
}

size_t ra_ring_fwd_workspace_size(const ra_ring_args *a) {
  clear_error();
  if (check_ring(a) != RA_OK) return 0;
  return ws_layout(a).total;
}

ra_status ra_ring_fwd(const ra_ring_args *a, void *workspace, size_t workspace_bytes,
                      ra_stream compute_s, ra_stream copy_s) {
  clear_error();
  ra_status st = check_ring(a);
  if (st != RA_OK) return st;
  if (a->n == 0) return RA_OK;
  const WsLayout L = ws_layout(a);
  if (!workspace || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", L.total, workspace_bytes);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(RA_ERR_ALIGNMENT, "workspace must be 256-byte aligned");

  hipStream_t cs = (hipStream_t)compute_s, xs = (hipStream_t)copy_s;
  char *ws = (char *)workspace;
  const int R = a->R, n = a->n, nr = a->n_ranks, r0 = a->rank0;
  const bool contig = a->layout == RA_LAYOUT_CONTIGUOUS;
  const int elt = elt_bytes(a->dtype);
  const int64_t blk = (int64_t)a->B * a->Hkv * n * a->d;  // elements of one K block
  const size_t blk_bytes = (size_t)blk * elt;
  const bool packed = ring_packs_v(a);
  const int64_t n_pad = packed ? packed_n(n) : n;
  const int64_t blkv = (int64_t)a->B * a->Hkv * a->d * n_pad;  // elements of one V block
  const size_t blkv_bytes = (size_t)blkv * elt;
  // The side copy's form: thin where the hop's products outlast its bytes
  // (it runs beside the block kernel), else the 64-workgroup copy.
  const bool thin = thin_handoff(2.0 * (double)nr * (blk_bytes + blkv_bytes),
                                 (double)nr * a->B * a->Hq * (double)n * n *
                                     (a->causal ? 0.5 : 1.0),
                                 a->d, 1.0);
  // moving: blocks travel through the receive buffers (COPY, FORWARD).  In
  // FORWARD mode, on the packed path and on hops too short for the thin copy
  // to hide (the side copy would compete with the block kernel for memory),
  // the block kernel writes each block whose next holder is a computed rank
  // itself; side copies carry the rest (blocks entering from ranks that are
  // not computed; none on a full ring).  On long hops FORWARD copies as COPY:
  // the thin copy costs the kernel nothing there, and the forwarding
  // instantiation of the d = 128 kernel measured 4 % slower per launch than
  // the plain one (compiler scheduling of its tile loop), more than the copy.
  const bool moving = a->handoff != RA_HANDOFF_SWAP && R > 1;
  const bool in_kernel = moving && a->handoff == RA_HANDOFF_FORWARD && packed && !thin;
  const bool copy = moving && !(in_kernel && nr == R);
  const int64_t qz = (int64_t)a->B * a->Hq * n * a->d;
  const int64_t rows = (int64_t)nr * a->B * a->Hq * n;
  float *o_acc = (float *)(ws + L.o_acc), *m_acc = (float *)(ws + L.m_acc),
        *l_acc = (float *)(ws + L.l_acc);
  float *o_blk = (float *)(ws + L.o_blk), *m_blk = (float *)(ws + L.m_blk),
        *l_blk = (float *)(ws + L.l_blk);
  const char *ksh = (const char *)a->k_sh;
  const char *vsh = packed ? (const char *)(ws + L.vpack) : (const char *)a->v_sh;
  char *kb[2] = {ws + L.kbuf[0], ws + L.kbuf[1]};
  char *vb[2] = {ws + L.vbuf[0], ws + L.vbuf[1]};

  EventLease lease;
  RA_HIP(lease.acquire((size_t)2 * R + 2), "hipEventCreate");
  const std::vector<hipEvent_t> &ev = lease.ev;
  hipEvent_t ev_entry = ev[0], ev_join = ev[1];
  auto ev_comp = [&](int h) { return ev[2 + 2 * h]; };
  auto ev_copy = [&](int h) { return ev[3 + 2 * h]; };

  // V of every source block in the packed layout the block kernel reads
  if (packed)
    RA_HIP(launch_pack_v(a->v_sh, ws + L.vpack, elt, (int64_t)R * a->B * a->Hkv, a->Hkv, n, a->d,
                         (int64_t)a->Hkv * n * a->d, (int64_t)n * a->d, a->d, cs),
           "pack kernel");
  if (copy) {
    RA_HIP(hipEventRecord(ev_entry, cs), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(xs, ev_entry, 0), "hipStreamWaitEvent");
  }

  // block pointer that computed rank index k holds at hop h (copy mode)
  auto front = [&](const char *sh, char *const *buf, size_t bbytes, int h, int k) -> const char * {
    if (h == 0) return sh + (size_t)((r0 + k) % R) * bbytes;
    return buf[(h - 1) & 1] + (size_t)k * bbytes;
  };

  BatchParams p{};
  p.q = a->q_sh;
  p.q_zstride = qz;
  p.kv_zstride = blk;
  p.kv_vzstride = blkv;
  p.v_packed = packed ? 1 : 0;
  p.qs_b = (int64_t)a->Hq * n * a->d;
  p.qs_h = (int64_t)n * a->d;
  p.qs_t = a->d;
  p.ks_b = (int64_t)a->Hkv * n * a->d;
  p.ks_h = (int64_t)n * a->d;
  p.ks_t = a->d;
  p.vs_b = (int64_t)a->Hkv * a->d * n_pad;
  p.vs_h = (int64_t)a->d * n_pad;
  p.vs_t = n_pad;
  if (!packed) {
    p.vs_b = p.ks_b;
    p.vs_h = p.ks_h;
    p.vs_t = p.ks_t;
  }
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.nq = n;
  p.nk = n;
  p.d = a->d;
  p.nz = nr;
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.qg_add = contig ? (int64_t)r0 * n : r0;
  p.qg_z = contig ? n : 1;
  p.q_step = contig ? 1 : R;
  p.kg_add = 0;
  p.kg_mult = contig ? n : 1;
  p.k_step = contig ? 1 : R;
  p.kg_smod = R;
  if (a->layout == RA_LAYOUT_ZIGZAG) {  // two affine chunks per rank
    p.zz_c = n / 2;
    p.zz_R = R;
    p.q_rank0 = r0;
  }
  p.o_zstride = qz;
  p.os_b = p.qs_b;
  p.os_h = p.qs_h;
  p.os_t = a->d;
  p.ml_zstride = (int64_t)a->B * a->Hq * n;

  const DebugDelay dbg = debug_delay();
  for (int h = 0; h < R; ++h) {
    // ---- compute hop h: every computed rank r attends to the block of source (r - h) mod R
    if (copy && h > 0) RA_HIP(hipStreamWaitEvent(cs, ev_copy(h - 1), 0), "hipStreamWaitEvent");
    RA_HIP(launch_delay(dbg.compute, cs), "delay kernel");
    p.kg_s0 = ((r0 - h) % R + R) % R;
    if (moving && h > 0) {
      p.k = kb[(h - 1) & 1];
      p.v = vb[(h - 1) & 1];
      p.kv_idx0 = 0;
      p.kv_idx_mod = nr;
    } else if (moving) {
      p.k = ksh;
      p.v = vsh;
      p.kv_idx0 = r0;
      p.kv_idx_mod = R;
    } else {
      p.k = ksh;
      p.v = vsh;
      p.kv_idx0 = p.kg_s0;
      p.kv_idx_mod = R;
    }
    const bool into_acc = a->merge_mode == RA_MERGE_FUSED || h == 0;
    p.o = into_acc ? o_acc : o_blk;
    p.m = into_acc ? m_acc : m_blk;
    p.l = into_acc ? l_acc : l_blk;
    p.accumulate = (a->merge_mode == RA_MERGE_FUSED && h > 0) ? 1 : 0;
    // the fused state only needs m + ln l; a separate partial is merged by m
    p.exact_m = a->merge_mode == RA_MERGE_FUSED ? 0 : 1;
    // FORWARD: computed rank k hands its block to computed rank k + 1 (on a
    // full ring the last one to rank 0) through buffer h & 1, which hop h+1
    // reads and hop h-1 was the last to read (same stream)
    p.fwd = (in_kernel && h + 1 < R) ? 1 : 0;
    p.fk = kb[h & 1];
    p.fv = vb[h & 1];
    p.fwd_wrap = nr == R ? 1 : 0;
    if (a->hop_events)
      RA_HIP(hipEventRecord((hipEvent_t)a->hop_events[2 * h], cs), "hipEventRecord");
    RA_HIP(launch_block_fwd(p, a->dtype, cs), "block kernel");
    if (a->hop_events)
      RA_HIP(hipEventRecord((hipEvent_t)a->hop_events[2 * h + 1], cs), "hipEventRecord");
    if (!into_acc)
      RA_HIP(launch_merge(o_acc, m_acc, l_acc, o_blk, m_blk, l_blk, rows, a->d, cs),
             "merge kernel");
    if (!copy || h + 1 >= R) continue;
    RA_HIP(hipEventRecord(ev_comp(h), cs), "hipEventRecord");
    // ---- hand-off for hop h+1 on the copy stream: rank r receives what its
    // ring predecessor r-1 holds now.  The destination buffer was last read by
    // hop h-1's compute.
    if (h >= 1) RA_HIP(hipStreamWaitEvent(xs, ev_comp(h - 1), 0), "hipStreamWaitEvent");
    RA_HIP(launch_delay(dbg.copy, xs), "delay kernel");
    for (int t = 0; t < 2; ++t) {
      const char *sh = t ? vsh : ksh;
      char *const *buf = t ? vb : kb;
      const size_t bb = t ? blkv_bytes : blk_bytes;
      char *dst_base = buf[h & 1];
      const char *run_src = nullptr;
      char *run_dst = nullptr;
      size_t run_len = 0;
      for (int k = 0; k < nr; ++k) {
        const int r = r0 + k;
        const int rp = (r - 1 + R) % R;
        const int kp = ((rp - r0) % R + R) % R;
        if (in_kernel && kp < nr) continue;  // written by the block kernel of rank kp
        const char *src = kp < nr ? front(sh, buf, bb, h, kp)
                                  : sh + (size_t)(((r - 1 - h) % R + R) % R) * bb;
        char *dst = dst_base + (size_t)k * bb;
        if (run_len && src == run_src + run_len && dst == run_dst + run_len) {
          run_len += bb;
          continue;
        }
        if (run_len) RA_HIP(launch_handoff_copy(run_dst, run_src, run_len, xs, thin), "hand-off copy");
        run_src = src;
        run_dst = dst;
        run_len = bb;
      }
      if (run_len) RA_HIP(launch_handoff_copy(run_dst, run_src, run_len, xs, thin), "hand-off copy");
    }
    RA_HIP(hipEventRecord(ev_copy(h), xs), "hipEventRecord");
  }
  if (copy) {
    RA_HIP(hipEventRecord(ev_join, xs), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(cs, ev_join, 0), "hipStreamWaitEvent");
  }
  RA_HIP(launch_finalize(o_acc, m_acc, l_acc, a->o, a->lse, a->dtype, rows, a->d, cs),
         "finalize kernel");
  return RA_OK;
}

size_t ra_block_bwd_workspace_size(const ra_block_bwd_args *a) {
  clear_error();
  if (check_block_bwd(a) != RA_OK) return 0;
  return block_bwd_ws(a).total;
}

ra_status ra_block_bwd(const ra_block_bwd_args *a, void *workspace, size_t workspace_bytes,
                       ra_stream stream) {
  clear_error();
  ra_status st = check_block_bwd(a);
  if (st != RA_OK) return st;
  if (a->n_q == 0) return RA_OK;
  const BwdWs L = block_bwd_ws(a);
  if (!workspace || workspace_bytes < L.total || (uintptr_t)workspace % 256)
    return fail(RA_ERR_WORKSPACE, "workspace must be >= %zu bytes, 256-byte aligned", L.total);
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  const int64_t d = a->d;
  const int64_t qs[3] = {(int64_t)a->Hq * a->n_q * d, (int64_t)a->n_q * d, d};
  const int64_t ks[3] = {(int64_t)a->Hkv * a->n_k * d, (int64_t)a->n_k * d, d};
  RA_HIP(launch_bwd_prep(a->o, a->dout, a->lse, (float *)(ws + L.nd), (float *)(ws + L.nl),
                         a->dtype, (int64_t)a->B * a->Hq * a->n_q, a->d, s), "bwd prep");
  RA_HIP(launch_pack_v(a->q, ws + L.qT, 2, (int64_t)a->B * a->Hq, a->Hq, a->n_q, d, qs[0], qs[1],
                       qs[2], s), "pack q");
  RA_HIP(launch_pack_v(a->dout, ws + L.doT, 2, (int64_t)a->B * a->Hq, a->Hq, a->n_q, d, qs[0],
                       qs[1], qs[2], s), "pack dout");
  if (a->n_k > 0)
    RA_HIP(launch_pack_v(a->k, ws + L.kT, 2, (int64_t)a->B * a->Hkv, a->Hkv, a->n_k, d, ks[0],
                         ks[1], ks[2], s), "pack k");
  BwdParams P{};
  BatchParams &p = P.a;
  p.q = a->q;
  p.k = a->n_k > 0 ? a->k : a->q;
  p.v = a->n_k > 0 ? a->v : a->q;
  p.kv_idx0 = 0;
  p.kv_idx_mod = 1;
  p.qs_b = qs[0];
  p.qs_h = qs[1];
  p.qs_t = qs[2];
  p.ks_b = p.vs_b = ks[0];
  p.ks_h = p.vs_h = ks[1];
  p.ks_t = p.vs_t = ks[2];
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.nq = a->n_q;
  p.nk = a->n_k;
  p.d = a->d;
  p.nz = 1;
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.qg_add = a->q_gid0;
  p.q_step = a->q_gid_step;
  p.kg_add = a->k_gid0;
  p.k_step = a->k_gid_step;
  p.kg_smod = 1;
  P.dout = a->dout;
  P.qT = ws + L.qT;
  P.doT = ws + L.doT;
  P.kT = ws + L.kT;
  P.nl = (const float *)(ws + L.nl);
  P.nD = (const float *)(ws + L.nd);
  P.dq = a->dq;
  P.dk = a->dk;
  P.dv = a->dv;
  RA_HIP(launch_bwd(P, a->dtype, s), "backward kernels");
  return RA_OK;
}

size_t ra_ring_bwd_workspace_size(const ra_ring_bwd_args *a) {
  clear_error();
  if (check_ring_bwd(a) != RA_OK) return 0;
  return ring_bwd_ws(a).total;
}

ra_status ra_ring_bwd(const ra_ring_bwd_args *a, void *workspace, size_t workspace_bytes,
                      ra_stream compute_s, ra_stream copy_s) {
  clear_error();
  ra_status st = check_ring_bwd(a);
  if (st != RA_OK) return st;
  if (a->n == 0) return RA_OK;
  const RingBwdWs L = ring_bwd_ws(a);
  if (!workspace || workspace_bytes < L.total || (uintptr_t)workspace % 256)
    return fail(RA_ERR_WORKSPACE, "workspace must be >= %zu bytes, 256-byte aligned", L.total);
  hipStream_t s = (hipStream_t)compute_s, xs = (hipStream_t)copy_s;
  char *ws = (char *)workspace;
  const int R = a->R, n = a->n, nr = a->n_ranks, r0 = a->rank0;
  const bool copy = a->handoff != RA_HANDOFF_SWAP && R > 1;  // FORWARD moves like COPY here
  const int64_t d = a->d;
  const bool contig = a->layout == RA_LAYOUT_CONTIGUOUS;
  const int64_t qz = (int64_t)a->B * a->Hq * n * d;   // elements of one query shard
  const int64_t kz = (int64_t)a->B * a->Hkv * n * d;  // elements of one K/V block
  const int64_t n_pad = packed_n(n);
  const int64_t kTz = (int64_t)a->B * a->Hkv * d * n_pad;  // elements of one packed K^T block
  float *dq = (float *)(ws + L.dq), *dk = (float *)(ws + L.dk), *dv = (float *)(ws + L.dv);
  EventLease lease;
  if (copy) RA_HIP(lease.acquire((size_t)3 * R + 2), "hipEventCreate");
  const std::vector<hipEvent_t> &ev = lease.ev;
  RA_HIP(launch_zero(dq, nr * qz, s), "zero dq");
  RA_HIP(launch_zero(dk, R * kz, s), "zero dk");
  RA_HIP(launch_zero(dv, R * kz, s), "zero dv");
  RA_HIP(launch_bwd_prep(a->o_sh, a->dout_sh, a->lse, (float *)(ws + L.D), (float *)(ws + L.nl),
                         a->dtype, (int64_t)nr * a->B * a->Hq * n, a->d, s), "bwd prep");
  RA_HIP(launch_pack_v(a->q_sh, ws + L.qT, 2, (int64_t)nr * a->B * a->Hq, a->Hq, n, d,
                       (int64_t)a->Hq * n * d, (int64_t)n * d, d, s), "pack q");
  RA_HIP(launch_pack_v(a->dout_sh, ws + L.doT, 2, (int64_t)nr * a->B * a->Hq, a->Hq, n, d,
                       (int64_t)a->Hq * n * d, (int64_t)n * d, d, s), "pack dout");
  RA_HIP(launch_pack_v(a->k_sh, ws + L.kT, 2, (int64_t)R * a->B * a->Hkv, a->Hkv, n, d,
                       (int64_t)a->Hkv * n * d, (int64_t)n * d, d, s), "pack k");
  BwdParams P{};
  BatchParams &p = P.a;
  p.q = a->q_sh;
  p.q_zstride = qz;
  p.kv_zstride = kz;
  p.kv_vzstride = kz;
  p.qs_b = (int64_t)a->Hq * n * d;
  p.qs_h = (int64_t)n * d;
  p.qs_t = d;
  p.ks_b = p.vs_b = (int64_t)a->Hkv * n * d;
  p.ks_h = p.vs_h = (int64_t)n * d;
  p.ks_t = p.vs_t = d;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.nq = n;
  p.nk = n;
  p.d = a->d;
  p.nz = nr;
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.qg_add = contig ? (int64_t)r0 * n : r0;
  p.qg_z = contig ? n : 1;
  p.q_step = contig ? 1 : R;
  p.kg_add = 0;
  p.kg_mult = contig ? n : 1;
  p.k_step = contig ? 1 : R;
  p.kg_smod = R;
  if (a->layout == RA_LAYOUT_ZIGZAG) {
    p.zz_c = n / 2;
    p.zz_R = R;
    p.q_rank0 = r0;
  }
  p.ml_zstride = (int64_t)a->B * a->Hq * n;
  P.dout = a->dout_sh;
  P.qT = ws + L.qT;
  P.doT = ws + L.doT;
  P.qT_zstride = (int64_t)a->B * a->Hq * d * n_pad;
  P.kT_zstride = kTz;
  P.nl = (const float *)(ws + L.nl);
  P.nD = (const float *)(ws + L.D);
  P.dq = dq;
  P.dq_zstride = qz;
  P.dk_zstride = kz;

  // One travelling quantity of a block: its copy at home (block index s of a
  // home array with `bytes` per block) and the two receive buffers (computed
  // rank k at offset k*bytes).  At hop h computed rank k holds, in COPY mode,
  // home[(r0 + k) mod R] for h = 0 and buf[(h - 1) & 1][k] after that.
  struct Part {
    char *home;
    char *buf[2];
    size_t bytes;
  };
  const Part parts[5] = {
      {(char *)a->k_sh, {ws + L.kbuf[0], ws + L.kbuf[1]}, (size_t)kz * 2},
      {(char *)a->v_sh, {ws + L.vbuf[0], ws + L.vbuf[1]}, (size_t)kz * 2},
      {ws + L.kT, {ws + L.kTbuf[0], ws + L.kTbuf[1]}, (size_t)kTz * 2},
      {(char *)dk, {ws + L.dkbuf[0], ws + L.dkbuf[1]}, (size_t)kz * 4},
      {(char *)dv, {ws + L.dvbuf[0], ws + L.dvbuf[1]}, (size_t)kz * 4}};
  auto front = [&](const Part &x, int h, int k) -> char * {
    if (h == 0) return x.home + (size_t)((r0 + k) % R) * x.bytes;
    return x.buf[(h - 1) & 1] + (size_t)k * x.bytes;
  };
  // copies merged into contiguous runs (one launch per run)
  struct Runs {
    char *dst = nullptr;
    const char *src = nullptr;
    size_t len = 0;
  };
  // the backward hop's kernels do about 3.2 times the forward's MFMA work
  const bool thin = thin_handoff(
      2.0 * (double)nr * (parts[0].bytes + parts[1].bytes + parts[2].bytes + parts[3].bytes +
                          parts[4].bytes),
      (double)nr * a->B * a->Hq * (double)n * n * (a->causal ? 0.5 : 1.0), a->d, 3.2);
  auto add_copy = [&](Runs &r, char *dst, const char *src, size_t bytes) -> ra_status {
    if (r.len && src == r.src + r.len && dst == r.dst + r.len) {
      r.len += bytes;
      return RA_OK;
    }
    if (r.len) RA_HIP(launch_handoff_copy(r.dst, r.src, r.len, xs, thin), "hand-off copy");
    r.dst = dst;
    r.src = src;
    r.len = bytes;
    return RA_OK;
  };
  auto flush = [&](Runs &r) -> ra_status {
    if (r.len) RA_HIP(launch_handoff_copy(r.dst, r.src, r.len, xs, thin), "hand-off copy");
    r.len = 0;
    return RA_OK;
  };
  // before hop h+1 rank k receives what its ring predecessor held at hop h:
  // the front of computed rank k-1, or (predecessor not computed here) the
  // block's home copy -- where a block's accumulators also wait while it
  // passes ranks outside the computed set
  auto hand_off = [&](int h, int first, int last) -> ra_status {
    for (int pi = first; pi <= last; ++pi) {
      const Part &x = parts[pi];
      Runs run;
      for (int k = 0; k < nr; ++k) {
        const int r = r0 + k;
        const int kp = ((r - 1 - r0) % R + R) % R;
        const char *src = kp < nr ? front(x, h, kp)
                                  : x.home + (size_t)(((r - 1 - h) % R + R) % R) * x.bytes;
        if ((st = add_copy(run, x.buf[h & 1] + (size_t)k * x.bytes, src, x.bytes)) != RA_OK)
          return st;
      }
      if ((st = flush(run)) != RA_OK) return st;
    }
    return RA_OK;
  };
  // accumulators of computed rank k's block go home (it leaves the computed
  // set, or the ring has ended); at h = 0 the front is the home copy
  auto send_home = [&](int h, int k) -> ra_status {
    if (h == 0) return RA_OK;
    const int src_rank = ((r0 + k - h) % R + R) % R;
    for (int pi = 3; pi <= 4; ++pi)
      RA_HIP(launch_handoff_copy(parts[pi].home + (size_t)src_rank * parts[pi].bytes,
                                 front(parts[pi], h, k), parts[pi].bytes, xs, thin),
             "hand-off copy");
    return RA_OK;
  };

  hipEvent_t ev_entry = copy ? ev[0] : nullptr, ev_join = copy ? ev[1] : nullptr;
  auto ev_comp = [&](int h) { return ev[2 + 3 * h]; };     // hop h's kernels done
  auto ev_kv = [&](int h) { return ev[3 + 3 * h]; };       // K, V, K^T of hop h+1 in place
  auto ev_acc = [&](int h) { return ev[4 + 3 * h]; };      // dK, dV of hop h+1 in place
  if (copy) {
    RA_HIP(hipEventRecord(ev_entry, s), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(xs, ev_entry, 0), "hipStreamWaitEvent");
  }
  const DebugDelay dbg = debug_delay();
  for (int h = 0; h < R; ++h) {
    // hop h: computed rank r0 + z meets the block of source (r0 + z - h) mod R
    p.kg_s0 = ((r0 - h) % R + R) % R;
    if (copy) {
      p.k = front(parts[0], h, 0);
      p.v = front(parts[1], h, 0);
      P.kT = front(parts[2], h, 0);
      P.dk = (float *)front(parts[3], h, 0);
      P.dv = (float *)front(parts[4], h, 0);
      p.kv_idx0 = 0;
      p.kv_idx_mod = h == 0 ? R : nr;
      if (h == 0) {  // blocks at home: computed rank z holds block (r0 + z) mod R
        p.k = a->k_sh;
        p.v = a->v_sh;
        P.kT = ws + L.kT;
        P.dk = dk;
        P.dv = dv;
        p.kv_idx0 = r0;
      }
    } else {  // in place: rank z's block is (kg_s0 + z) mod R of the home arrays
      p.k = a->k_sh;
      p.v = a->v_sh;
      P.kT = ws + L.kT;
      P.dk = dk;
      P.dv = dv;
      p.kv_idx0 = p.kg_s0;
      p.kv_idx_mod = R;
    }
    // dQ needs only the block's K and V; dK/dV also the block's accumulators
    if (copy && h > 0) RA_HIP(hipStreamWaitEvent(s, ev_kv(h - 1), 0), "hipStreamWaitEvent");
    RA_HIP(launch_delay(dbg.compute, s), "delay kernel");
    RA_HIP(launch_bwd(P, a->dtype, s, kBwdQ), "backward dq kernel");
    if (copy && h > 0) RA_HIP(hipStreamWaitEvent(s, ev_acc(h - 1), 0), "hipStreamWaitEvent");
    RA_HIP(launch_bwd(P, a->dtype, s, kBwdKV), "backward dk/dv kernels");
    if (!copy) continue;
    RA_HIP(hipEventRecord(ev_comp(h), s), "hipEventRecord");
    if (h + 1 < R) {
      // K, V, K^T for hop h+1: read-only this hop, so they move while hop h
      // computes; the receive buffer was last read by hop h-1
      if (h >= 1) RA_HIP(hipStreamWaitEvent(xs, ev_comp(h - 1), 0), "hipStreamWaitEvent");
      RA_HIP(launch_delay(dbg.copy, xs), "delay kernel");
      if ((st = hand_off(h, 0, 2)) != RA_OK) return st;
      RA_HIP(hipEventRecord(ev_kv(h), xs), "hipEventRecord");
      // the accumulators are final for hop h once its kernels are done; they
      // move during hop h+1's dQ kernel
      RA_HIP(hipStreamWaitEvent(xs, ev_comp(h), 0), "hipStreamWaitEvent");
      RA_HIP(launch_delay(dbg.copy, xs), "delay kernel");
      if ((st = hand_off(h, 3, 4)) != RA_OK) return st;
      const int next = (r0 + nr) % R;  // the rank after the computed set
      if (nr < R && !(next >= r0 && next < r0 + nr))
        if ((st = send_home(h, nr - 1)) != RA_OK) return st;
      RA_HIP(hipEventRecord(ev_acc(h), xs), "hipEventRecord");
    } else {
      RA_HIP(hipStreamWaitEvent(xs, ev_comp(h), 0), "hipStreamWaitEvent");
      for (int k = 0; k < nr; ++k)
        if ((st = send_home(h, k)) != RA_OK) return st;
    }
  }
  if (copy) {
    RA_HIP(hipEventRecord(ev_join, xs), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(s, ev_join, 0), "hipStreamWaitEvent");
  }
  RA_HIP(launch_cast(dq, a->dq_sh, a->dtype, nr * qz, s), "cast dq");
  RA_HIP(launch_cast(dk, a->dk_sh, a->dtype, R * kz, s), "cast dk");
  RA_HIP(launch_cast(dv, a->dv_sh, a->dtype, R * kz, s), "cast dv");
  return RA_OK;
}

size_t ra_decode_fwd_workspace_size(const ra_decode_args *a) {
  clear_error();
  if (check_decode(a) != RA_OK) return 0;
  return decode_ws_bytes(decode_plan(a));
}

ra_status ra_decode_fwd(const ra_decode_args *a, void *workspace, size_t workspace_bytes,
                        ra_stream stream) {
  clear_error();
  ra_status st = check_decode(a);
  if (st != RA_OK) return st;
  DecodeParams p = decode_plan(a);
  const size_t need = decode_ws_bytes(p);
  if (!workspace || workspace_bytes < need || (uintptr_t)workspace % 256)
    return fail(RA_ERR_WORKSPACE, "workspace must be >= %zu bytes, 256-byte aligned", need);
  return run_decode(a, p, (char *)workspace, (hipStream_t)stream);
}

ra_status ra_decode_fwd_noalloc(const ra_decode_args *a, ra_stream stream) {
  clear_error();
  ra_status st = check_decode(a);
  if (st != RA_OK) return st;
  DecodeParams p = decode_plan(a);
  const size_t need = decode_ws_bytes(p);
  if (need > kDecodeScratchBytes)
    return fail(RA_ERR_UNSUPPORTED,
                "these arguments need %zu bytes of partials; the allocation-free decode holds %zu "
                "(use ra_decode_fwd with a workspace)",
                need, kDecodeScratchBytes);
  void *ws = nullptr;
  RA_HIP(decode_scratch(&ws), "scratch address");
  return run_decode(a, p, (char *)ws, (hipStream_t)stream);
}

ra_status ra_causal_work(int32_t layout, int64_t S, int32_t R, int64_t *W) {
  clear_error();
  if (!known_layout(layout)) return fail(RA_ERR_INVALID_ARG, "unknown layout %d", layout);
  if (R < 1 || S < 0 || S % R) return fail(RA_ERR_SHAPE, "need R >= 1, S >= 0, S %% R == 0");
  if (layout == RA_LAYOUT_ZIGZAG && S % (2 * (int64_t)R))
    return fail(RA_ERR_SHAPE, "zig-zag needs S %% 2R == 0");
  if (!W) return fail(RA_ERR_INVALID_ARG, "W is NULL");
  const int64_t n = S / R;
  for (int32_t r = 0; r < R; ++r) {
    int64_t total = 0;
    for (int32_t h = 0; h < R; ++h) {
      const int32_t s = ((r - h) % R + R) % R;
      // key ids increase along the block, so the allowed keys of query i
      // form a prefix: count it by binary search over the block's ids
      for (int64_t i = 0; i < n; ++i) {
        const int64_t gq = layout_gid(layout, R, n, r, i);
        int64_t lo = 0, hi = n;  // first key with id > gq
        while (lo < hi) {
          const int64_t mid = (lo + hi) / 2;
          if (layout_gid(layout, R, n, s, mid) <= gq)
            lo = mid + 1;
          else
            hi = mid;
        }
        total += lo;
      }
    }
    W[r] = total;
  }
  return RA_OK;
}

}  // extern "C"
