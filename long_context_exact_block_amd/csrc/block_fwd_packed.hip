// block_fwd_packed.hip -- the block-attention kernel the ring runs for 16-bit
// inputs, reading V from the packed transposed layout, plus the packing
// kernel.
//
// Same computation as the row-V kernel (partial attention of a query shard
// against one arriving K/V block, folded into the running online-softmax
// state; aiunderstanding.org "Sequenzparallelität und Ringaufmerksamkeit",
// "Tiefer Einblick", and the Thai version's technical-insight section), with
// a layout chosen for gfx950:
//  * V is packed once per block to [d][keys] with the keys of every 16 in the
//    order the PV product consumes probabilities (see packed_n), so the V^T
//    operand of O^T += V^T P^T is a plain 16-byte LDS read like the K operand
//    (the LDS transpose read delivers ~1/3 of the bytes per clock).
//  * K tiles are loaded two tiles ahead and V^T tiles one tile ahead, by
//    buffer loads that write LDS directly (no staging registers), issued by
//    the four waves that start each tile with QK and exponentials; two K and
//    three V^T stages, one barrier per tile, the loop unrolled by two so every
//    K offset is an immediate.  16-byte chunks are XOR-swizzled by row for
//    gfx950's 64 LDS banks so every read pattern is conflict-free.
//  * 8 waves x 32 queries per workgroup (256 rows), two waves per SIMD; QK of
//    tile t+1 is interleaved with the exponentials of tile t; K fragments are
//    read one k-step ahead (245 VGPRs: two waves leave room on each SIMD for
//    the one-wave hand-off copy) and V^T fragments one PV group ahead.  In the
//    fused ring the upper four waves run PV half a tile late (before instead
//    of after the QK/exponential phase), so the waves sharing a SIMD are in
//    opposite phases.
//  * Between hops only m + ln l matters, so the fused ring skips the per-tile
//    row max: exponentials use the running maximum and a tile whose
//    probabilities grow too large is redone after raising it.
//  * Grouped heads (2, 4 or 8 query heads per K/V head): a workgroup serves
//    all query heads of its K/V head from each loaded tile, 256 / group rows of
//    each (same-run: as fast as one head per workgroup -- each tile already
//    serves 256 rows, and the heads' workgroups ran together on one XCD).
//  * At d = 64 in the fused ring a lean variant (attn_lean64_kernel) trades the
//    in-wave pipelining for registers, so two workgroups share a CU.
//  * Forwarding instantiations (the ring's FORWARD hand-off on short hops)
//    also write the K/V block they stream to the next rank's receive buffer
//    (the highthink.cn Ring Attention article, "Zig Zag Ring Attention
//    通信和计算重叠": a rank passes on the block it holds while it computes).
#include <cfloat>
#include <cmath>
#include <type_traits>

#include "attn_common.h"

namespace ra {
namespace {

using namespace attn;

constexpr int kPW = 8;          // waves per workgroup
constexpr int kPBM = kPW * 32;  // query rows per workgroup
constexpr int kPBN = 64;        // keys per tile
constexpr int kLW = kPW / 2;    // waves that issue the tile loads (waves 0 .. kLW-1)

// key held by packed position q (an involution: quads 1 and 2 of each 16 swap)
__device__ __forceinline__ int perm16(int q) {
  const int quad = (q >> 2) & 3;
  const int sq = (quad == 1) ? 2 : (quad == 2 ? 1 : quad);
  return (q & ~15) | (sq << 2) | (q & 3);
}

// LDS has 64 four-byte banks on gfx950; a 16-lane group reading 16 bytes each
// is conflict-free when its 16 addresses fall on 16 distinct 16-byte bank
// groups.  Rows of 256 bytes (K, d = 128) start on the same bank: swizzle the
// 16-byte chunk by row & 15.  Rows of 128 bytes (K at d = 64, every V^T tile)
// alternate between the two halves of the banks: swizzle by (row >> 1) & 7.
template <int ROW_BYTES>
__device__ __forceinline__ int chunk_swz(int row) {
  return ROW_BYTES == 256 ? (row & 15) : ((row >> 1) & 7);
}

// Raw buffer descriptor word 3 for gfx9-family parts: 32-bit dword data, no
// swizzle, no index stride.
constexpr int kBufWord3 = 0x00020000;
// s_waitcnt immediate waiting for vmcnt == 0 only (lgkmcnt, expcnt at max)
constexpr int kWaitVm0 = 0x0F70;
// cache policy of the forwarded tiles' stores (and direct loads): non-temporal, so
// they do not evict the K/V tiles the workgroups running beside reuse from L2
constexpr int kNT = 2;
typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes per lane

// Workgroup barrier for the tile loop of the forwarding kernels: global
// stores issued before it (the forwarded K/V tiles) stay in flight across it.
// A memory fence would wait for them too (it cannot tell them from the loads
// into LDS, which count on the same counter), so the ordering is explicit:
// each loading wave has waited for its own loads into LDS before it arrives,
// and every wave's LDS reads are complete (lgkmcnt 0); the asm statement
// keeps the compiler from moving memory operations across the barrier.
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("s_barrier" ::: "memory");
}

// 16 bytes per lane from a raw buffer straight into LDS: lane l's bytes land
// at dst + 16 l (dst is wave-uniform; it goes to M0).  A plain device function:
// used directly in the kernel template, the builtin keeps the host pass from
// emitting the kernel's launch stub.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, lds_void *dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, soff, 0, 0);
}

// EXACT: track the exact row maximum so that the stored m is the row max of
// this call's scores (a block partial's statistic).  Otherwise the stored m is
// the running reference maximum the stored l is relative to (same m + ln l),
// which is all a state carried from hop to hop needs; the exponentials are then
// taken against the running maximum without a per-tile row max, and a tile
// whose probabilities would exceed 2^kTau (a larger maximum arrived) is redone
// after rescaling.
template <int D, bool BF16, bool EXACT, bool FWD>
__global__ void __launch_bounds__(512) attn_packed_kernel(BatchParams p, int ntq, int hshift) {
  using M = Mfma16<BF16>;
  constexpr int KS = D / 16;             // k-steps of the QK product
  constexpr int DT = D / 32;             // 32-wide d tiles of O
  constexpr int KROW = D * 2;            // bytes per K row in LDS
  constexpr int KTILE = kPBN * KROW;     // bytes of a K tile
  constexpr int VROW = kPBN * 2;         // bytes per V^T row (64 keys)
  constexpr int VTILE = D * VROW;        // bytes of a V^T tile
  constexpr int VBASE = 2 * KTILE;       // LDS: K stages 0, 1, then V^T stages 0, 1, 2
  constexpr int KPW = KTILE / 1024 / kLW;  // 1 KB wave-loads per loading wave per K tile
  constexpr int VPW = VTILE / 1024 / kLW;
  constexpr int KRPI = 1024 / KROW;      // K rows per wave-load
  constexpr int CPR = D / 8;             // 16-byte chunks per K row
  constexpr int KA = 1;                  // K fragment read-ahead (k-steps)
  static_assert(KPW * kLW * 1024 == KTILE && VPW * kLW * 1024 == VTILE, "tile must split over the waves");
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  // the wave index is uniform: keep it in a scalar register
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // 2^hshift query heads of a K/V group per workgroup (GQA): wave w serves head
  // w >> (3 - hshift) of the group, rows of its 256 >> hshift
  Work w = hshift ? decode_items(p, ntq, 1) : decode(p, ntq);
  w.h += wave >> (3 - hshift);
  const int wave_r = wave & ((kPW >> hshift) - 1);  // the wave's 32-row slot in its head's rows
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;

  const short *qp = (const short *)p.q + w.z * p.q_zstride + w.b * p.qs_b + w.h * p.qs_h;
  const int kvi = (p.kv_idx0 + w.z) % p.kv_idx_mod;
  const short *kp = (const short *)p.k + kvi * p.kv_zstride + w.b * p.ks_b + w.kvh * p.ks_h;
  const short *vp = (const short *)p.v + kvi * p.kv_vzstride + w.b * p.vs_b + w.kvh * p.vs_h;
  const IdMap qid = query_ids(p, w.z), kid = key_ids(p, w.z);
  const float c = p.scale * kLog2e;

  const int i_wg0 = w.qtile * (kPBM >> hshift);
  const int i_wg1 = min(p.nq, i_wg0 + (kPBM >> hshift)) - 1;
  const int iw0 = i_wg0 + wave_r * 32;
  const int iw1 = min(p.nq - 1, iw0 + 31);
  const bool wave_rows = iw0 < p.nq;
  const int i = iw0 + c32;
  const bool valid = i < p.nq;

  const int kv_wg = key_prefix(p, kid, qid(i_wg1));
  const int ntiles = (kv_wg + kPBN - 1) / kPBN;
  const int kv_wl = wave_rows ? key_prefix(p, kid, qid(iw1)) : 0;
  const int kv_wf = wave_rows ? key_prefix(p, kid, qid(iw0)) : 0;
  const int ntiles_w = (kv_wl + kPBN - 1) / kPBN;
  const int nfull_w = kv_wf / kPBN;
  const int jlim = key_prefix(p, kid, qid(i));
  // FWD: this workgroup's share [f0, f1) of the block's 64-key tiles, written
  // to the next rank's receive buffer (tiles split over the query tiles; one
  // head of the group when heads are work items of their own)
  int f0 = 0, f1 = 0;
  const short *fkp = nullptr, *fvp = nullptr;
  if (FWD) {
    const int dz = w.z + 1 < p.nz ? w.z + 1 : (p.fwd_wrap ? 0 : -1);
    if (dz >= 0 && (hshift || w.h == w.kvh * (p.Hq / p.Hkv))) {
      const int64_t ntk = (p.nk + kPBN - 1) / kPBN;
      f0 = (int)(w.qtile * ntk / ntq);
      f1 = (int)((w.qtile + 1) * ntk / ntq);
      fkp = (const short *)p.fk + dz * p.kv_zstride + w.b * p.ks_b + w.kvh * p.ks_h;
      fvp = (const short *)p.fv + dz * p.kv_vzstride + w.b * p.vs_b + w.kvh * p.vs_h;
    }
  }
  if (!FWD && ntiles == 0 && p.accumulate) return;  // nothing to add to the running state

  f32x16 O[DT];
  float m_run, m_top, lsum;
  auto init_state = [&]() {  // the running state, or an empty one
    if (p.accumulate) {
      load_state<D>(p, w, i, valid, c, O, m_run, m_top, lsum);
    } else {
      m_run = -FLT_MAX;
      m_top = -FLT_MAX;
      lsum = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
    }
  };

  // Tile loads go through buffer descriptors: the per-lane byte offsets are
  // fixed, the tile moves the (scalar) base, and K rows past the end of the
  // block read as zero (they are masked).  Offsets fit in 32 bits: the host
  // bounds the K row stride and the packed V row length.
  // Only waves 0 .. kLW-1 (one per SIMD; in the fused ring the ones that
  // start a tile with QK and exponentials) issue the loads: a direct-to-LDS
  // load holds its wave at issue for a long time, and these waves absorb
  // that best (2 % faster than all eight loading, 1 % faster than the other
  // four, in same-run comparisons).
  const bool loader = wave < kLW;
  const uint32_t krow_b = (uint32_t)p.ks_t * 2;
  uint32_t kvo[KPW];
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int idx = (loader ? wave : 0) + kLW * u;
    const int row = idx * KRPI + lane / CPR;
    const int ch = (lane % CPR) ^ chunk_swz<KROW>(row);
    kvo[u] = row * krow_b + ch * 16;
  }
  uint32_t vvo[VPW];
#pragma unroll
  for (int u = 0; u < VPW; ++u) {
    const int idx = (loader ? wave : 0) + kLW * u;
    const int dr = idx * 8 + (lane >> 3);
    vvo[u] = dr * VROW + (((lane & 7) ^ chunk_swz<VROW>(dr)) * 16);  // within a V^T tile
  }
  // the (b, h) slice of packed V: vs_t = n_pad, tiles of VTILE bytes
  const uint32_t vslice_b = (uint32_t)D * (uint32_t)p.vs_t * 2u;
  const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc((void *)vp, 0, (int)vslice_b, kBufWord3);
  auto k_rsrc = [&](const short *base, int tk) {  // K tile tk: its rows only
    const int rows = min(p.nk - tk * kPBN, kPBN);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(base + (int64_t)tk * kPBN * p.ks_t), 0,
                                             (int)(rows * krow_b), kBufWord3);
  };
  // FWD: a loading wave writes out what it loaded, from the LDS it landed in,
  // at the same per-lane offsets (rows past the block end are dropped by the
  // descriptor's range check).  The stores go out after the wave's tile loads
  // of the same iteration; memory operations count down in issue order, so
  // the end-of-tile wait for the loads leaves the stores in flight.  Returns
  // the number of stores issued.
  auto fwd_k = [&](int tk, int kstage) {
    if (!FWD || !loader || tk < f0 || tk >= f1) return 0;
    const auto dst = k_rsrc(fkp, tk);
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const u32x4 x =
          *(const u32x4 *)(lds + kstage * KTILE + kLW * 1024 * u + wave * 1024 + 16 * lane);
      __builtin_amdgcn_raw_buffer_store_b128(x, dst, kvo[u], 0, kNT);
    }
    return KPW;
  };
  auto fwd_v = [&](int tv, int vso) {  // vso: byte offset of the V^T stage
    if (!FWD || !loader || tv < f0 || tv >= f1) return 0;
    const auto dst = __builtin_amdgcn_make_buffer_rsrc((void *)fvp, 0, (int)vslice_b, kBufWord3);
#pragma unroll
    for (int u = 0; u < VPW; ++u) {
      const u32x4 x =
          *(const u32x4 *)(lds + VBASE + vso + kLW * 1024 * u + wave * 1024 + 16 * lane);
      __builtin_amdgcn_raw_buffer_store_b128(x, dst, vvo[u], tv * VTILE, kNT);
    }
    return VPW;
  };
  static_assert(KPW == VPW, "the waits below take 0, KPW or 2 KPW stores");
  auto wait_loads = [&](int stores) {  // this wave's loads have landed
    if (stores == 0)
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    else if (stores == KPW)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | KPW);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | (2 * KPW));
  };
  // tiles [max(f0, t0), f1), which this workgroup does not stream: global to
  // global through registers, each tile's 1 KB pieces spread over the eight
  // waves with all of a wave's loads in flight together
  auto fwd_direct = [&](int t0) {
    if (!FWD) return;
    constexpr int KC = KTILE / 1024 / kPW, VC = VTILE / 1024 / kPW;
    const auto vdst = __builtin_amdgcn_make_buffer_rsrc((void *)fvp, 0, (int)vslice_b, kBufWord3);
    for (int t = max(f0, t0); t < f1; ++t) {
      const auto ksrc = k_rsrc(kp, t), kdst = k_rsrc(fkp, t);
      u32x4 xk[KC], xv[VC];
      uint32_t ko[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        ko[j] = ((wave + kPW * j) * KRPI + lane / CPR) * krow_b + (lane % CPR) * 16;
        xk[j] = __builtin_amdgcn_raw_buffer_load_b128(ksrc, ko[j], 0, kNT);
      }
#pragma unroll
      for (int j = 0; j < VC; ++j)
        xv[j] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, (wave + kPW * j) * 1024 + 16 * lane,
                                                      t * VTILE, kNT);
#pragma unroll
      for (int j = 0; j < KC; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(xk[j], kdst, ko[j], 0, kNT);
#pragma unroll
      for (int j = 0; j < VC; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(xv[j], vdst, (wave + kPW * j) * 1024 + 16 * lane,
                                               t * VTILE, kNT);
    }
  };
  if (FWD && ntiles == 0 && p.accumulate) {
    fwd_direct(0);
    return;
  }
  if (ntiles > 0) {
    // A loading wave's share of K tile tk / V^T tile tv goes straight into an LDS
    // stage (buffer loads with the LDS destination in M0: lane l's 16 bytes
    // land at base + 16 l, so the swizzle is applied on the source side).
    // Completion is awaited (vmcnt) before the barrier that publishes the stage.
    // (loading waves only: the callers test it)
    auto load_k = [&](int tk, int kstage) {
      const auto krsrc = k_rsrc(kp, tk);
#pragma unroll
      for (int u = 0; u < KPW; ++u)
        dma16(krsrc, (lds_void *)(lds + kstage * KTILE + kLW * 1024 * u + wave * 1024), kvo[u], 0);
    };
    auto load_v = [&](int tv, int vso) {  // vso: byte offset of the V^T stage
#pragma unroll
      for (int u = 0; u < VPW; ++u)
        dma16(vrsrc, (lds_void *)(lds + VBASE + vso + kLW * 1024 * u + wave * 1024), vvo[u],
              tv * VTILE);
    };

    // The first tiles, the Q fragments and the running state are requested
    // together, so their latencies overlap: K tiles 0 and 1 and V^T tile 0
    // (awaited before the prologue's barrier) ...
    if (loader) {
      load_k(0, 0);
      if (ntiles > 1) load_k(1, 1);
      load_v(0, 0);
    }
    // ... Q fragments (B operand of S^T = K Q^T): d = 16ks + 8hl .. +7 of
    // this lane's row ...
    s16x8 qf[KS];
    {
      const short *qrow = qp + (int64_t)(valid ? i : 0) * p.qs_t;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s16x8 v = *(const s16x8 *)(qrow + 16 * ks + 8 * hl);
        if (!valid) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
        qf[ks] = v;
      }
    }
    // ... and the running state.
    init_state();

    // Per-lane LDS read offsets.  Row kh*32 + c32 (K) and 32dt + c32 (V^T)
    // share the swizzle of row c32, so kh, dt and the stage are immediates.
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      koff[ks] = c32 * KROW + (((2 * ks + hl) ^ chunk_swz<KROW>(c32)) << 4);
    int voff[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)  // q4 = 2*kh + cc -> logical chunk 2*q4 + hl
      voff[q4] = VBASE + c32 * VROW + (((2 * q4 + hl) ^ chunk_swz<VROW>(c32)) << 4);

    auto rowmax = [&](const f32x16 (&x)[2]) {
      float m = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, x[kh][r]);
      return m;
    };
    // probabilities of tile S against the running maximum, packed for the PV
    // product; returns this lane's sum of them
    auto probs = [&](const f32x16 (&S)[2], s16x8 (&P)[4]) {
      const float nm = -m_run;
      float ls = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x16 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = __builtin_amdgcn_exp2f(fmaf(S[q4 >> 1][8 * (q4 & 1) + e], c, nm));
          ls += pb[e];
        }
        P[q4] = M::pack(pb, 0);
      }
      return ls;
    };
    auto rescale = [&](float mt) {  // running maximum -> max(m_run, mt)
      const float mn = fmaxf(m_run, mt);
      const float al = __builtin_amdgcn_exp2f(m_run - mn);
      lsum *= al;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= al;
      m_run = mn;
    };

    // Prologue: K tiles 0 and 1, V^T tile 0 resident; S^T of tile 0.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    fwd_k(0, 0);
    f32x16 S[2], S1[2];
    float mx = -INFINITY;  // EXACT: row max of the next tile's S (before masking)
    if (0 < ntiles_w) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[kh][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          S[kh] = M::mma(*(const s16x8 *)(lds + koff[ks] + kh * 32 * KROW), qf[ks], S[kh]);
      if (EXACT) mx = rowmax(S);
    }

    constexpr int NSTEP = 2 * KS;      // QK MFMAs per tile (two 32-key halves)
    constexpr int EPS = 32 / NSTEP;    // exponentials per QK MFMA
    // The two waves sharing a SIMD run the same work half a tile apart: a
    // leading wave does [QK(t+1) with the exponentials of t, then PV(t)], a
    // lagging wave [PV(t-1), then QK(t+1) with the exponentials of t], so
    // while one issues MFMAs only, the other has VALU work to overlap.
    // (the exact-max variant keeps all waves leading: its extra row-max state
    // does not fit the registers of both orders)
    const bool lag = !EXACT && wave >= kPW / 2;
    s16x8 P[4];        // probabilities of the tile whose PV is pending
    s16x8 va0[DT];     // its first group of V^T fragments, read ahead
    // byte offsets of the V^T stages of tiles t, t+1 and t-1 (stage t % 3)
    int vcur = 0, vnext = VTILE, vprev = 2 * VTILE;
    // The per-tile tests as one scalar compare each: a loading wave loads K
    // tile t+2 while t < kload_end and V^T tile t+1 while t < vload_end; a
    // lagging wave runs the PV of tile t-1 while t-1 < pv_lag_n (unsigned, so
    // not at t = 0).
    const int kload_end = loader ? ntiles - 2 : 0;
    const int vload_end = loader ? ntiles - 1 : 0;
    const unsigned pv_lag_n = lag ? (unsigned)ntiles_w : 0u;
    // O^T += V^T P^T for the V^T tile in stage offset vso (va0 read already);
    // EXACT: returns the row max of Sm, computed in the MFMA shadow
    auto pv = [&](int vso, const f32x16 (&Sm)[2]) {
      s16x8 va[4][DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) va[0][dt] = va0[dt];
      float mxn = -INFINITY;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (q4 + 1 < 4) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            va[q4 + 1][dt] = *(const s16x8 *)(lds + voff[q4 + 1] + vso + dt * 32 * VROW);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] = M::mma(va[q4][dt], P[q4], O[dt]);
        if (EXACT) {
#pragma unroll
          for (int r = 0; r < 8; ++r) mxn = fmaxf(mxn, Sm[q4 >> 1][8 * (q4 & 1) + r]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return mxn;
    };
    // Tile t (PAR = t & 1).  After the barrier at its start, K tile t+1 (K
    // stage PAR ^ 1) and V^T tile t (stage t % 3), loaded during tile t-1, are
    // visible; K stage PAR (tile t, read in tile t-1) and V^T stage (t+1) % 3
    // (tile t-2, whose PV the lagging waves finished in tile t-1) are free for
    // K tile t+2 and V^T tile t+1, loaded now and awaited at the end.
    auto tile = [&](auto par_c, const int t, f32x16 (&Sc)[2], f32x16 (&Sn)[2]) {
      constexpr int PAR = decltype(par_c)::value;
      // also at t = 0: K stage 0 is read by the prologue's QK of tile 0
      if constexpr (FWD)
        lds_barrier();
      else
        __syncthreads();
      if (t < kload_end) load_k(t + 2, PAR);
      if (t < vload_end) load_v(t + 1, vnext);
      int stores = t + 1 < ntiles ? fwd_k(t + 1, PAR ^ 1) : 0;
      stores += fwd_v(t, vcur);
      if ((unsigned)(t - 1) < pv_lag_n) {
        const float m2 = pv(vprev, Sc);
        if (EXACT) mx = m2;
      }
      if (t < ntiles_w) {
        const bool diag = t >= nfull_w;  // causal diagonal or ragged end of the block
        if (diag) {
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = t * kPBN + kh * 32 + (r >> 2) * 8 + 4 * hl + (r & 3);
              if (j >= jlim) Sc[kh][r] = -INFINITY;
            }
        }
        if (EXACT) {
          if (diag) mx = rowmax(Sc);
          mx = half_max(mx);
          const float mt = mx * c;
          m_top = fmaxf(m_top, mt);
          if (wave_any(mt > m_run + kTau)) rescale(mt);
        }
        const float nm = -m_run;

        // QK of the next tile (discarded when the wave has none), one MFMA at
        // a time, each followed by a share of this tile's exponentials.
        const char *stn = lds + (PAR ^ 1) * KTILE;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) Sn[kh][r] = 0.f;
        // K fragments in a rolling window: those of k-step ks + KA are read
        // while k-step ks is multiplied
        s16x8 ka[KS][2];
#pragma unroll
        for (int d = 0; d < KA; ++d)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
            ka[d][kh] = *(const s16x8 *)(stn + koff[d] + kh * 32 * KROW);
        float ls = 0.f;
        f32x16 pbuf;
        // While a wave interleaves QK with the exponentials it takes issue
        // priority over the other wave of its SIMD, whose PV phase is MFMAs
        // only and fills the MFMA pipe around it (3 % faster than equal
        // priorities; priority during PV instead is slower).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int step = 0; step < NSTEP; ++step) {
          const int ks = step >> 1, kh = step & 1;
          if (kh == 0 && ks + KA < KS) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              ka[ks + KA][h2] = *(const s16x8 *)(stn + koff[ks + KA] + h2 * 32 * KROW);
          }
          if (step == NSTEP - 2) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
              va0[dt] = *(const s16x8 *)(lds + voff[0] + vcur + dt * 32 * VROW);
          }
          Sn[kh] = M::mma(ka[ks][kh], qf[ks], Sn[kh]);
#pragma unroll
          for (int v = 0; v < EPS; ++v) {
            const int e = EPS * step + v;  // element of S: half e/16, register e%16
            const float pv = __builtin_amdgcn_exp2f(fmaf(Sc[e >> 4][e & 15], c, nm));
            ls += pv;  // l sums the unrounded probabilities
            pbuf[e & 7] = pv;
            if ((e & 7) == 7) P[e >> 3] = M::pack(pbuf, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (!EXACT) {
          // a probability above 2^kTau means a new maximum: rescale and redo
          if (wave_any(ls > kSumLimit)) {
            rescale(half_max(rowmax(Sc)) * c);
            ls = probs(Sc, P);
          }
        }
        lsum += ls;
        if (!lag) {
          const float m2 = pv(vcur, Sn);
          if (EXACT) mx = m2;
        }
      }
      wait_loads(stores);  // this wave's tile loads have landed
      const int vfree = vprev;
      vprev = vcur;
      vcur = vnext;
      vnext = vfree;
    };
    // two tiles per iteration so the K stages are immediates and the S
    // register sets swap roles instead of being copied
    for (int t = 0; t < ntiles; t += 2) {
      tile(std::integral_constant<int, 0>(), t, S, S1);
      if (t + 1 >= ntiles) break;
      tile(std::integral_constant<int, 1>(), t + 1, S1, S);
    }
    // the lagging waves' PV of the last tile (no stage is reloaded any more)
    if (lag && ntiles_w == ntiles) pv(vprev, S);
    fwd_direct(ntiles);
  } else {
    fwd_direct(0);
    init_state();
  }
  store_state<D>(p, w, i, valid, O, m_run, EXACT ? m_top : m_run, lsum);
}


// Lean variant for d = 64 (both folds, and the public block partial).  At
// d = 64 a 64-key tile is 16 MFMAs against 32 exponentials per wave, and a
// workgroup's key blocks are short (the 512-token shards: 8 tiles), so
// per-workgroup costs -- the running state in and out, the first
// loads, the tile barrier -- weigh as much as the products.  This variant
// gives up the in-wave pipelining (QK of the next tile under the exponentials
// of this one, lagging waves) for registers: at <= 128 VGPRs two workgroups
// share a CU, four waves per SIMD, and one workgroup's state traffic and
// barrier waits run beside the other's products.  Same arithmetic in the same
// order as attn_packed_kernel<64, *, EXACT>; K and V^T tiles one tile ahead,
// two stages each (32 KB of LDS).
template <bool BF16, bool EXACT, bool FWD>
__global__ void __launch_bounds__(512, 4) attn_lean64_kernel(BatchParams p, int ntq, int hshift) {
  using M = Mfma16<BF16>;
  constexpr int D = 64;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int KROW = D * 2;
  constexpr int KTILE = kPBN * KROW;
  constexpr int VROW = kPBN * 2;
  constexpr int VTILE = D * VROW;
  constexpr int VBASE = 2 * KTILE;  // LDS: K stages 0, 1, then V^T stages 0, 1
  constexpr int KPW = KTILE / 1024 / kLW;
  constexpr int VPW = VTILE / 1024 / kLW;
  constexpr int KRPI = 1024 / KROW;
  constexpr int CPR = D / 8;
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Work w = hshift ? decode_items(p, ntq, 1) : decode(p, ntq);
  w.h += wave >> (3 - hshift);
  const int wave_r = wave & ((kPW >> hshift) - 1);
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;

  const short *qp = (const short *)p.q + w.z * p.q_zstride + w.b * p.qs_b + w.h * p.qs_h;
  const int kvi = (p.kv_idx0 + w.z) % p.kv_idx_mod;
  const short *kp = (const short *)p.k + kvi * p.kv_zstride + w.b * p.ks_b + w.kvh * p.ks_h;
  const short *vp = (const short *)p.v + kvi * p.kv_vzstride + w.b * p.vs_b + w.kvh * p.vs_h;
  const IdMap qid = query_ids(p, w.z), kid = key_ids(p, w.z);
  const float c = p.scale * kLog2e;

  const int i_wg0 = w.qtile * (kPBM >> hshift);
  const int i_wg1 = min(p.nq, i_wg0 + (kPBM >> hshift)) - 1;
  const int iw0 = i_wg0 + wave_r * 32;
  const int iw1 = min(p.nq - 1, iw0 + 31);
  const bool wave_rows = iw0 < p.nq;
  const int i = iw0 + c32;
  const bool valid = i < p.nq;

  const int kv_wg = key_prefix(p, kid, qid(i_wg1));
  const int ntiles = (kv_wg + kPBN - 1) / kPBN;
  const int kv_wl = wave_rows ? key_prefix(p, kid, qid(iw1)) : 0;
  const int kv_wf = wave_rows ? key_prefix(p, kid, qid(iw0)) : 0;
  const int ntiles_w = (kv_wl + kPBN - 1) / kPBN;
  const int nfull_w = kv_wf / kPBN;
  const int jlim = key_prefix(p, kid, qid(i));
  // FWD: as in attn_packed_kernel
  int f0 = 0, f1 = 0;
  const short *fkp = nullptr, *fvp = nullptr;
  if (FWD) {
    const int dz = w.z + 1 < p.nz ? w.z + 1 : (p.fwd_wrap ? 0 : -1);
    if (dz >= 0 && (hshift || w.h == w.kvh * (p.Hq / p.Hkv))) {
      const int64_t ntk = (p.nk + kPBN - 1) / kPBN;
      f0 = (int)(w.qtile * ntk / ntq);
      f1 = (int)((w.qtile + 1) * ntk / ntq);
      fkp = (const short *)p.fk + dz * p.kv_zstride + w.b * p.ks_b + w.kvh * p.ks_h;
      fvp = (const short *)p.fv + dz * p.kv_vzstride + w.b * p.vs_b + w.kvh * p.vs_h;
    }
  }
  if (!FWD && ntiles == 0 && p.accumulate) return;

  f32x16 O[DT];
  float m_run, m_top, lsum;
  auto init_state = [&]() {
    if (p.accumulate) {
      load_state<D>(p, w, i, valid, c, O, m_run, m_top, lsum);
    } else {
      m_run = -FLT_MAX;
      m_top = -FLT_MAX;
      lsum = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
    }
  };

  static_assert(KROW == 128 && VROW == 128 && KPW == 2 && VPW == 2, "d = 64 layout");
  // A loading wave's two 1 KB pieces of a tile are 32 rows apart, which
  // keeps the row swizzle: the second offset is the first plus 32 rows.
  const bool loader = wave < kLW;
  const uint32_t krow_b = (uint32_t)p.ks_t * 2;
  uint32_t kvo0, vvo0;
  {
    const int row = (loader ? wave : 0) * KRPI + lane / CPR;
    kvo0 = row * krow_b + (((lane % CPR) ^ chunk_swz<KROW>(row)) * 16);
    const int dr = (loader ? wave : 0) * 8 + (lane >> 3);
    vvo0 = dr * VROW + (((lane & 7) ^ chunk_swz<VROW>(dr)) * 16);
  }
  const uint32_t vslice_b = (uint32_t)D * (uint32_t)p.vs_t * 2u;
  const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc((void *)vp, 0, (int)vslice_b, kBufWord3);
  auto k_rsrc = [&](const short *base, int tk) {  // K tile tk: its rows only
    const int rows = min(p.nk - tk * kPBN, kPBN);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(base + (int64_t)tk * kPBN * p.ks_t), 0,
                                             (int)(rows * krow_b), kBufWord3);
  };
  // FWD: tile t, resident in LDS stage st, written out by the waves that
  // loaded it, at the offsets they loaded it from: read before, and stored
  // after, the same waves' loads of the next tile (as in attn_packed_kernel)
  struct Fwd {
    u32x4 x[4];
    bool on;
  };
  auto fwd_read = [&](int t, int st) {
    Fwd f;
    f.on = FWD && loader && t >= f0 && t < f1;
    if (f.on) {
      // the lane's 16-byte slot, rebuilt from the lane id here (kept live
      // across the tile it is spilled, and its reload waits for the stores)
      int slot;
      asm volatile(
          "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
          "v_mbcnt_hi_u32_b32 %0, -1, %0\n\t"
          "v_lshlrev_b32 %0, 4, %0"
          : "=v"(slot));
      const char *ks = lds + st * KTILE + wave * 1024 + slot;
      const char *vs = lds + VBASE + st * VTILE + wave * 1024 + slot;
      f.x[0] = *(const u32x4 *)ks;
      f.x[1] = *(const u32x4 *)(ks + kLW * 1024);
      f.x[2] = *(const u32x4 *)vs;
      f.x[3] = *(const u32x4 *)(vs + kLW * 1024);
    }
    return f;
  };
  auto fwd_store = [&](const Fwd &f, int t) {
    if (!f.on) return 0;
    const auto kdst = k_rsrc(fkp, t);
    const auto vdst = __builtin_amdgcn_make_buffer_rsrc((void *)fvp, 0, (int)vslice_b, kBufWord3);
    __builtin_amdgcn_raw_buffer_store_b128(f.x[0], kdst, kvo0, 0, kNT);
    __builtin_amdgcn_raw_buffer_store_b128(f.x[1], kdst, kvo0 + 32 * krow_b, 0, kNT);
    __builtin_amdgcn_raw_buffer_store_b128(f.x[2], vdst, vvo0, t * VTILE, kNT);
    __builtin_amdgcn_raw_buffer_store_b128(f.x[3], vdst, vvo0, t * VTILE + 32 * VROW, kNT);
    return 4;
  };
  // tiles [max(f0, t0), f1) this workgroup does not stream: global to global,
  // one 1 KB piece of K and one of V^T per wave and tile
  auto fwd_direct = [&](int t0) {
    if (!FWD) return;
    static_assert(KTILE == kPW * 1024 && VTILE == kPW * 1024, "one piece per wave");
    const auto vdst = __builtin_amdgcn_make_buffer_rsrc((void *)fvp, 0, (int)vslice_b, kBufWord3);
    for (int t = max(f0, t0); t < f1; ++t) {
      const auto ksrc = k_rsrc(kp, t), kdst = k_rsrc(fkp, t);
      const uint32_t ko = (wave * KRPI + lane / CPR) * krow_b + (lane % CPR) * 16;
      const uint32_t vo = wave * 1024 + 16 * lane;
      const u32x4 xk = __builtin_amdgcn_raw_buffer_load_b128(ksrc, ko, 0, kNT);
      const u32x4 xv = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, vo, t * VTILE, kNT);
      __builtin_amdgcn_raw_buffer_store_b128(xk, kdst, ko, 0, kNT);
      __builtin_amdgcn_raw_buffer_store_b128(xv, vdst, vo, t * VTILE, kNT);
    }
  };
  if (FWD && ntiles == 0 && p.accumulate) {
    fwd_direct(0);
    return;
  }
  if (ntiles > 0) {
    // (loading waves only: the callers test it)
    auto load_k = [&](int tk, int kstage) {
      const auto krsrc = k_rsrc(kp, tk);
      char *dst = lds + kstage * KTILE + wave * 1024;
      dma16(krsrc, (lds_void *)dst, kvo0, 0);
      dma16(krsrc, (lds_void *)(dst + kLW * 1024), kvo0 + 32 * krow_b, 0);
    };
    auto load_v = [&](int tv, int vstage) {
      char *dst = lds + VBASE + vstage * VTILE + wave * 1024;
      dma16(vrsrc, (lds_void *)dst, vvo0, tv * VTILE);
      dma16(vrsrc, (lds_void *)(dst + kLW * 1024), vvo0, tv * VTILE + 32 * VROW);
    };
    if (loader) {
      load_k(0, 0);
      load_v(0, 0);
    }
    s16x8 qf[KS];
    {
      const short *qrow = qp + (int64_t)(valid ? i : 0) * p.qs_t;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s16x8 v = *(const s16x8 *)(qrow + 16 * ks + 8 * hl);
        if (!valid) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
        qf[ks] = v;
      }
    }
    init_state();
    // LDS read offsets: K row c32 (+32 kh) chunk 2 ks + hl and V^T row c32
    // (+32 dt) chunk 2 q4 + hl, both swizzled by row c32: base ^ (j << 5)
    // for j = ks or q4 (the chunk index sits in bits 4-6)
    const int rbase = c32 * KROW + ((hl ^ chunk_swz<KROW>(c32)) << 4);

    auto rowmax = [&](const f32x16 (&x)[2]) {
      float m = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, x[kh][r]);
      return m;
    };
    auto probs = [&](const f32x16 (&S)[2], s16x8 (&P)[4]) {
      const float nm = -m_run;
      float ls = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x16 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = __builtin_amdgcn_exp2f(fmaf(S[q4 >> 1][8 * (q4 & 1) + e], c, nm));
          ls += pb[e];
        }
        P[q4] = M::pack(pb, 0);
      }
      return ls;
    };
    auto rescale = [&](float mt) {
      const float mn = fmaxf(m_run, mt);
      const float al = __builtin_amdgcn_exp2f(m_run - mn);
      lsum *= al;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= al;
      m_run = mn;
    };

    // Tile t sits in stage t & 1; the other stage, last read in tile t-1,
    // takes tile t+1, published by the barrier at the end of tile t.  A
    // loading wave loads while t < load_end (one scalar compare per tile).
    const int load_end = loader ? ntiles - 1 : 0;
    auto tile = [&](auto st_c, const int t) {
      constexpr int ST = decltype(st_c)::value;
      const Fwd fw = fwd_read(t, ST);
      if (t < load_end) {
        load_k(t + 1, ST ^ 1);
        load_v(t + 1, ST ^ 1);
      }
      const int stores = fwd_store(fw, t);
      if (t < ntiles_w) {
        // the offsets are rebuilt per tile from one register (kept out of
        // the loop's live set)
        int rb = rbase;
        asm volatile("" : "+v"(rb));
        const int ro[4] = {rb, rb ^ 32, rb ^ 64, rb ^ 96};
        f32x16 S[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) S[kh][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
            S[kh] = M::mma(*(const s16x8 *)(lds + ro[ks] + ST * KTILE + kh * 32 * KROW), qf[ks],
                           S[kh]);
        if (t >= nfull_w) {
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = t * kPBN + kh * 32 + (r >> 2) * 8 + 4 * hl + (r & 3);
              if (j >= jlim) S[kh][r] = -INFINITY;
            }
        }
        s16x8 P[4];
        float ls;
        if (EXACT) {  // the tile's row maximum first, as in attn_packed_kernel
          const float mt = half_max(rowmax(S)) * c;
          m_top = fmaxf(m_top, mt);
          if (wave_any(mt > m_run + kTau)) rescale(mt);
          ls = probs(S, P);
        } else {
          ls = probs(S, P);
          if (wave_any(ls > kSumLimit)) {
            rescale(half_max(rowmax(S)) * c);
            ls = probs(S, P);
          }
        }
        lsum += ls;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            O[dt] = M::mma(
                *(const s16x8 *)(lds + ro[q4] + VBASE + ST * VTILE + dt * 32 * VROW), P[q4], O[dt]);
      }
      // this wave's loads of tile t+1 have landed (its stores may still run)
      if (stores)
        __builtin_amdgcn_s_waitcnt(kWaitVm0 | 4);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if constexpr (FWD)
        lds_barrier();
      else
        __syncthreads();
    };
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
      tile(std::integral_constant<int, 0>(), t);
      if (t + 1 >= ntiles) break;
      tile(std::integral_constant<int, 1>(), t + 1);
    }
    fwd_direct(ntiles);
  } else {
    fwd_direct(0);
    init_state();
  }
  store_state<D>(p, w, i, valid, O, m_run, EXACT ? m_top : m_run, lsum);
}

// V rows [b][h][j][c] (strides) -> packed [bh][tile][c][64]; one workgroup
// per (bh, 64-key tile): coalesced 16-byte loads of key rows, LDS transpose,
// coalesced 16-byte stores of 8 packed positions (the tile is one block).
__global__ void __launch_bounds__(256) pack_v_kernel(const short *__restrict__ v,
                                                     short *__restrict__ vp, int64_t H, int64_t n,
                                                     int64_t n_pad, int d, int64_t vs_b,
                                                     int64_t vs_h, int64_t vs_t) {
  __shared__ short tile[kPBN][128 + 8];
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / H, h = bh % H;
  const int64_t j0 = (int64_t)blockIdx.x * kPBN;
  const short *src = v + b * vs_b + h * vs_h;
  const int c8n = d / 8;
  for (int e = threadIdx.x; e < kPBN * c8n; e += blockDim.x) {
    const int key = e / c8n, c8 = e % c8n;
    const int64_t j = j0 + key;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (j < n) val = *(const uint4 *)(src + j * vs_t + c8 * 8);
    *(uint4 *)&tile[key][c8 * 8] = val;
  }
  __syncthreads();
  short *dst = vp + bh * (int64_t)d * n_pad + j0 * d;  // tile j0/64 of d x 64
  for (int e = threadIdx.x; e < d * (kPBN / 8); e += blockDim.x) {
    const int cidx = e / (kPBN / 8), g = e % (kPBN / 8);
    short out[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) out[u] = tile[perm16(g * 8 + u)][cidx];
    uint4 val;
    val.x = (unsigned short)out[0] | ((unsigned)(unsigned short)out[1] << 16);
    val.y = (unsigned short)out[2] | ((unsigned)(unsigned short)out[3] << 16);
    val.z = (unsigned short)out[4] | ((unsigned)(unsigned short)out[5] << 16);
    val.w = (unsigned short)out[6] | ((unsigned)(unsigned short)out[7] << 16);
    *(uint4 *)(dst + cidx * kPBN + g * 8) = val;
  }
}

template <int D, bool BF16, bool EXACT, bool FWD>
hipError_t launch_packed(const BatchParams &p, hipStream_t s) {
  const int hpg = p.Hq / p.Hkv;
  const int hshift = (hpg == 2 || hpg == 4 || hpg == 8) ? (hpg == 2 ? 1 : hpg == 4 ? 2 : 3) : 0;
  const int rows = kPBM >> hshift;
  const int ntq = (p.nq + rows - 1) / rows;
  const int64_t nwg = (int64_t)ntq * p.nz * p.B * p.Hkv * (hshift ? 1 : hpg);
  const size_t lds = (size_t)2 * kPBN * D * 2 + (size_t)3 * D * kPBN * 2;
  // more than 64 KB of LDS per workgroup must be opted into, once per process
  // (a function-local static: initialised once even with several host threads)
  static const hipError_t attr =
      lds > 65536 ? hipFuncSetAttribute((const void *)attn_packed_kernel<D, BF16, EXACT, FWD>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
                  : hipSuccess;
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((attn_packed_kernel<D, BF16, EXACT, FWD>), dim3((unsigned)nwg), dim3(512),
                     lds, s, p, ntq, hshift);
  return hipGetLastError();
}

template <bool BF16, bool EXACT, bool FWD>
hipError_t launch_lean64(const BatchParams &p, hipStream_t s) {
  const int hpg = p.Hq / p.Hkv;
  const int hshift = (hpg == 2 || hpg == 4 || hpg == 8) ? (hpg == 2 ? 1 : hpg == 4 ? 2 : 3) : 0;
  const int rows = kPBM >> hshift;
  const int ntq = (p.nq + rows - 1) / rows;
  const int64_t nwg = (int64_t)ntq * p.nz * p.B * p.Hkv * (hshift ? 1 : hpg);
  const size_t lds = (size_t)2 * kPBN * 64 * 2 + (size_t)2 * 64 * kPBN * 2;
  hipLaunchKernelGGL((attn_lean64_kernel<BF16, EXACT, FWD>), dim3((unsigned)nwg), dim3(512), lds,
                     s, p, ntq, hshift);
  return hipGetLastError();
}

template <int D, bool BF16, bool FWD>
hipError_t launch_packed_f(const BatchParams &p, hipStream_t s) {
  if constexpr (D == 64)  // every packed-V call at d = 64 runs the lean kernel
    return p.exact_m ? launch_lean64<BF16, true, FWD>(p, s) : launch_lean64<BF16, false, FWD>(p, s);
  else
    return p.exact_m ? launch_packed<D, BF16, true, FWD>(p, s)
                     : launch_packed<D, BF16, false, FWD>(p, s);
}

template <int D, bool BF16>
hipError_t launch_packed_m(const BatchParams &p, hipStream_t s) {
  // the forwarding instantiation only where some problem forwards its block
  const bool fwd = p.fwd && (p.nz > 1 || p.fwd_wrap);
  return fwd ? launch_packed_f<D, BF16, true>(p, s) : launch_packed_f<D, BF16, false>(p, s);
}

}  // namespace

hipError_t launch_block_fwd_packed(const BatchParams &p, int dtype, hipStream_t s) {
  if (dtype == RA_DT_BF16)
    return p.d == 64 ? launch_packed_m<64, true>(p, s) : launch_packed_m<128, true>(p, s);
  return p.d == 64 ? launch_packed_m<64, false>(p, s) : launch_packed_m<128, false>(p, s);
}

hipError_t launch_pack_v(const void *v, void *vp, int elt, int64_t BH, int64_t H, int64_t n,
                         int64_t d, int64_t vs_b, int64_t vs_h, int64_t vs_t, hipStream_t s) {
  if (BH == 0 || n == 0) return hipSuccess;
  (void)elt;
  const int64_t n_pad = packed_n(n);
  dim3 grid((unsigned)(n_pad / kPBN), (unsigned)BH);
  hipLaunchKernelGGL(pack_v_kernel, grid, dim3(256), 0, s, (const short *)v, (short *)vp, H, n,
                     n_pad, (int)d, vs_b, vs_h, vs_t);
  return hipGetLastError();
}

}  // namespace ra
