// bwd.hip -- gradients of exact attention for one batch of (query shard,
// K/V block) problems: the unit of work of one hop of the backward ring.
//
// Training on long contexts is the headline use of ring attention
// (highthink.cn article, introduction; aiunderstanding.org guide, "Reale
// Umsetzung"); the pages give no backward algorithm, so the kernels compute
// the derivative of the forward definition, with the forward's softmax
// statistics (LSE per query row) and D = <dO, O>:
//   p = exp(s - lse), dP = dO v^T, dS = p (dP - D),
//   dV += p^T dO, dK += scale dS^T q, dQ += scale dS k.
// Blocks contribute additively, so every hop adds its block's share.
//
// gfx950 design.  The two MFMA operands of a 32x32x16 product both want
// their reduction dimension contiguous per lane, so each product picks the
// orientation whose operands are plain 16-byte reads.  Three kernels per hop:
//  * bwd_kv_kernel<dV> and bwd_kv_kernel<dK> (a workgroup owns 256 keys, a
//    wave 32; loop over the query heads of the K/V head and 64-query tiles):
//    S = Q K^T (and dP = dO V^T) with Q, dO rows from LDS and this lane's K,
//    V rows in registers, so a lane owns a key column; dV^T += dO^T P or
//    dK^T += Q^T dS then read dO^T / Q^T from the packed transposed layout
//    (the one V uses in the forward), whose query order matches how P and dS
//    sit in the registers.  dV and dK are separate kernels so that a wave's
//    state fits 256 registers; S is computed by both.
//  * bwd_dq_kernel (a workgroup owns 256 queries, a wave 32; loops over
//    64-key tiles): S^T = K Q^T and dP^T = V dO^T as in the forward (a lane
//    owns a query), dQ^T += K^T dS^T with K^T packed.
// Loaded bytes per MFMA are what these kernels pay for most (the loads
// stream into LDS next to the operand reads), so every kernel runs two waves
// per SIMD over 256 rows per workgroup: one loaded tile serves 256 rows.
// Only waves 0-3 (one per SIMD) issue the tile loads: a direct-to-LDS load
// holds its wave at issue for a long time, and with the other four waves
// free of them the backward pass runs 5-6 % faster than with all eight
// loading (3 % with waves 4-7 loading instead).
// Each workgroup owns its output tile, so the fp32 accumulation is plain
// read-add-write: no atomics, deterministic.
#include <cfloat>
#include <cmath>
#include <type_traits>

#include "attn_common.h"

namespace ra {
namespace {

using namespace attn;

constexpr int kKW = 8;       // dV / dK waves per workgroup (two per SIMD, 256 registers each)
constexpr int kQW = 8;       // dQ waves per workgroup (two per SIMD, 256 registers each)
constexpr int kRoleV = 0, kRoleK = 1;
constexpr int kBT = 64;      // rows of a staged tile (queries in dV / dK, keys in dQ)
constexpr int kLW = 4;       // waves that issue the tile loads (waves 0 .. kLW-1, one per SIMD)

template <int ROW_BYTES>
__device__ __forceinline__ int swz16(int row) {  // 16-byte chunk swizzle, 64 LDS banks
  return ROW_BYTES == 256 ? (row & 15) : ((row >> 1) & 7);
}

// 16-byte operand read of row `row`, logical chunk `ch`, of a swizzled LDS tile
template <int ROW_BYTES>
__device__ __forceinline__ s16x8 rd(const char *base, int row, int ch) {
  return *(const s16x8 *)(base + row * ROW_BYTES + ((ch ^ swz16<ROW_BYTES>(row)) << 4));
}

constexpr int kBufWord3B = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family)
typedef __attribute__((address_space(3))) void lds_void;

// Buffer loads that write LDS directly: lane l's bytes land at dst + size*l
// (dst is wave-uniform, it goes to M0).  Plain device functions: written in a
// kernel template, the builtin keeps the host pass from emitting the launch stub.
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, lds_void *dst, uint32_t voff,
                                       uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4b(__amdgpu_buffer_rsrc_t r, lds_void *dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, soff, 0, 0);
}
// num_records is an unsigned 32-bit byte count; the host bounds every slice to 4 GiB
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  const int64_t lim = bytes < 0xffffffffll ? bytes : 0xffffffffll;
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)(uint32_t)lim, kBufWord3B);
}

// A tile of ROWS rows x ROW_BYTES goes into a swizzled LDS tile by NW loading
// waves: wave-load u covers rows (wave + NW u) * RPI .. + RPI - 1; lane l lands
// at LDS chunk l % CPR of its row and fetches the chunk that belongs there
// (the swizzle is an involution).  The swizzle of a row depends on its
// position in a 16-row (or 32-row) period only, which wave-load u shifts by a
// multiple of it, so every wave-load uses the per-lane offset of u = 0
// (tile_voff, computed once) plus u * NW * RPI rows in the scalar offset.
// row_bytes: source row pitch (bytes); soff: offset of the tile's first row.
template <int ROW_BYTES>
__device__ __forceinline__ uint32_t tile_voff(uint32_t row_bytes, int wave, int lane) {
  constexpr int CPR = ROW_BYTES / 16, RPI = 1024 / ROW_BYTES;
  const int row = wave * RPI + lane / CPR;
  const int ch = (lane % CPR) ^ swz16<ROW_BYTES>(row);
  return (uint32_t)row * row_bytes + (uint32_t)ch * 16;
}
template <int ROW_BYTES, int ROWS, int NW>
__device__ __forceinline__ void load_tile(char *dst, __amdgpu_buffer_rsrc_t r, uint32_t row_bytes,
                                          uint32_t voff, uint32_t soff, int wave) {
  constexpr int RPI = 1024 / ROW_BYTES;
  constexpr int NU = ROWS * ROW_BYTES / 1024 / NW;
  static_assert(NU * NW * 1024 == ROWS * ROW_BYTES, "tile must split over the waves");
  static_assert(NW * RPI % 16 == 0, "wave-loads must shift rows by whole swizzle periods");
#pragma unroll
  for (int u = 0; u < NU; ++u)
    dma16b(r, (lds_void *)(dst + (wave + NW * u) * 1024), voff,
           soff + (uint32_t)(NW * RPI * u) * row_bytes);
}

// first local query index i with qid(i) >= kg (nq if none); ids increase with i
__device__ __forceinline__ int first_query(const IdMap &q, int nq, int64_t kg) {
  int lo = 0, hi = nq;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (q(mid) >= kg)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// Stage of the dV / dK kernels: Q rows | (dK: dO rows) | packed dO^T (dV) or
// Q^T (dK) | nl[64] | (dK: -D[64])
template <int D, int ROLE>
constexpr size_t kv_stage_bytes() {
  return ROLE == kRoleV ? (size_t)2 * kBT * D * 2 + kBT * 4
                        : (size_t)3 * kBT * D * 2 + 2 * kBT * 4;
}
template <int D>
constexpr size_t dq_stage_bytes() {
  return (size_t)3 * kBT * D * 2;  // K, V rows, K^T tile
}

// dV (ROLE kRoleV) or dK (kRoleK) of a batch of problems: a workgroup owns
// 256 keys (a wave 32, two waves per SIMD) and loops over the query heads of
// its K/V head and the 64-query tiles that may see its keys.  S = Q K^T with
// Q rows from LDS and this lane's K row in registers (a lane owns a key
// column), then
//   dV: P = exp2(S c + nl), dV^T += dO^T P;
//   dK: dP - D = dO V^T - D as well, dS = P (dP - D), dK^T += Q^T dS,
// with dO^T / Q^T from the packed transposed layout, whose query order inside
// each 16 matches how P and dS sit in the registers.  The two gradients run
// as two kernels so that each wave's state fits 256 registers (dV and dK
// together need more, which allowed one wave per SIMD and half the keys per
// workgroup, i.e. twice the loaded bytes per MFMA): computing S twice costs
// less than those loads.
template <int D, bool BF16, int ROLE>
__global__ void __launch_bounds__(kKW * 64) bwd_kv_kernel(BwdParams P) {
  using M = Mfma16<BF16>;
  constexpr bool DK = ROLE == kRoleK;
  const BatchParams &p = P.a;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int RB = D * 2;          // bytes of a Q / dO row
  constexpr int TB = kBT * 2;        // bytes of a packed Q^T / dO^T row (64 queries)
  constexpr int TQ = kBT * RB;       // bytes of a row tile
  constexpr int TT = D * TB;         // bytes of a packed tile
  constexpr int KWG = kKW * 32;      // keys per workgroup
  constexpr int OFF_T = DK ? 2 * TQ : TQ;     // packed tile
  constexpr int OFF_NL = OFF_T + TT;          // nl[64], then (dK) -D[64]
  constexpr size_t ST = kv_stage_bytes<D, ROLE>();
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  // workgroup -> (key tile, problem, batch, K/V head); key tile slowest so the
  // heaviest causal tiles (most queries after them) start first
  const int per_kt = p.nz * p.B * p.Hkv;
  int idx = blockIdx.x;
  const int kt = idx / per_kt;
  idx -= kt * per_kt;
  const int kvh = idx % p.Hkv;
  idx /= p.Hkv;
  const int b = idx % p.B;
  const int z = idx / p.B;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;
  const IdMap qid = query_ids(p, z), kid = key_ids(p, z);
  const int kvi = (p.kv_idx0 + z) % p.kv_idx_mod;
  const short *kp = (const short *)p.k + kvi * p.kv_zstride + b * p.ks_b + kvh * p.ks_h;
  const short *vp = (const short *)p.v + kvi * p.kv_vzstride + b * p.vs_b + kvh * p.vs_h;
  const int G = p.Hq / p.Hkv;
  const float c = p.scale * kLog2e;

  // this wave's 32 keys and this lane's key column
  const int j0w = kt * KWG + wave * 32;
  const int jw = j0w + c32;
  const bool kvalid = jw < p.nk;
  const bool wave_keys = j0w < p.nk;
  const int64_t klast = wave_keys ? kid(min(j0w + 31, p.nk - 1)) : INT64_MAX;
  // First local query row that may see this lane's key (ids increase with the
  // row), and the same for the wave's last key: rows from imax_w on see every
  // key of the wave.  A lane past the block end keeps 0: its column is never
  // stored.
  const int imin = (p.causal && kvalid) ? first_query(qid, p.nq, kid(jw)) : 0;
  const int imax_w = (p.causal && wave_keys) ? first_query(qid, p.nq, klast) : 0;

  // B operands of S = Q K^T (and dP = dO V^T): this lane's K (V) row
  s16x8 kB[KS], vB[DK ? KS : 1];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s16x8 x = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if (kvalid) x = *(const s16x8 *)(kp + (int64_t)jw * p.ks_t + 16 * ks + 8 * hl);
    kB[ks] = x;
    if (DK) {
      s16x8 y = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
      if (kvalid) y = *(const s16x8 *)(vp + (int64_t)jw * p.vs_t + 16 * ks + 8 * hl);
      vB[DK ? ks : 0] = y;
    }
  }
  f32x16 acc[DT];  // dV^T or dK^T of this lane's key
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  // query tiles that can see any key of this workgroup, for every query head
  // of the K/V head: iteration f = hq * per + (qt - qt0), heads outermost
  const int64_t kwg = kid(min(kt * KWG, p.nk - 1));
  const int qt0 = (p.causal ? first_query(qid, p.nq, kwg) : 0) / kBT;
  const int nqt = (p.nq + kBT - 1) / kBT;
  const int per = nqt - qt0;
  const int nf = per > 0 ? G * per : 0;
  const int nq_pad = nqt * kBT;
  const uint32_t rowb = (uint32_t)p.qs_t * 2;
  const uint32_t vo_r = tile_voff<RB>(rowb, wave, lane), vo_t = tile_voff<TB>(TB, wave, lane);
  // Loads walk the tiles (head hq, query tile qt) in iteration order; the
  // buffer descriptors of a head are built when the walk reaches it.
  int iss_hq = 0, iss_qt = qt0;
  __amdgpu_buffer_rsrc_t r_q, r_do, r_t, r_nl, r_nD;
  auto set_head = [&](const int hq) {
    const int h = kvh * G + hq;
    const int64_t qoff = p.q_zstride * z + b * p.qs_b + h * p.qs_h;
    const int64_t rows_bytes = (int64_t)p.nq * rowb;
    r_q = rsrc((const short *)p.q + qoff, rows_bytes);
    if (DK) r_do = rsrc((const short *)P.dout + qoff, rows_bytes);
    const int64_t toff = P.qT_zstride * z + ((int64_t)b * p.Hq + h) * D * nq_pad;
    r_t = rsrc((const short *)(DK ? P.qT : P.doT) + toff, (int64_t)D * nq_pad * 2);
    const int64_t moff = p.ml_zstride * z + ((int64_t)b * p.Hq + h) * p.nq;
    r_nl = rsrc(P.nl + moff, (int64_t)p.nq * 4);
    if (DK) r_nD = rsrc(P.nD + moff, (int64_t)p.nq * 4);
  };
  set_head(0);
  // The next tile of the walk into `stage` (rows, the packed tile, the row
  // statistics), issued right after the barrier by the loading waves; then
  // the walk advances (every wave keeps it, only the loaders use it).
  auto issue = [&](const int stage) {
    char *st = lds + stage * ST;
    const uint32_t so = (uint32_t)iss_qt * kBT * rowb;
    if (wave < kLW) {
      load_tile<RB, kBT, kLW>(st, r_q, rowb, vo_r, so, wave);
      if (DK) load_tile<RB, kBT, kLW>(st + TQ, r_do, rowb, vo_r, so, wave);
      load_tile<TB, D, kLW>(st + OFF_T, r_t, TB, vo_t, (uint32_t)iss_qt * TT, wave);
    }
    if (wave == 0) {
      dma4b(r_nl, (lds_void *)(st + OFF_NL), lane * 4, (uint32_t)iss_qt * kBT * 4);
      if (DK) dma4b(r_nD, (lds_void *)(st + OFF_NL + kBT * 4), lane * 4, (uint32_t)iss_qt * kBT * 4);
    }
    if (++iss_qt == nqt) {
      iss_qt = qt0;
      if (++iss_hq < G) set_head(iss_hq);
    }
  };

  // Iteration f: tile f has landed (each loading wave waits for its own
  // loads, then the barrier) and stage (f+1)&1, last read in iteration f-1,
  // takes tile f+1.  FULL: every
  // query of the tile sees every key of the wave.
  auto step = [&](const int f, const int qt, auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const bool more = f + 1 < nf;
    if (more) issue((f + 1) & 1);
    const char *st = lds + (f & 1) * ST;
    const char *sQ = st, *sdO = st + TQ, *sT = st + OFF_T;
    const float *sNl = (const float *)(st + OFF_NL);
    const float *sND = sNl + kBT;
    const int i0 = qt * kBT;

    // The tile in two halves of 32 queries (ib): S (and dP - D) for the
    // half, then its two groups of 16 queries (kq = 2 ib + g) into the
    // gradient.  Element e of S is query 32 ib + 8(e/4) + 4 hl + e%4 of the
    // tile, key column jw.  The causal mask is the initial value of S: -inf
    // where the row comes before imin (p = exp2(S c + nl) = 0 there), else 0.
    // Rows past the end of the shard need none: their Q and dO rows and
    // packed columns are zero, so they add nothing.  Rows with no key at all
    // have nl = -inf, so p = 0.
    // A operands of S / dP run KA k-steps ahead; the first KA of half 1 and
    // its nl (and -D) are read during the gradient products of half 0; a
    // half's first dO^T / Q^T group during its own last k-steps.
    constexpr int KA = 2;
    s16x8 aq[2][KS], ao[2][DK ? KS : 1];
    float4 l4[2][4], nd4[2][DK ? 4 : 1];
    auto read_a = [&](const int ib, const int ks) {
      aq[ib][ks] = rd<RB>(sQ, 32 * ib + c32, 2 * ks + hl);
      if (DK) ao[ib][DK ? ks : 0] = rd<RB>(sdO, 32 * ib + c32, 2 * ks + hl);
    };
    auto read_rows = [&](const int ib) {  // nl (and -D) of the half's rows
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        l4[ib][rg] = *(const float4 *)(sNl + 32 * ib + 8 * rg + 4 * hl);
        if (DK) nd4[ib][DK ? rg : 0] = *(const float4 *)(sND + 32 * ib + 8 * rg + 4 * hl);
      }
    };
    read_rows(0);
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) read_a(0, ks);

    auto half = [&](const int ib) {
      f32x16 S, dP;
      if (DK) {  // dP starts at -D of its row, so the product leaves dP - D
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float4 x = nd4[ib][DK ? rg : 0];
          dP[4 * rg + 0] = x.x;
          dP[4 * rg + 1] = x.y;
          dP[4 * rg + 2] = x.z;
          dP[4 * rg + 3] = x.w;
        }
      }
      if (FULL) {
#pragma unroll
        for (int e = 0; e < 16; ++e) S[e] = 0.f;
      } else {
        const int lo = imin - (i0 + 32 * ib + 4 * hl);  // first allowed element row
#pragma unroll
        for (int e = 0; e < 16; ++e) S[e] = 8 * (e >> 2) + (e & 3) >= lo ? 0.f : -INFINITY;
      }
      s16x8 ct[2][DT];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + KA < KS) {
          read_a(ib, ks + KA);
        } else if (ks + KA == KS) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) ct[0][dt] = rd<TB>(sT, 32 * dt + c32, 4 * ib + hl);
        }
        S = M::mma(aq[ib][ks], kB[ks], S);
        if (DK) dP = M::mma(ao[ib][DK ? ks : 0], vB[DK ? ks : 0], dP);
        __builtin_amdgcn_sched_barrier(0);
      }
      auto elem = [&](const int g) {  // group g: registers 8g .. 8g+7, packed B operand
        f32x16 v;
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          const float4 x = l4[ib][2 * g + rg];
          const float nl[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int e = 8 * g + 4 * rg + u;
            const float pe = __builtin_amdgcn_exp2f(fmaf(S[e], c, nl[u]));
            v[4 * rg + u] = DK ? pe * dP[e] : pe;
          }
        }
        return M::pack(v, 0);
      };
      // group 1's operands are read and its P (dS) computed while the MFMAs
      // of group 0 run; during group 1's, the first operands of half 1
      s16x8 cur = elem(0);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if (g == 0) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) ct[1][dt] = rd<TB>(sT, 32 * dt + c32, 4 * ib + 2 + hl);
        } else if (ib == 0) {
          read_rows(1);
#pragma unroll
          for (int ks = 0; ks < KA; ++ks) read_a(1, ks);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = M::mma(ct[g][dt], cur, acc[dt]);
        if (g == 0) cur = elem(1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (DK) {
      half(0);
      half(1);
      return;
    }
    // dV: the two halves software-pipelined so that MFMA and VALU work
    // overlap inside the wave: S of half 1 runs under the exponentials of
    // group (0, 0); each group's dV^T MFMAs run under the next group's
    // exponentials.
    //   phase 0: S(0) | phase 1: S(1) + P(0,0) | phase 2: dV(0,0) + P(0,1) |
    //   phase 3: dV(0,1) + P(1,0) | phase 4: dV(1,0) + P(1,1) | phase 5: dV(1,1)
    f32x16 Sv[2];
    auto init_s = [&](const int ib) {
      if (FULL) {
#pragma unroll
        for (int e = 0; e < 16; ++e) Sv[ib][e] = 0.f;
      } else {
        const int lo = imin - (i0 + 32 * ib + 4 * hl);  // first allowed element row
#pragma unroll
        for (int e = 0; e < 16; ++e) Sv[ib][e] = 8 * (e >> 2) + (e & 3) >= lo ? 0.f : -INFINITY;
      }
    };
    // A operands of S: one stream over both halves' 2 KS k-steps, KA ahead
    auto read_next = [&](const int kk) {  // k-step kk of the 2 KS stream
      if (kk < 2 * KS) read_a(kk / KS, kk % KS);
    };
    auto pe_of = [&](const int ib, const int g, const int u8) {  // element u8 of group (ib, g)
      const int rg = u8 >> 2, u = u8 & 3;
      const float4 x = l4[ib][2 * g + rg];
      const float nl = u == 0 ? x.x : (u == 1 ? x.y : (u == 2 ? x.z : x.w));
      return __builtin_amdgcn_exp2f(fmaf(Sv[ib][8 * g + u8], c, nl));
    };
    s16x8 cv[2][DT];  // dO^T fragments of two groups
    auto read_ct = [&](const int gi) {  // group gi = 2 ib + g into buffer gi & 1
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) cv[gi & 1][dt] = rd<TB>(sT, 32 * dt + c32, 2 * gi + hl);
    };
    init_s(0);
    // phase 0
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      read_next(ks + KA);
      if (ks == 0) read_rows(1);
      Sv[0] = M::mma(aq[0][ks], kB[ks], Sv[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    init_s(1);
    // phase 1
    f32x16 pv;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      read_next(KS + ks + KA);
      if (ks == 1) read_ct(0);
      if (ks == KS - 2) read_ct(1);
      Sv[1] = M::mma(aq[1][ks], kB[ks], Sv[1]);
#pragma unroll
      for (int u8 = (8 * ks) / KS; u8 < (8 * (ks + 1)) / KS; ++u8) pv[u8] = pe_of(0, 0, u8);
      __builtin_amdgcn_sched_barrier(0);
    }
    s16x8 cur = M::pack(pv, 0);
    // phases 2..5: group gi's MFMAs, two elements of group gi + 1 per MFMA
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if (gi >= 1 && gi + 1 < 4) read_ct(gi + 1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        acc[dt] = M::mma(cv[gi & 1][dt], cur, acc[dt]);
        if (gi + 1 < 4) {
#pragma unroll
          for (int u8 = (8 * dt) / DT; u8 < (8 * (dt + 1)) / DT; ++u8)
            pv[u8] = pe_of((gi + 1) >> 1, (gi + 1) & 1, u8);
        }
      }
      if (gi + 1 < 4) cur = M::pack(pv, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Per wave the tiles of each query head come as a run of partial tiles (the
  // causal diagonal; a tile where the wave sees nothing runs fully masked, so
  // the accumulator stays on one path) and then a run of full ones: two loops
  // with one body each keep the mask code out of the full tiles.
  if (nf > 0) issue(0);
  int f = 0, qt = qt0;  // qt: query tile of iteration f
  auto next = [&]() {
    ++f;
    if (++qt == nqt) qt = qt0;
  };
  while (f < nf) {
    for (; f < nf && qt * kBT < imax_w; next()) step(f, qt, std::false_type());
    for (; f < nf && qt * kBT >= imax_w; next()) step(f, qt, std::true_type());
  }
  if (!kvalid) return;
  // element e of acc[dt]: d = 32dt + 8(e/4) + 4hl + e%4 of key jw
  const int64_t ko = P.dk_zstride * kvi + ((int64_t)(b * p.Hkv + kvh) * p.nk + jw) * D;
  float *out = (DK ? P.dk : P.dv) + ko;
  const float sc = DK ? p.scale : 1.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int dd = 32 * dt + 8 * rg + 4 * hl;
      float4 a = *(float4 *)(out + dd);
      a.x += sc * acc[dt][4 * rg + 0];
      a.y += sc * acc[dt][4 * rg + 1];
      a.z += sc * acc[dt][4 * rg + 2];
      a.w += sc * acc[dt][4 * rg + 3];
      *(float4 *)(out + dd) = a;
    }
}

template <int D, bool BF16>
__global__ void __launch_bounds__(kQW * 64) bwd_dq_kernel(BwdParams P) {
  using M = Mfma16<BF16>;
  const BatchParams &p = P.a;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int RB = D * 2;    // bytes of a K / V row
  constexpr int TB = kBT * 2;  // bytes of a packed K^T row (64 keys)
  constexpr int TQ = kBT * RB;
  constexpr int TT = D * TB;
  constexpr size_t ST = dq_stage_bytes<D>();
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  // stage layout: sK | sV | sKT

  // workgroup -> (query tile, problem, batch, query head); query tile slowest,
  // last tiles (most keys before them) first
  constexpr int QWG = kQW * 32;  // queries per workgroup
  const int nqt = (p.nq + QWG - 1) / QWG;
  const int per_qt = p.nz * p.B * p.Hq;
  int idx = blockIdx.x;
  const int qtr = idx / per_qt;
  idx -= qtr * per_qt;
  const int qt = p.causal ? nqt - 1 - qtr : qtr;
  const int h = idx % p.Hq;
  idx /= p.Hq;
  const int b = idx % p.B;
  const int z = idx / p.B;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;
  const IdMap qid = query_ids(p, z), kid = key_ids(p, z);
  const int kvh = h / (p.Hq / p.Hkv);
  const int kvi = (p.kv_idx0 + z) % p.kv_idx_mod;
  const short *kp = (const short *)p.k + kvi * p.kv_zstride + b * p.ks_b + kvh * p.ks_h;
  const short *vp = (const short *)p.v + kvi * p.kv_vzstride + b * p.vs_b + kvh * p.vs_h;
  const int nk_pad = (p.nk + 63) / 64 * 64;
  const short *kT = (const short *)P.kT + P.kT_zstride * kvi + ((int64_t)b * p.Hkv + kvh) * D * nk_pad;
  const float c = p.scale * kLog2e;

  // this wave's 32 queries and this lane's query
  const int iw0 = qt * QWG + wave * 32;
  const int iw = iw0 + c32;
  const bool valid = iw < p.nq;
  const int64_t qoff = p.q_zstride * z + b * p.qs_b + h * p.qs_h;
  s16x8 qB[KS], dB[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s16x8 x = (s16x8){0, 0, 0, 0, 0, 0, 0, 0}, y = x;
    if (valid) {
      x = *(const s16x8 *)((const short *)p.q + qoff + (int64_t)iw * p.qs_t + 16 * ks + 8 * hl);
      y = *(const s16x8 *)((const short *)P.dout + qoff + (int64_t)iw * p.qs_t + 16 * ks + 8 * hl);
    }
    qB[ks] = x;
    dB[ks] = y;
  }
  const int64_t moff = p.ml_zstride * z + ((int64_t)b * p.Hq + h) * p.nq;
  float nl = -INFINITY, nd = 0.f;
  if (valid) {
    nl = P.nl[moff + iw];
    nd = P.nD[moff + iw];
  }
  const int jlim = valid ? key_prefix(p, kid, qid(iw)) : 0;
  const int iw_last = min(iw0 + 31, p.nq - 1), i_wg_last = min(qt * QWG + QWG - 1, p.nq - 1);
  const bool wave_rows = iw0 < p.nq;
  const int ntiles = (key_prefix(p, kid, qid(i_wg_last)) + kBT - 1) / kBT;
  const int ntiles_w = wave_rows ? (key_prefix(p, kid, qid(iw_last)) + kBT - 1) / kBT : 0;
  const int nfull_w = wave_rows ? key_prefix(p, kid, qid(iw0)) / kBT : 0;

  const uint32_t rowb = (uint32_t)p.ks_t * 2, vrowb = (uint32_t)p.vs_t * 2;
  const int64_t kbytes = (int64_t)p.nk * rowb;
  const auto kr = rsrc(kp, kbytes), vr = rsrc(vp, (int64_t)p.nk * vrowb),
             tr = rsrc(kT, (int64_t)D * nk_pad * 2);
  const uint32_t vo_k = tile_voff<RB>(rowb, wave, lane), vo_v = tile_voff<RB>(vrowb, wave, lane),
                 vo_t = tile_voff<TB>(TB, wave, lane);
  // tile t into `stage` (K rows, V rows, packed K^T), issued right after the
  // barrier by the loading waves only
  auto issue = [&](int t, int stage) {
    if (wave >= kLW) return;
    char *st = lds + stage * ST;
    load_tile<RB, kBT, kLW>(st, kr, rowb, vo_k, (uint32_t)t * kBT * rowb, wave);
    load_tile<RB, kBT, kLW>(st + TQ, vr, vrowb, vo_v, (uint32_t)t * kBT * vrowb, wave);
    load_tile<TB, D, kLW>(st + 2 * TQ, tr, TB, vo_t, (uint32_t)t * TT, wave);
  };

  f32x16 dQt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dQt[dt][e] = 0.f;

  // Iteration t: tile t has landed, stage (t+1)&1 takes tile t+1.  MODE 2: a
  // full tile (every key allowed for every query of the wave), 1: a diagonal
  // or ragged one, whose mask is the initial value of S^T (-inf for keys at or
  // past jlim, which includes keys past the block end), 0: nothing for this
  // wave, loads only.
  auto step = [&](const int t, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const bool more = t + 1 < ntiles;
    if (more) issue(t + 1, (t + 1) & 1);
    if (MODE == 0) return;
    const char *st = lds + (t & 1) * ST;
    const char *sK = st, *sV = st + TQ, *sKT = st + 2 * TQ;
    const int j0 = t * kBT;
    // S^T = K Q^T and dP^T = V dO^T, A operands one k-step ahead; dP^T starts
    // at -D of this lane's row, so the product leaves dP - D.  Element e of
    // S^T[kb] is key j0 + 32kb + 8(e/4) + 4hl + e%4 of this lane's query.
    f32x16 S[2], dP[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        S[kb][e] = MODE == 2 || j0 + 32 * kb + 8 * (e >> 2) + 4 * hl + (e & 3) < jlim
                       ? 0.f
                       : -INFINITY;
        dP[kb][e] = nd;
      }
    s16x8 ak[KS][2], av[KS][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      ak[0][kb] = rd<RB>(sK, 32 * kb + c32, hl);
      av[0][kb] = rd<RB>(sV, 32 * kb + c32, hl);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          ak[ks + 1][kb] = rd<RB>(sK, 32 * kb + c32, 2 * (ks + 1) + hl);
          av[ks + 1][kb] = rd<RB>(sV, 32 * kb + c32, 2 * (ks + 1) + hl);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        S[kb] = M::mma(ak[ks][kb], qB[ks], S[kb]);
        dP[kb] = M::mma(av[ks][kb], dB[ks], dP[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // group kq (16 keys: half kq/2, registers 8(kq%2) .. +7): dS^T packed
    auto elem = [&](int kq) {
      const int kb = kq >> 1, e0 = 8 * (kq & 1);
      f32x16 dv;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u;
        const float pe = __builtin_amdgcn_exp2f(fmaf(S[kb][e], c, nl));
        dv[u] = pe * dP[kb][e];
      }
      return M::pack(dv, 0);
    };
    // dQ^T += K^T dS^T over the tile's 64 keys, group kq + 1 prepared while
    // the MFMAs of group kq run
    s16x8 ct[4][DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ct[0][dt] = rd<TB>(sKT, 32 * dt + c32, hl);
    s16x8 cur = elem(0);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      if (kq + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) ct[kq + 1][dt] = rd<TB>(sKT, 32 * dt + c32, 2 * (kq + 1) + hl);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dQt[dt] = M::mma(ct[kq][dt], cur, dQt[dt]);
      if (kq + 1 < 4) cur = elem(kq + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the wave's tiles come as full ones, then diagonal / ragged ones, then
  // ones it has nothing in: one loop per kind keeps the mask code out of the
  // full tiles
  if (ntiles > 0) issue(0, 0);
  const int nfull = min(nfull_w, ntiles_w);
  int t = 0;
  for (; t < nfull; ++t) step(t, std::integral_constant<int, 2>());
  for (; t < ntiles_w; ++t) step(t, std::integral_constant<int, 1>());
  for (; t < ntiles; ++t) step(t, std::integral_constant<int, 0>());
  if (!valid) return;
  float *dq = P.dq + P.dq_zstride * z + (((int64_t)b * p.Hq + h) * p.nq + iw) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * dt + 8 * rg + 4 * hl;
      float4 a = *(float4 *)(dq + d0);
      a.x += p.scale * dQt[dt][4 * rg + 0];
      a.y += p.scale * dQt[dt][4 * rg + 1];
      a.z += p.scale * dQt[dt][4 * rg + 2];
      a.w += p.scale * dQt[dt][4 * rg + 3];
      *(float4 *)(dq + d0) = a;
    }
}

// Per query row (16-bit inputs, one wave per row): nD = -<dO, O> (the
// starting value of the dP accumulators, which then hold dP - D), and the
// exponent offset nl = -lse log2(e) of p = exp2(s c + nl), -inf for a row
// with no key (lse = -inf), so that its probabilities come out as 0.
template <typename T>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const T *__restrict__ o,
                                                       const T *__restrict__ dout,
                                                       const float *__restrict__ lse,
                                                       float *__restrict__ nD,
                                                       float *__restrict__ nl, int64_t rows,
                                                       int d) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int c = lane; c < d; c += 64)
    acc += (float)o[row * d + c] * (float)dout[row * d + c];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    nD[row] = -acc;
    const float x = lse[row];
    nl[row] = x > -INFINITY ? -x * kLog2e : -INFINITY;
  }
}

__global__ void __launch_bounds__(256) zero_kernel(float4 *__restrict__ x, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) x[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename T>
__global__ void __launch_bounds__(256) cast_kernel(const float4 *__restrict__ x,
                                                   T *__restrict__ y, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = x[i];
  T *o = y + 4 * i;
  o[0] = (T)v.x;
  o[1] = (T)v.y;
  o[2] = (T)v.z;
  o[3] = (T)v.w;
}

// parts: bit 0 the dK/dV kernels, bit 1 the dQ kernel
template <int D, bool BF16>
hipError_t launch_bwd_d(const BwdParams &P, hipStream_t s, int parts) {
  const BatchParams &p = P.a;
  const int64_t groups = (int64_t)p.nz * p.B;
  constexpr size_t lv = 2 * kv_stage_bytes<D, kRoleV>(), lk = 2 * kv_stage_bytes<D, kRoleK>(),
                   l2 = 2 * dq_stage_bytes<D>();
  // more than 64 KB of LDS per workgroup must be opted into, once per process
  // (a function-local static: initialised once even with several host threads)
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute((const void *)bwd_kv_kernel<D, BF16, kRoleV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lv);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)bwd_kv_kernel<D, BF16, kRoleK>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lk);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)bwd_dq_kernel<D, BF16>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)l2);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (p.nk > 0 && (parts & 1)) {
    const int64_t n1 = groups * p.Hkv * ((p.nk + kKW * 32 - 1) / (kKW * 32));
    hipLaunchKernelGGL((bwd_kv_kernel<D, BF16, kRoleV>), dim3((unsigned)n1), dim3(kKW * 64), lv,
                       s, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_kv_kernel<D, BF16, kRoleK>), dim3((unsigned)n1), dim3(kKW * 64), lk,
                       s, P);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(parts & 2)) return hipSuccess;
  const int64_t n2 = groups * p.Hq * ((p.nq + kQW * 32 - 1) / (kQW * 32));
  hipLaunchKernelGGL((bwd_dq_kernel<D, BF16>), dim3((unsigned)n2), dim3(kQW * 64), l2, s, P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const void *o, const void *dout, const float *lse, float *nD,
                           float *nl, int dtype, int64_t rows, int32_t d, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (dtype == RA_DT_BF16)
    hipLaunchKernelGGL(bwd_prep_kernel<__bf16>, dim3(blocks), dim3(256), 0, s,
                       (const __bf16 *)o, (const __bf16 *)dout, lse, nD, nl, rows, d);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<_Float16>, dim3(blocks), dim3(256), 0, s,
                       (const _Float16 *)o, (const _Float16 *)dout, lse, nD, nl, rows, d);
  return hipGetLastError();
}

hipError_t launch_zero(float *x, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;  // callers pass multiples of 4 (rows of d floats)
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     (float4 *)x, n4);
  return hipGetLastError();
}

hipError_t launch_cast(const float *x, void *y, int dtype, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const dim3 g((unsigned)((n4 + 255) / 256));
  if (dtype == RA_DT_BF16)
    hipLaunchKernelGGL(cast_kernel<__bf16>, g, dim3(256), 0, s, (const float4 *)x, (__bf16 *)y, n4);
  else
    hipLaunchKernelGGL(cast_kernel<_Float16>, g, dim3(256), 0, s, (const float4 *)x,
                       (_Float16 *)y, n4);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams &p, int dtype, hipStream_t s, int parts) {
  if (p.a.nq == 0) return hipSuccess;
  if (dtype == RA_DT_BF16)
    return p.a.d == 64 ? launch_bwd_d<64, true>(p, s, parts) : launch_bwd_d<128, true>(p, s, parts);
  return p.a.d == 64 ? launch_bwd_d<64, false>(p, s, parts) : launch_bwd_d<128, false>(p, s, parts);
}

}  // namespace ra
