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
//  * K and V^T tiles are prefetched two tiles ahead: each wave loads its
//    share into registers right after the tile's barrier and writes it to a
//    free LDS stage after its compute (three stages, one barrier per tile);
//    16-byte chunks are XOR-swizzled by row for gfx950's 64 LDS banks so every
//    read pattern is conflict-free.
//  * 8 waves x 32 queries per workgroup (256 rows), two waves per SIMD; QK of
//    tile t+1 is interleaved with the exponentials of tile t and PV of tile t
//    with the row max of tile t+1.
#include <cfloat>
#include <cmath>

#include "attn_common.h"

namespace ra {
namespace {

using namespace attn;

constexpr int kPW = 8;          // waves per workgroup
constexpr int kPBM = kPW * 32;  // query rows per workgroup
constexpr int kPBN = 64;        // keys per tile

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

template <int D, bool BF16>
__global__ void __launch_bounds__(512) attn_packed_kernel(BatchParams p, int ntq) {
  using M = Mfma16<BF16>;
  constexpr int KS = D / 16;             // k-steps of the QK product
  constexpr int DT = D / 32;             // 32-wide d tiles of O
  constexpr int KROW = D * 2;            // bytes per K row in LDS
  constexpr int KTILE = kPBN * KROW;     // bytes of a K tile
  constexpr int VROW = kPBN * 2;         // bytes per V^T row (64 keys)
  constexpr int VTILE = D * VROW;        // bytes of a V^T tile
  constexpr int STAGE = KTILE + VTILE;
  constexpr int NSTAGE = 3;              // LDS stages: tiles t, t+1 read; t+2 being written
  constexpr int KINSTR = KTILE / 1024;   // 1 KB wave-instructions per K tile
  constexpr int VINSTR = VTILE / 1024;
  constexpr int KPW = KINSTR / kPW;      // per wave per tile
  constexpr int VPW = VINSTR / kPW;
  constexpr int KRPI = 1024 / KROW;      // K rows per wave-instruction
  constexpr int CPR = D / 8;             // 16-byte chunks per K row
  static_assert(KINSTR % kPW == 0 && VINSTR % kPW == 0, "tile must split over the waves");
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const Work w = decode(p, ntq);
  // the wave index is uniform: keep it in a scalar register
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;

  const short *qp = (const short *)p.q + w.z * p.q_zstride + w.b * p.qs_b + w.h * p.qs_h;
  const int kvi = (p.kv_idx0 + w.z) % p.kv_idx_mod;
  const short *kp = (const short *)p.k + kvi * p.kv_zstride + w.b * p.ks_b + w.kvh * p.ks_h;
  const short *vp = (const short *)p.v + kvi * p.kv_vzstride + w.b * p.vs_b + w.kvh * p.vs_h;
  const int64_t qg0 = p.qg_add + w.z * p.qg_z;
  const int64_t kg0 = p.kg_add + (int64_t)((p.kg_s0 + w.z) % p.kg_smod) * p.kg_mult;
  const float c = p.scale * kLog2e;

  const int i_wg0 = w.qtile * kPBM;
  const int i_wg1 = min(p.nq, i_wg0 + kPBM) - 1;
  const int iw0 = i_wg0 + wave * 32;
  const int iw1 = min(p.nq - 1, iw0 + 31);
  const bool wave_rows = iw0 < p.nq;
  const int i = iw0 + c32;
  const bool valid = i < p.nq;

  const int kv_wg = key_prefix(p, kg0, qg0 + (int64_t)i_wg1 * p.q_step);
  const int ntiles = (kv_wg + kPBN - 1) / kPBN;
  const int kv_wl = wave_rows ? key_prefix(p, kg0, qg0 + (int64_t)iw1 * p.q_step) : 0;
  const int kv_wf = wave_rows ? key_prefix(p, kg0, qg0 + (int64_t)iw0 * p.q_step) : 0;
  const int ntiles_w = (kv_wl + kPBN - 1) / kPBN;
  const int nfull_w = kv_wf / kPBN;
  const int jlim = key_prefix(p, kg0, qg0 + (int64_t)i * p.q_step);

  if (ntiles == 0 && p.accumulate) return;  // nothing to add to the running state

  f32x16 O[DT];
  float m_run, m_top, lsum;
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

  if (ntiles > 0) {
    // Q fragments (B operand of S^T = K Q^T): d = 16ks + 8hl .. +7 of this lane's row
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

    // Per-lane DMA sources for tile 0 (later tiles add a uniform offset) and
    // the matching LDS destinations (uniform per wave).
    const short *ksrc[KPW];
    int krow[KPW], klch[KPW];
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const int idx = wave + kPW * u;
      krow[u] = idx * KRPI + lane / CPR;
      klch[u] = (lane % CPR) ^ chunk_swz<KROW>(krow[u]);
      ksrc[u] = kp + (int64_t)krow[u] * p.ks_t + klch[u] * 8;
    }
    const short *vsrc[VPW];
#pragma unroll
    for (int u = 0; u < VPW; ++u) {
      const int idx = wave + kPW * u;
      const int dr = idx * 8 + (lane >> 3);
      vsrc[u] = vp + (int64_t)dr * p.vs_t + (((lane & 7) ^ chunk_swz<VROW>(dr)) * 8);
    }
    // One wave's share of a tile is KPW + VPW 16-byte-per-lane pieces.
    // fetch() loads them into registers (asynchronous; a wave may have many
    // loads in flight), commit() writes them into an LDS stage.  gfx950's
    // global_load_lds stalls the issuing wave until its data has landed, so
    // it is not used for the per-tile prefetch.
    // (returned by value: an array captured by the lambdas would be demoted
    // to scratch memory)
    struct Staged {
      uint4 v[KPW + VPW];
    };
    auto fetch = [&](int t) {
      Staged g;
      const bool tail = (t + 1) * kPBN > p.nk;  // ragged last tile: clamp K rows
#pragma unroll
      for (int u = 0; u < KPW; ++u) {
        const short *src = ksrc[u] + (int64_t)t * kPBN * p.ks_t;
        if (tail) {
          int j = t * kPBN + krow[u];
          j = j < p.nk ? j : p.nk - 1;
          src = kp + (int64_t)j * p.ks_t + klch[u] * 8;
        }
        g.v[u] = *(const uint4 *)src;
      }
#pragma unroll
      for (int u = 0; u < VPW; ++u) g.v[KPW + u] = *(const uint4 *)(vsrc[u] + t * kPBN);
      return g;
    };
    auto commit = [&](const Staged &g, int stage) {
      char *st = lds + stage * STAGE + lane * 16;
#pragma unroll
      for (int u = 0; u < KPW; ++u) *(uint4 *)(st + (wave + kPW * u) * 1024) = g.v[u];
#pragma unroll
      for (int u = 0; u < VPW; ++u) *(uint4 *)(st + KTILE + (wave + kPW * u) * 1024) = g.v[KPW + u];
    };

    // Per-lane LDS read offsets within a stage.  Row kh*32 + c32 (K) and
    // 32dt + c32 (V^T) share the swizzle of row c32, so kh and dt become
    // immediate offsets.
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      koff[ks] = c32 * KROW + (((2 * ks + hl) ^ chunk_swz<KROW>(c32)) << 4);
    int voff[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)  // q4 = 2*kh + cc -> logical chunk 2*q4 + hl
      voff[q4] = KTILE + c32 * VROW + (((2 * q4 + hl) ^ chunk_swz<VROW>(c32)) << 4);

    // S^T = K Q^T for tile t into dst (prologue only; the loop interleaves it)
    auto qk = [&](int t, f32x16 (&dst)[2]) {
      const char *st = lds + (t % NSTAGE) * STAGE;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[kh][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          dst[kh] = M::mma(*(const s16x8 *)(st + koff[ks] + kh * 32 * KROW), qf[ks], dst[kh]);
    };
    auto rowmax = [&](const f32x16 (&x)[2]) {
      float m = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, x[kh][r]);
      return m;
    };

    // Prologue: tiles 0 and 1 resident.
    commit(fetch(0), 0);
    if (ntiles > 1) commit(fetch(1), 1);
    __syncthreads();
    f32x16 S[2];
    float mx = -INFINITY;  // row max of S (before masking)
    if (0 < ntiles_w) {
      qk(0, S);
      mx = rowmax(S);
    }

    // Iteration t: softmax and PV of tile t, overlapped with QK of tile t+1
    // and the row max of tile t+1.  Stage (t+3) % 4 == (t-1) % 4 was last
    // read in iteration t-1, so after the barrier it can receive tile t+3.
    constexpr int NSTEP = 2 * KS;      // QK MFMAs per tile (two 32-key halves)
    constexpr int EPS = 32 / NSTEP;    // exponentials per QK MFMA
    f32x16 S1[2];
    auto tile = [&](const int t, const int u, f32x16 (&Sc)[2], f32x16 (&Sn)[2]) {
      // u == t % NSTAGE
      // Tile t+1 was committed at the end of tile t-1; after this barrier it
      // is visible, and stage (t+2) % 3 -- last read in tile t-1 -- is free.
      if (t + 1 < ntiles && t > 0) __syncthreads();
      const bool pre = t + 2 < ntiles;
      Staged g;
      if (pre) g = fetch(t + 2);  // in flight during this tile's compute
      if (t >= ntiles_w) {
        if (pre) commit(g, (u + 2) % NSTAGE);
        return;
      }
      if (t >= nfull_w) {  // causal diagonal or ragged end of the block
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = t * kPBN + kh * 32 + (r >> 2) * 8 + 4 * hl + (r & 3);
            if (j >= jlim) Sc[kh][r] = -INFINITY;
          }
        mx = rowmax(Sc);
      }
      mx = half_max(mx);
      const float mt = mx * c;
      m_top = fmaxf(m_top, mt);
      if (wave_any(mt > m_run + kTau)) {
        const float mn = fmaxf(m_run, mt);
        const float al = __builtin_amdgcn_exp2f(m_run - mn);
        lsum *= al;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[dt][r] *= al;
        m_run = mn;
      }
      const float nm = -m_run;

      // Part 1: QK of the next tile (from a resident stage; discarded when
      // the wave has no next tile), one MFMA at a time, each followed by a
      // share of this tile's exponentials.
      const char *stn = lds + (t + 1 < ntiles ? (u + 1) % NSTAGE : u) * STAGE;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) Sn[kh][r] = 0.f;
      // K fragments in a rolling window: those of k-step ks + 1 are read
      // while k-step ks is multiplied
      s16x8 ka[KS][2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) ka[0][kh] = *(const s16x8 *)(stn + koff[0] + kh * 32 * KROW);
      float ls = 0.f;
      f32x16 pbuf;
      s16x8 P[4];
#pragma unroll
      for (int step = 0; step < NSTEP; ++step) {
        const int ks = step >> 1, kh = step & 1;
        if (kh == 0 && ks + 1 < KS) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            ka[ks + 1][h2] = *(const s16x8 *)(stn + koff[ks + 1] + h2 * 32 * KROW);
        }
        Sn[kh] = M::mma(ka[ks][kh], qf[ks], Sn[kh]);
#pragma unroll
        for (int v = 0; v < EPS; ++v) {
          const int e = EPS * step + v;  // element of S: half e/16, register e%16
          const float pv = __builtin_amdgcn_exp2f(fmaf(Sc[e >> 4][e & 15], c, nm));
          ls += pv;
          pbuf[e & 7] = pv;
          if ((e & 7) == 7) P[e >> 3] = M::pack(pbuf, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      lsum += ls;

      // Part 2: PV of this tile, each group of MFMAs followed by a share of
      // the next tile's row max.
      const char *st = lds + u * STAGE;
      float mxn = -INFINITY;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        s16x8 a[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          a[dt] = *(const s16x8 *)(st + voff[q4] + dt * 32 * VROW);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] = M::mma(a[dt], P[q4], O[dt]);
#pragma unroll
        for (int r = 0; r < 8; ++r) mxn = fmaxf(mxn, Sn[q4 >> 1][8 * (q4 & 1) + r]);
        __builtin_amdgcn_sched_barrier(0);
      }
      mx = mxn;
      if (pre) commit(g, (u + 2) % NSTAGE);
    };
    // two tiles per iteration so the S register sets swap roles instead of
    // being copied
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, t % NSTAGE, S, S1);
      if (t + 1 >= ntiles) break;
      tile(t + 1, (t + 1) % NSTAGE, S1, S);
    }
  }
  store_state<D>(p, w, i, valid, O, m_run, m_top, lsum);
}

// V rows [b][h][j][c] (strides) -> packed [bh][c][n_pad]; one workgroup per
// (bh, 64-key window): coalesced 16-byte loads of key rows, LDS transpose,
// coalesced 16-byte stores of 8 packed positions.
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
  short *dst = vp + bh * (int64_t)d * n_pad + j0;
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
    *(uint4 *)(dst + (int64_t)cidx * n_pad + g * 8) = val;
  }
}

template <int D, bool BF16>
hipError_t launch_packed(const BatchParams &p, hipStream_t s) {
  const int ntq = (p.nq + kPBM - 1) / kPBM;
  const int64_t nwg = (int64_t)ntq * p.nz * p.B * p.Hq;
  const size_t lds = (size_t)3 * (kPBN * D * 2 + D * kPBN * 2);
  static bool attr_set = false;  // more than 64 KB of LDS per workgroup must be opted into
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_packed_kernel<D, BF16>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((attn_packed_kernel<D, BF16>), dim3((unsigned)nwg), dim3(512), lds, s, p,
                     ntq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_fwd_packed(const BatchParams &p, int dtype, hipStream_t s) {
  if (dtype == RA_DT_BF16) return p.d == 64 ? launch_packed<64, true>(p, s) : launch_packed<128, true>(p, s);
  return p.d == 64 ? launch_packed<64, false>(p, s) : launch_packed<128, false>(p, s);
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
