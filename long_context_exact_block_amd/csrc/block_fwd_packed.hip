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
//  * K and V^T tiles go from HBM straight into LDS with global_load_lds
//    (no staging registers), double-buffered with one barrier per tile; 16-byte
//    chunks are XOR-swizzled by row so every LDS read pattern is conflict-free.
//  * 8 waves x 32 queries per workgroup (256 rows), two waves per SIMD, so one
//    wave's softmax VALU work overlaps the other's MFMAs.
#include <cfloat>
#include <cmath>

#include "attn_common.h"

namespace ra {
namespace {

using namespace attn;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kPW = 8;          // waves per workgroup
constexpr int kPBM = kPW * 32;  // query rows per workgroup
constexpr int kPBN = 64;        // keys per tile

// 16 bytes per lane from global memory straight into LDS at lds_wave_base +
// 16*lane (the LDS base must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void *g, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)g, (lds_void_t *)lds_wave_base, 16, 0, 0);
}

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

// s_waitcnt with only vmcnt limited (expcnt, lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
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
  constexpr int NSTAGE = 4;              // LDS stages: tiles t, t+1 read; t+2, t+3 landing
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
    auto issue = [&](int t, int stage) {
      char *st = lds + stage * STAGE;
      const int64_t koffs = (int64_t)t * kPBN * p.ks_t;
      const bool tail = (t + 1) * kPBN > p.nk;  // ragged last tile: clamp rows
#pragma unroll
      for (int u = 0; u < KPW; ++u) {
        const short *src = ksrc[u] + koffs;
        if (tail) {
          int j = t * kPBN + krow[u];
          j = j < p.nk ? j : p.nk - 1;
          src = kp + (int64_t)j * p.ks_t + klch[u] * 8;
        }
        dma16(src, st + (wave + kPW * u) * 1024);
      }
#pragma unroll
      for (int u = 0; u < VPW; ++u)
        dma16(vsrc[u] + t * kPBN, st + KTILE + (wave + kPW * u) * 1024);
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

    // Prologue: up to three tiles in flight, tile 0 resident.
    issue(0, 0);
    if (ntiles > 1) issue(1, 1);
    if (ntiles > 2) issue(2, 2);
    if (ntiles > 2)
      wait_vmcnt<2 * (KPW + VPW)>();
    else if (ntiles > 1)
      wait_vmcnt<KPW + VPW>();
    else
      wait_vmcnt<0>();
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
      if (t + 1 < ntiles) {
        if (t + 2 < ntiles)
          wait_vmcnt<KPW + VPW>();  // tile t+1 landed; t+2 may be in flight
        else
          wait_vmcnt<0>();
        __syncthreads();
        if (t + 3 < ntiles) issue(t + 3, (u + 3) % NSTAGE);
      }
      if (t >= ntiles_w) return;
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
      s16x8 ka[KS][2];
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          ka[ks][kh] = *(const s16x8 *)(stn + koff[ks] + kh * 32 * KROW);
      float ls = 0.f;
      f32x16 pbuf;
      s16x8 P[4];
#pragma unroll
      for (int step = 0; step < NSTEP; ++step) {
        const int ks = step >> 1, kh = step & 1;
        if (step == 2) {  // second half of the K fragments
#pragma unroll
          for (int k2 = KS / 2; k2 < KS; ++k2)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              ka[k2][h2] = *(const s16x8 *)(stn + koff[k2] + h2 * 32 * KROW);
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
    };
    for (int t = 0; t < ntiles; ++t) {
      tile(t, t % NSTAGE, S, S1);
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) S[kh] = S1[kh];
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
  const size_t lds = (size_t)4 * (kPBN * D * 2 + D * kPBN * 2);
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
