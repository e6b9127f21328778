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
  constexpr int KINSTR = KTILE / 1024;   // 1 KB wave-instructions per K tile
  constexpr int VINSTR = VTILE / 1024;
  constexpr int KRPI = 1024 / KROW;      // K rows per wave-instruction
  constexpr int CPR = D / 8;             // 16-byte chunks per K row
  static_assert(KINSTR % kPW == 0 && VINSTR % kPW == 0, "tile must split over the waves");
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const Work w = decode(p, ntq);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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

    auto issue = [&](int t, int buf) {
      char *st = lds + buf * STAGE;
#pragma unroll
      for (int u = 0; u < KINSTR / kPW; ++u) {
        const int idx = wave + kPW * u;
        const int r = idx * KRPI + lane / CPR;
        const int lch = (lane % CPR) ^ (r & 7);
        int j = t * kPBN + r;
        j = j < p.nk ? j : p.nk - 1;
        dma16(kp + (int64_t)j * p.ks_t + lch * 8, st + idx * 1024);
      }
#pragma unroll
      for (int u = 0; u < VINSTR / kPW; ++u) {
        const int idx = wave + kPW * u;
        const int dr = idx * 8 + (lane >> 3);
        const int lch = (lane & 7) ^ (dr & 7);
        dma16(vp + (int64_t)dr * p.vs_t + t * kPBN + lch * 8, st + KTILE + idx * 1024);
      }
    };

    issue(0, 0);
    for (int t = 0; t < ntiles; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (t + 1 < ntiles) issue(t + 1, (t + 1) & 1);
      if (t < ntiles_w) {
        const char *st = lds + (t & 1) * STAGE;
        f32x16 S[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) S[kh][r] = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int r = kh * 32 + c32;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const s16x8 a = *(const s16x8 *)(st + r * KROW + (((2 * ks + hl) ^ (r & 7)) << 4));
            S[kh] = M::mma(a, qf[ks], S[kh]);
          }
        }
        if (t >= nfull_w) {  // causal diagonal or ragged end of the block
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = t * kPBN + kh * 32 + (r >> 2) * 8 + 4 * hl + (r & 3);
              if (j >= jlim) S[kh][r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kh][r]);
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
        float ls = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            f32x16 pv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pv[e] = __builtin_amdgcn_exp2f(fmaf(S[kh][8 * cc + e], c, nm));
              ls += pv[e];
            }
            const s16x8 P = M::pack(pv, 0);
            const int lc = 4 * kh + 2 * cc + hl;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const int dr = 32 * dt + c32;
              const s16x8 a = *(const s16x8 *)(st + KTILE + dr * VROW + ((lc ^ (dr & 7)) << 4));
              O[dt] = M::mma(a, P, O[dt]);
            }
          }
        lsum += ls;
      }
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
  const size_t lds = (size_t)2 * (kPBN * D * 2 + D * kPBN * 2);
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
