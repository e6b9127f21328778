// block_fwd.hip -- partial attention of query shards against K/V blocks on
// gfx950 matrix cores, with the online-softmax running state either written
// fresh (one hop's partial) or continued from the accumulator (the running
// state carried across hops).
//
// What is computed (per query row i, allowed keys A_i of the block):
//   s_j = scale * <q_i, k_j>, m = max s_j, l = sum exp(s_j - m),
//   O = sum exp(s_j - m) v_j / l       (empty A_i: O = 0, m = -inf, l = 0)
// and, when continuing, the same quantities over the union of the keys of
// all blocks seen so far.  Source: aiunderstanding.org guide
// "Sequenzparallelität und Ringaufmerksamkeit", section "Tiefer Einblick"
// (each arriving block's partial attention is accumulated with online
// softmax) and its Thai version, technical-insight section (running maximum,
// running normaliser, earlier partial sums rescaled when a larger maximum
// appears).  Causal rule (key allowed iff its token is not after the query's
// token, diagonal included): highthink.cn Ring Attention article, section
// "Zig Zag Ring Attention 通信和计算重叠".
//
// Design (16-bit inputs):
//  * Transposed products so every lane owns one query:  S^T = K Q^T and
//    O^T += V^T P^T with v_mfma_f32_32x32x16_{bf16,f16}.  In the 32x32
//    accumulator lane l holds query column l%32 and 16 key rows, so the row
//    max / row sum are in-lane reductions plus one v_permlane32_swap.
//  * The S^T accumulator registers, packed to 16 bits, are directly the B
//    operand of the PV product (key order inside a 16-key step is permuted
//    the same way on both operands; the sum over keys does not care).
//  * K and V tiles sit row-major in LDS (16-byte chunks XOR-swizzled by row,
//    conflict-free for both read patterns).  K fragments are ds_read_b128;
//    V^T fragments come from ds_read_b64_tr_b16 (LDS transpose read), so no
//    transposed copy of V is ever written.
//  * 4 waves x 64 queries (two 32-query blocks per wave share every K and V
//    fragment read from LDS), 64-key tiles, LDS double-buffered, one barrier
//    per tile.
//  * Softmax in the exp2 domain with scale*log2(e) folded into one FMA; the
//    running max is only raised when a tile beats it by more than 8 (log2
//    units), so O is rarely rescaled; exact max tracked separately for the
//    outputs.  l is summed in fp32 from the unrounded probabilities.
//  * Causal work: per workgroup and per wave the allowed keys are a prefix of
//    the block (ids are increasing in both layouts); tiles past the prefix
//    are never loaded or computed, fully allowed tiles skip the mask.
//  * Grid order: heaviest causal query tiles first; workgroups sharing a K/V
//    head are placed on the same XCD (dispatch is round-robin over 8 XCDs)
//    so their K/V tiles hit that XCD's L2.
// fp32 inputs use a simpler v_mfma_f32_32x32x2_f32 kernel with the same
// accumulator layout and softmax code.
#include <cfloat>
#include <cmath>

#include "attn_common.h"

namespace ra {
namespace {

using namespace attn;

// ---------------------------------------------------------------------------
// 16-bit kernel
constexpr int kWaves = 4;
constexpr int kQB = 2;                      // 32-query blocks per wave
constexpr int kBM = kWaves * kQB * 32;      // 256 query rows per workgroup
constexpr int kBN = 64;                     // keys per tile
constexpr int kNKH = kBN / 32;              // 32-key halves per tile

template <int D, bool BF16>
__global__ void __launch_bounds__(256) attn_block16_kernel(BatchParams p, int ntq) {
  using M = Mfma16<BF16>;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CH = kBN * CPR / 256;        // chunks per thread per tensor
  constexpr int KS = D / 16;                 // k-steps of the QK product
  constexpr int DT = D / 32;                 // 32-wide d tiles of O
  constexpr int TILE = kBN * D;              // elements per K (or V) tile
  extern __shared__ __attribute__((aligned(16))) short lds[];  // [2 buf][K, V][TILE]

  const Work w = decode(p, ntq);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;

  const short *qp = (const short *)p.q + w.z * p.q_zstride + w.b * p.qs_b + w.h * p.qs_h;
  const int kvi = (p.kv_idx0 + w.z) % p.kv_idx_mod;
  const short *kp = (const short *)p.k + kvi * p.kv_zstride + w.b * p.ks_b + w.kvh * p.ks_h;
  const short *vp = (const short *)p.v + kvi * p.kv_vzstride + w.b * p.vs_b + w.kvh * p.vs_h;
  const IdMap qid = query_ids(p, w.z), kid = key_ids(p, w.z);
  const float c = p.scale * kLog2e;

  const int i_wg0 = w.qtile * kBM;
  const int i_wg1 = min(p.nq, i_wg0 + kBM) - 1;
  const int iw0 = i_wg0 + wave * (kQB * 32);
  const int iw1 = min(p.nq - 1, iw0 + kQB * 32 - 1);
  const bool wave_rows = iw0 < p.nq;

  const int kv_wg = key_prefix(p, kid, qid(i_wg1));
  const int ntiles = (kv_wg + kBN - 1) / kBN;
  const int kv_wl = wave_rows ? key_prefix(p, kid, qid(iw1)) : 0;
  const int kv_wf = wave_rows ? key_prefix(p, kid, qid(iw0)) : 0;
  const int ntiles_w = (kv_wl + kBN - 1) / kBN;
  const int nfull_w = kv_wf / kBN;

  if (ntiles == 0 && p.accumulate) return;  // nothing to add to the running state

  // per-lane row bookkeeping
  int row[kQB], jlim[kQB];
  bool valid[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    row[qb] = iw0 + qb * 32 + c32;
    valid[qb] = row[qb] < p.nq;
    jlim[qb] = key_prefix(p, kid, qid(row[qb]));
  }

  f32x16 O[kQB][DT];
  float m_run[kQB], m_top[kQB], lsum[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    if (p.accumulate) {
      load_state<D>(p, w, row[qb], valid[qb], c, O[qb], m_run[qb], m_top[qb], lsum[qb]);
    } else {
      m_run[qb] = -FLT_MAX;
      m_top[qb] = -FLT_MAX;
      lsum[qb] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[qb][dt][r] = 0.f;
    }
  }

  if (ntiles > 0) {
    // Q fragments (B operand of S^T = K Q^T): lane holds d = 16ks + 8hl .. +7 of its row
    s16x8 qf[kQB][KS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const short *qrow = qp + (int64_t)(valid[qb] ? row[qb] : 0) * p.qs_t;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s16x8 v = *(const s16x8 *)(qrow + 16 * ks + 8 * hl);
        if (!valid[qb]) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
        qf[qb][ks] = v;
      }
    }

    uint4 stk[CH], stv[CH];
    auto gload = [&](int t) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int cid = threadIdx.x + 256 * u;
        const int r = cid / CPR, ch = cid % CPR;
        int j = t * kBN + r;
        j = j < p.nk ? j : p.nk - 1;
        stk[u] = *(const uint4 *)(kp + (int64_t)j * p.ks_t + ch * 8);
        stv[u] = *(const uint4 *)(vp + (int64_t)j * p.vs_t + ch * 8);
      }
    };
    auto lstore = [&](int buf) {
      short *lk = lds + buf * 2 * TILE;
      short *lv = lk + TILE;
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int cid = threadIdx.x + 256 * u;
        const int r = cid / CPR, ch = cid % CPR;
        const int off = r * D + ((ch ^ swz(r)) << 3);
        *(uint4 *)(lk + off) = stk[u];
        *(uint4 *)(lv + off) = stv[u];
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const int cur = t & 1;
      if (t + 1 < ntiles) gload(t + 1);
      if (t < ntiles_w) {
        const short *lk = lds + cur * 2 * TILE;
        const short *lv = lk + TILE;
        f32x16 S[kQB][kNKH];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
          for (int kh = 0; kh < kNKH; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) S[qb][kh][r] = 0.f;
        // S^T = K Q^T : each K fragment feeds both query blocks
#pragma unroll
        for (int kh = 0; kh < kNKH; ++kh) {
          const int r = kh * 32 + c32;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const s16x8 a = *(const s16x8 *)(lk + r * D + (((2 * ks + hl) ^ swz(r)) << 3));
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) S[qb][kh] = M::mma(a, qf[qb][ks], S[qb][kh]);
          }
        }
        // causal / ragged mask only where some key of the tile is not allowed
        if (t >= nfull_w) {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int kh = 0; kh < kNKH; ++kh)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int j = t * kBN + kh * 32 + (r >> 2) * 8 + 4 * hl + (r & 3);
                if (j >= jlim[qb]) S[qb][kh][r] = -INFINITY;
              }
        }
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          softmax_tile<D, kNKH>(S[qb], O[qb], c, m_run[qb], m_top[qb], lsum[qb]);
        // O^T += V^T P^T : V^T fragments by LDS transpose reads
        const int G = lane >> 4, i16 = lane & 15;
#pragma unroll
        for (int kh = 0; kh < kNKH; ++kh)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            s16x8 P[kQB];
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) P[qb] = M::pack(S[qb][kh], 8 * cc);
            const int vr = kh * 32 + 16 * cc + 4 * hl + (i16 >> 2);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const int vc = 32 * dt + 16 * (G & 1) + 4 * (i16 & 3);
              const short *a0 = lv + vr * D + (((vc >> 3) ^ swz(vr)) << 3) + (vc & 7);
              const short *a1 = lv + (vr + 8) * D + (((vc >> 3) ^ swz(vr + 8)) << 3) + (vc & 7);
              const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)a0);
              const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)a1);
              const s16x8 a = (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
              for (int qb = 0; qb < kQB; ++qb) O[qb][dt] = M::mma(a, P[qb], O[qb][dt]);
            }
          }
      }
      if (t + 1 < ntiles) lstore(cur ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
    store_state<D>(p, w, row[qb], valid[qb], O[qb], m_run[qb], m_top[qb], lsum[qb]);
}

// ---------------------------------------------------------------------------
// fp32 kernel: 4 waves x 32 queries, 32-key tiles, v_mfma_f32_32x32x2_f32.
constexpr int kBM32 = 128;
constexpr int kBN32 = 32;

template <int D>
__global__ void __launch_bounds__(256) attn_block32_kernel(BatchParams p, int ntq) {
  constexpr int LD = D + 1;  // padded LDS row (floats)
  constexpr int DT = D / 32;
  __shared__ float lk[kBN32 * LD];
  __shared__ float lv[kBN32 * LD];

  const Work w = decode(p, ntq);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;
  const float *qp = (const float *)p.q + w.z * p.q_zstride + w.b * p.qs_b + w.h * p.qs_h;
  const int kvi = (p.kv_idx0 + w.z) % p.kv_idx_mod;
  const float *kp = (const float *)p.k + kvi * p.kv_zstride + w.b * p.ks_b + w.kvh * p.ks_h;
  const float *vp = (const float *)p.v + kvi * p.kv_vzstride + w.b * p.vs_b + w.kvh * p.vs_h;
  const IdMap qid = query_ids(p, w.z), kid = key_ids(p, w.z);
  const float c = p.scale * kLog2e;

  const int i_wg0 = w.qtile * kBM32;
  const int i_wg1 = min(p.nq, i_wg0 + kBM32) - 1;
  const int kv_wg = key_prefix(p, kid, qid(i_wg1));
  const int ntiles = (kv_wg + kBN32 - 1) / kBN32;
  if (ntiles == 0 && p.accumulate) return;

  const int i = i_wg0 + wave * 32 + c32;
  const bool valid = i < p.nq;
  const int jl = key_prefix(p, kid, qid(i));

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

  float qf[D / 2];
  {
    const float *qrow = qp + (int64_t)(valid ? i : 0) * p.qs_t;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = valid ? qrow[2 * ks + hl] : 0.f;
  }

  for (int t = 0; t < ntiles; ++t) {
    for (int e = threadIdx.x; e < kBN32 * D; e += 256) {
      const int r = e / D, col = e % D;
      int j = t * kBN32 + r;
      j = j < p.nk ? j : p.nk - 1;
      lk[r * LD + col] = kp[(int64_t)j * p.ks_t + col];
      lv[r * LD + col] = vp[(int64_t)j * p.vs_t + col];
    }
    __syncthreads();
    f32x16 S[1];
#pragma unroll
    for (int r = 0; r < 16; ++r) S[0][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
      S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(lk[c32 * LD + 2 * ks + hl], qf[ks], S[0], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = t * kBN32 + (r >> 2) * 8 + 4 * hl + (r & 3);
      if (j >= jl) S[0][r] = -INFINITY;
    }
    softmax_tile<D, 1>(S, O, c, m_run, m_top, lsum);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + 4 * hl + (r & 3);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(lv[key * LD + 32 * dt + c32], S[0][r], O[dt],
                                                    0, 0, 0);
      }
    __syncthreads();
  }
  store_state<D>(p, w, i, valid, O, m_run, m_top, lsum);
}

template <int D, bool BF16>
hipError_t launch16(const BatchParams &p, hipStream_t s) {
  const int ntq = (p.nq + kBM - 1) / kBM;
  const int64_t nwg = (int64_t)ntq * p.nz * p.B * p.Hq;
  const size_t lds = (size_t)2 * 2 * kBN * D * sizeof(short);
  hipLaunchKernelGGL((attn_block16_kernel<D, BF16>), dim3((unsigned)nwg), dim3(256), lds, s, p,
                     ntq);
  return hipGetLastError();
}

template <int D>
hipError_t launch32(const BatchParams &p, hipStream_t s) {
  const int ntq = (p.nq + kBM32 - 1) / kBM32;
  const int64_t nwg = (int64_t)ntq * p.nz * p.B * p.Hq;
  hipLaunchKernelGGL((attn_block32_kernel<D>), dim3((unsigned)nwg), dim3(256), 0, s, p, ntq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_fwd(const BatchParams &p, int dtype, hipStream_t s) {
  if ((int64_t)p.nq * p.nz * p.B * p.Hq == 0) return hipSuccess;
  if (p.v_packed) return launch_block_fwd_packed(p, dtype, s);
  if (dtype == RA_DT_BF16) return p.d == 64 ? launch16<64, true>(p, s) : launch16<128, true>(p, s);
  if (dtype == RA_DT_FP16)
    return p.d == 64 ? launch16<64, false>(p, s) : launch16<128, false>(p, s);
  return p.d == 64 ? launch32<64>(p, s) : launch32<128>(p, s);
}

}  // namespace ra
