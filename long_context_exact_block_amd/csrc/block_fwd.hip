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

#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // lazy rescale threshold (log2 units)

template <bool BF16>
struct Mfma16;

template <>
struct Mfma16<true> {
  static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ s16x8 pack(const f32x16 &p, int base) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)p[base + e];
    return __builtin_bit_cast(s16x8, r);
  }
};

template <>
struct Mfma16<false> {
  static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ s16x8 pack(const f32x16 &p, int base) {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)p[base + e];
    return __builtin_bit_cast(s16x8, r);
  }
};

// Lane l and lane l^32 hold two halves of the same query's keys.  After
// v_permlane32_swap(x, x) the two results hold {x[l], x[l^32]} in some order
// on every lane, so symmetric reductions need no lane select.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// Number of keys of the block allowed for a query with global id gq: the
// allowed keys are always a prefix because key ids increase with j.
__device__ __forceinline__ int key_prefix(const BatchParams &p, int64_t kg0, int64_t gq) {
  if (!p.causal) return p.nk;
  if (gq < kg0) return 0;
  int64_t c = (gq - kg0) / p.k_step + 1;
  return c < p.nk ? (int)c : p.nk;
}

struct Work {
  int z, b, h, kvh, qtile;
};

// Workgroup index -> (problem, batch, head, query tile).  Heaviest causal
// tiles first; when the number of K/V groups is a multiple of 8, all query
// tiles of one K/V group land on the same XCD.
__device__ __forceinline__ Work decode(const BatchParams &p, int ntq) {
  const int hpg = p.Hq / p.Hkv;
  const int NG = p.nz * p.B * p.Hkv;
  const int L = blockIdx.x;
  int trank, g, hh;
  if ((NG & 7) == 0) {
    const int xcd = L & 7, idx = L >> 3;
    const int per_xcd = (NG >> 3) * hpg;
    trank = idx / per_xcd;
    const int rem = idx - trank * per_xcd;
    const int gl = rem / hpg;
    hh = rem - gl * hpg;
    g = gl * 8 + xcd;
  } else {
    const int per_t = NG * hpg;
    trank = L / per_t;
    const int rem = L - trank * per_t;
    g = rem / hpg;
    hh = rem - g * hpg;
  }
  Work w;
  w.qtile = p.causal ? (ntq - 1 - trank) : trank;
  w.kvh = g % p.Hkv;
  const int zb = g / p.Hkv;
  w.b = zb % p.B;
  w.z = zb / p.B;
  w.h = w.kvh * hpg + hh;
  return w;
}

// Row-state load/store shared by both kernels.  The lane owns query row i and,
// in each 32x32 O^T tile dt, the 16 values d = 32dt + 8(r/4) + 4*half + r%4.
template <int D>
__device__ __forceinline__ void load_state(const BatchParams &p, const Work &w, int i, bool valid,
                                           float c, f32x16 (&O)[D / 32], float &m_run,
                                           float &m_top, float &lsum) {
  const int hl = (threadIdx.x >> 5) & 1;
  float m_acc = -INFINITY, l_acc = 0.f;
  if (valid) {
    const int64_t mi = w.z * p.ml_zstride + ((int64_t)w.b * p.Hq + w.h) * p.nq + i;
    m_acc = p.m[mi];
    l_acc = p.l[mi];
  }
  if (l_acc > 0.f) {
    m_run = m_acc * kLog2e;
    m_top = m_run;
    lsum = hl ? 0.f : l_acc;
    const float *orow = p.o + w.z * p.o_zstride + w.b * p.os_b + w.h * p.os_h + (int64_t)i * p.os_t;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 v = *(const float4 *)(orow + 32 * dt + 8 * rg + 4 * hl);
        O[dt][4 * rg + 0] = v.x * l_acc;
        O[dt][4 * rg + 1] = v.y * l_acc;
        O[dt][4 * rg + 2] = v.z * l_acc;
        O[dt][4 * rg + 3] = v.w * l_acc;
      }
  } else {
    m_run = -FLT_MAX;
    m_top = -FLT_MAX;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  }
  (void)c;
}

template <int D>
__device__ __forceinline__ void store_state(const BatchParams &p, const Work &w, int i, bool valid,
                                            const f32x16 (&O)[D / 32], float m_run, float m_top,
                                            float lsum) {
  const int hl = (threadIdx.x >> 5) & 1;
  const float lt = half_sum(lsum);
  if (!valid) return;
  float *orow = p.o + w.z * p.o_zstride + w.b * p.os_b + w.h * p.os_h + (int64_t)i * p.os_t;
  float mo, lo, inv;
  if (lt > 0.f) {
    inv = 1.f / lt;
    mo = m_top * kLn2;
    lo = lt * __builtin_amdgcn_exp2f(m_run - m_top);
  } else {
    inv = 0.f;
    mo = -INFINITY;
    lo = 0.f;
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      float4 v;
      v.x = O[dt][4 * rg + 0] * inv;
      v.y = O[dt][4 * rg + 1] * inv;
      v.z = O[dt][4 * rg + 2] * inv;
      v.w = O[dt][4 * rg + 3] * inv;
      *(float4 *)(orow + 32 * dt + 8 * rg + 4 * hl) = v;
    }
  if (hl == 0) {
    const int64_t mi = w.z * p.ml_zstride + ((int64_t)w.b * p.Hq + w.h) * p.nq + i;
    p.m[mi] = mo;
    p.l[mi] = lo;
  }
}

// Online-softmax update of one query block for one tile of 32*NKH keys held
// in S[kh] (masked entries already -inf).  Returns probabilities in S.
template <int D, int NKH>
__device__ __forceinline__ void softmax_tile(f32x16 (&S)[NKH], f32x16 (&O)[D / 32], float c,
                                             float &m_run, float &m_top, float &lsum) {
  float mx = -INFINITY;
#pragma unroll
  for (int kh = 0; kh < NKH; ++kh)
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
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[dt][r] *= al;
    m_run = mn;
  }
  const float nm = -m_run;
  float ls = 0.f;
#pragma unroll
  for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(S[kh][r], c, nm));
      ls += pv;
      S[kh][r] = pv;
    }
  lsum += ls;
}

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
  const short *vp = (const short *)p.v + kvi * p.kv_zstride + w.b * p.vs_b + w.kvh * p.vs_h;
  const int64_t qg0 = p.qg_add + w.z * p.qg_z;
  const int64_t kg0 = p.kg_add + (int64_t)((p.kg_s0 + w.z) % p.kg_smod) * p.kg_mult;
  const float c = p.scale * kLog2e;

  const int i_wg0 = w.qtile * kBM;
  const int i_wg1 = min(p.nq, i_wg0 + kBM) - 1;
  const int iw0 = i_wg0 + wave * (kQB * 32);
  const int iw1 = min(p.nq - 1, iw0 + kQB * 32 - 1);
  const bool wave_rows = iw0 < p.nq;

  const int kv_wg = key_prefix(p, kg0, qg0 + (int64_t)i_wg1 * p.q_step);
  const int ntiles = (kv_wg + kBN - 1) / kBN;
  const int kv_wl = wave_rows ? key_prefix(p, kg0, qg0 + (int64_t)iw1 * p.q_step) : 0;
  const int kv_wf = wave_rows ? key_prefix(p, kg0, qg0 + (int64_t)iw0 * p.q_step) : 0;
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
    jlim[qb] = key_prefix(p, kg0, qg0 + (int64_t)row[qb] * p.q_step);
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
  const float *vp = (const float *)p.v + kvi * p.kv_zstride + w.b * p.vs_b + w.kvh * p.vs_h;
  const int64_t qg0 = p.qg_add + w.z * p.qg_z;
  const int64_t kg0 = p.kg_add + (int64_t)((p.kg_s0 + w.z) % p.kg_smod) * p.kg_mult;
  const float c = p.scale * kLog2e;

  const int i_wg0 = w.qtile * kBM32;
  const int i_wg1 = min(p.nq, i_wg0 + kBM32) - 1;
  const int kv_wg = key_prefix(p, kg0, qg0 + (int64_t)i_wg1 * p.q_step);
  const int ntiles = (kv_wg + kBN32 - 1) / kBN32;
  if (ntiles == 0 && p.accumulate) return;

  const int i = i_wg0 + wave * 32 + c32;
  const bool valid = i < p.nq;
  const int jl = key_prefix(p, kg0, qg0 + (int64_t)i * p.q_step);

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
  if (dtype == RA_DT_BF16) return p.d == 64 ? launch16<64, true>(p, s) : launch16<128, true>(p, s);
  if (dtype == RA_DT_FP16)
    return p.d == 64 ? launch16<64, false>(p, s) : launch16<128, false>(p, s);
  return p.d == 64 ? launch32<64>(p, s) : launch32<128>(p, s);
}

}  // namespace ra
