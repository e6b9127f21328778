// attn_common.h -- device-side pieces shared by the block-attention kernels:
// MFMA wrappers, cross-half reductions, the workgroup -> work decode, the
// per-row running-state load/store and the online-softmax tile update.
//
// Online softmax (running maximum, running normaliser, earlier partial sums
// rescaled when a larger maximum appears): Thai Ring Attention guide,
// technical-insight section; aiunderstanding.org "Sequenzparallelität und
// Ringaufmerksamkeit", "Tiefer Einblick".  Causal rule (key allowed iff its
// token is not after the query's token): highthink.cn Ring Attention
// article, section "Zig Zag Ring Attention 通信和计算重叠".
#pragma once

#include <cfloat>
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // lazy rescale threshold (log2 units)
// A lane's sum of one tile's probabilities above this means some probability
// may exceed 2^kTau: the running maximum must be raised first.
constexpr float kSumLimit = 256.0f;

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

// Global token id of a local index: affine (contiguous and interleaved
// layouts: b0 + j*step), or two affine chunks of c tokens (zig-zag: b0 + j,
// then b1 + j - c).  Ids increase with j in every layout.
struct IdMap {
  int64_t b0, step, b1;
  int32_t c;  // 0: affine
  __device__ __forceinline__ int64_t operator()(int64_t j) const {
    return (c == 0 || j < c) ? b0 + j * step : b1 + (j - c);
  }
};

__device__ __forceinline__ IdMap zz_map(int64_t rank, const BatchParams &p) {
  IdMap m;
  m.b0 = rank * p.zz_c;
  m.step = 1;
  m.b1 = (2 * (int64_t)p.zz_R - 1 - rank) * p.zz_c;
  m.c = p.zz_c;
  return m;
}

// ids of the queries / keys of problem z of a batch
__device__ __forceinline__ IdMap query_ids(const BatchParams &p, int z) {
  if (p.zz_c) return zz_map(p.q_rank0 + z, p);
  IdMap m;
  m.b0 = p.qg_add + z * p.qg_z;
  m.step = p.q_step;
  m.b1 = 0;
  m.c = 0;
  return m;
}
__device__ __forceinline__ IdMap key_ids(const BatchParams &p, int z) {
  const int64_t src = (p.kg_s0 + z) % p.kg_smod;
  if (p.zz_c) return zz_map(src, p);
  IdMap m;
  m.b0 = p.kg_add + src * p.kg_mult;
  m.step = p.k_step;
  m.b1 = 0;
  m.c = 0;
  return m;
}

// Number of keys of the block allowed for a query with global id gq: the
// allowed keys are always a prefix because key ids increase with j.
__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}
__device__ __forceinline__ int key_prefix(const BatchParams &p, const IdMap &k, int64_t gq) {
  if (!p.causal) return p.nk;
  if (k.c) {  // ids <= gq in each chunk: the chunks are runs of consecutive ids
    const int64_t a = clamp64(gq - k.b0 + 1, 0, k.c);
    const int64_t b = clamp64(gq - k.b1 + 1, 0, (int64_t)p.nk - k.c);
    return (int)(a + b);
  }
  if (gq < k.b0) return 0;
  int64_t c = (gq - k.b0) / k.step + 1;
  return c < p.nk ? (int)c : p.nk;
}

struct Work {
  int z, b, h, kvh, qtile;
};

// Workgroup index -> (problem, batch, head, query tile).  When the number of
// K/V groups is a multiple of 8, all query tiles of one K/V group land on the
// same XCD (workgroups are dispatched round-robin over the 8 XCDs), and each
// XCD works through its groups one after another, each group's heaviest
// causal query tiles first: the workgroups running together on an XCD then
// read the same K/V tiles at about the same time, from that XCD's L2
// (measured: 4-8 % less time on the 32k MHA, 128k GQA and 512-token-shard
// workloads than when an XCD's concurrent workgroups span all its groups).
// Under the causal mask an XCD takes its groups two at a time, the pair's query
// tiles heaviest first, alternating between the two groups: group after group,
// the heaviest tile of the next group can start when the XCD is almost out of
// work and run on alone (short triangular blocks, such as 16 query tiles of 4 to
// 64 key tiles, lose ~5 % of a launch that way in a greedy schedule of 32 CUs).
// Otherwise heaviest tiles first over all groups.
// hpg: query heads of a K/V group that are work items of their own (1 when a
// workgroup serves all the heads of its group).
__device__ __forceinline__ Work decode_items(const BatchParams &p, int ntq, int hpg) {
  const int NG = p.nz * p.B * p.Hkv;
  const int L = blockIdx.x;
  int trank, g, hh;
  if ((NG & 7) == 0) {
    const int xcd = L & 7, idx = L >> 3;
    const int per_group = ntq * hpg;
    const int G8 = NG >> 3;  // groups per XCD
    int gl;
    const int pl = idx / (2 * per_group);
    if (p.causal && 2 * pl + 1 < G8) {  // groups 2 pl and 2 pl + 1, interleaved
      const int t2 = (idx - pl * 2 * per_group) / hpg;  // 2 trank + which
      hh = idx - pl * 2 * per_group - t2 * hpg;
      trank = t2 >> 1;
      gl = 2 * pl + (t2 & 1);
    } else {  // one group at a time (and the last group when their number is odd)
      gl = idx / per_group;
      const int rem = idx - gl * per_group;
      trank = rem / hpg;
      hh = rem - trank * hpg;
    }
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
  w.h = w.kvh * (p.Hq / p.Hkv) + hh;
  return w;
}
__device__ __forceinline__ Work decode(const BatchParams &p, int ntq) {
  return decode_items(p, ntq, p.Hq / p.Hkv);
}

// Row-state load/store shared by both kernels.  The lane owns query row i and,
// in each 32x32 O^T tile dt, the 16 values d = 32dt + 8(r/4) + 4*half + r%4.
// The load has no branch, so m, l and O are requested together (and a kernel
// can issue its first tile loads before them); a row that has seen no key yet
// (l = 0) starts from O = 0 whatever its stored O holds.
template <int D>
__device__ __forceinline__ void load_state(const BatchParams &p, const Work &w, int i, bool valid,
                                           float c, f32x16 (&O)[D / 32], float &m_run,
                                           float &m_top, float &lsum) {
  const int hl = (threadIdx.x >> 5) & 1;
  // Lanes past the end of the block read row 0 (every block that has work
  // has one) and drop what they read.
  const int ii = valid ? i : 0;
  const int64_t mi = w.z * p.ml_zstride + ((int64_t)w.b * p.Hq + w.h) * p.nq + ii;
  const float m_ld = p.m[mi];
  const float l_ld = p.l[mi];
  const float *orow = p.o + w.z * p.o_zstride + w.b * p.os_b + w.h * p.os_h + (int64_t)ii * p.os_t;
  float4 v[D / 32][4];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) v[dt][rg] = *(const float4 *)(orow + 32 * dt + 8 * rg + 4 * hl);
  const float m_acc = valid ? m_ld : -INFINITY;
  const float l_acc = valid ? l_ld : 0.f;
  const bool seen = l_acc > 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      O[dt][4 * rg + 0] = seen ? v[dt][rg].x * l_acc : 0.f;
      O[dt][4 * rg + 1] = seen ? v[dt][rg].y * l_acc : 0.f;
      O[dt][4 * rg + 2] = seen ? v[dt][rg].z * l_acc : 0.f;
      O[dt][4 * rg + 3] = seen ? v[dt][rg].w * l_acc : 0.f;
    }
  m_run = seen ? m_acc * kLog2e : -FLT_MAX;
  m_top = m_run;
  lsum = (seen && hl == 0) ? l_acc : 0.f;
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


}  // namespace attn
}  // namespace ra
