// decode.hip -- a few new query tokens against a KV cache split over R ranks.
//
// Each rank holds a contiguous run of the cache and computes the partial
// attention of the new queries against its run; the partials are folded by
// the online-softmax combine (running maximum, running normaliser, rescaled
// sums: Thai Ring Attention guide, technical-insight section;
// aiunderstanding.org "Sequenzparallelität und Ringaufmerksamkeit",
// "Häufig gestellte Fragen").  Serving long contexts this way is the
// inference use the German guide's "Reale Umsetzung" section and the
// sequence-parallel inference article describe.
//
// gfx950 design: decode is bound by reading the cache from HBM, and all query
// rows that share a K/V head (head-in-group x new token, up to 32 per column
// block) fit one 32-wide MFMA operand, so every key is read once per column
// block and no two waves need the same key: each wave streams its own key
// range through a private two-stage LDS ring, 64 keys per stage (the K rows
// and the packed V^T tile of 64 keys are each one contiguous block).  The
// stages are filled by non-temporal buffer loads that write LDS directly:
// every 1 KB load covers whole cache lines and streams past the caches, which
// on MI355X reads ~7.0 TB/s against ~5.9-6.2 TB/s for cached loads.  A wave
// waits only on its own loads (vmcnt), so the loop has no barrier.  The MFMA
// operands are 16-byte LDS reads with the forward kernel's swizzles.  At the
// end the waves of a workgroup fold their partials in LDS into one (O
// normalised, m, l); decode_reduce folds the partials of all workgroups of a
// row.
#include <cfloat>
#include <cmath>

#include <mutex>

#include "attn_common.h"

namespace ra {
namespace {

using namespace attn;

constexpr int kDW = kDecodeWaves;
constexpr int kMaxP = 4096;   // partials per row the reduction holds in LDS

// LDS row stride (floats) of the per-wave partials: +4 keeps the float4
// writes of the 32 columns on distinct bank groups
template <int D>
constexpr int sorow() { return D + 4; }
constexpr int kDT = 64;  // keys per tile (one packed V^T tile)
template <int D>
constexpr int dec_stage_bytes() { return 2 * kDT * D * 2; }  // K rows + V^T tile
template <int D>
constexpr size_t decode_lds_bytes() {
  const size_t fold = (size_t)kDW * 32 * sorow<D>() * 4 + 2 * kDW * 32 * 4;
  const size_t ring = (size_t)kDW * 2 * dec_stage_bytes<D>();
  return fold > ring ? fold : ring;
}
// LDS has 64 four-byte banks on gfx950: 16-byte chunks of a row are
// XOR-swizzled by row so the 16-byte operand reads of a 16-lane group hit 16
// distinct bank groups (256-byte rows: by row & 15; 128-byte rows, which
// alternate between the two halves of the banks: by (row >> 1) & 7).
template <int ROW_BYTES>
__device__ __forceinline__ int dswz(int row) {
  return ROW_BYTES == 256 ? (row & 15) : ((row >> 1) & 7);
}
typedef __attribute__((address_space(3))) void lds_void;
// 16 bytes per lane, non-temporal, from a raw buffer straight into LDS (lane
// l lands at dst + 16 l; dst goes to M0).  Cache policy 2 = nt.
__device__ __forceinline__ void dma16nt(__amdgpu_buffer_rsrc_t rsrc, lds_void *dst, uint32_t voff,
                                        uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, soff, 0, 2);
}
// s_waitcnt immediate waiting for vmcnt <= n only (n < 64; lgkmcnt, expcnt at max)
constexpr int dwait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

template <int D, bool BF16>
__global__ void __launch_bounds__(kDW * 64) decode_kernel(DecodeParams p) {
  using M = Mfma16<BF16>;
  constexpr int KS = D / 16;  // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;  // 32-row d tiles of O^T
  extern __shared__ __attribute__((aligned(1024))) float smem[];
  float *sO = smem;                                // [kDW][32][sorow]
  float *sM = smem + kDW * 32 * sorow<D>();        // [kDW][32] running max (log2 units)
  float *sL = sM + kDW * 32;                       // [kDW][32] sum
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5, c32 = lane & 31;

  // workgroup -> (rank r, batch b, kv head, key split); grid.y = column block
  int g = blockIdx.x;
  const int split = g % p.splits;
  g /= p.splits;
  const int kvh = g % p.Hkv;
  g /= p.Hkv;
  const int b = g % p.B;
  const int r = g / p.B;
  const int G = p.Hq / p.Hkv;
  const int ncols = G * p.nq;
  const int rows = p.B * p.Hq * p.nq;

  // this lane's column: query head kvh*G + col/nq, new token col%nq
  const int col = blockIdx.y * 32 + c32;
  const bool valid = col < ncols;
  const int hh = valid ? col / p.nq : 0;
  const int qi = valid ? col % p.nq : 0;
  const int h = kvh * G + hh;

  // keys of this wave: [j0, j1) of rank r's run
  const int j0 = (split * kDW + wave) * p.wave_keys;
  const int j1 = min(p.n, j0 + p.wave_keys);
  // key j of rank r is token r*n + j; it is allowed for query token qg iff
  // r*n + j <= qg, so the allowed keys form the prefix [0, jlim)
  int jlim = 0;
  if (valid) {
    if (!p.causal) {
      jlim = p.n;
    } else {
      const int64_t lim = p.q_gid0 + qi - (int64_t)r * p.n + 1;
      jlim = lim < 0 ? 0 : (lim > p.n ? p.n : (int)lim);
    }
  }
  // the wave's loop ends at the largest limit of its columns
  int jmax = jlim;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) jmax = max(jmax, __shfl_xor(jmax, o));
  const int jend = min(j1, jmax);

  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[dt][e] = 0.f;
  float m_run = -FLT_MAX, lsum = 0.f;

  if (j0 < jend) {
    const float c = p.scale * kLog2e;
    // Q^T fragments (B operand): d = 16ks + 8hl .. +7 of this lane's column
    s16x8 qf[KS];
    {
      const short *qrow = (const short *)p.q + ((int64_t)(b * p.Hq + h) * p.nq + qi) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s16x8 v = *(const s16x8 *)(qrow + 16 * ks + 8 * hl);
        if (!valid) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
        qf[ks] = v;
      }
    }
    const int64_t bh = ((int64_t)r * p.B + b) * p.Hkv + kvh;
    const short *kp = (const short *)p.k + bh * p.n * D;
    const short *vp = (const short *)p.v + bh * D * p.n_pad;
    // byte counts fit 32 bits: n <= 2^23 keys (checked on the host)
    const auto krsrc = __builtin_amdgcn_make_buffer_rsrc((void *)kp, 0, (int)((uint32_t)p.n * D * 2),
                                                         0x00020000);
    const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)vp, 0, (int)((uint32_t)D * (uint32_t)p.n_pad * 2), 0x00020000);
    constexpr int KROW = D * 2, KTB = kDT * KROW;   // K row / tile bytes
    constexpr int VROW = kDT * 2, VTB = D * VROW;   // packed V^T row / tile bytes
    constexpr int NK = KTB / 1024, NV = VTB / 1024;  // 1 KB loads per tile
    constexpr int SB = dec_stage_bytes<D>();
    char *ring = (char *)smem + wave * 2 * SB;      // this wave's two stages
    // load tile jt (a multiple of 64) into stage st: 1 KB u of the K tile is
    // rows u*RPI.., lane l its chunk l % CPR, fetched from the swizzled source
    auto issue = [&](int jt, int st) {
      char *dst = ring + st * SB;
#pragma unroll
      for (int u = 0; u < NK; ++u) {
        constexpr int CPR = KROW / 16, RPI = 1024 / KROW;
        const int row = u * RPI + lane / CPR;
        const int ch = (lane % CPR) ^ dswz<KROW>(row);
        dma16nt(krsrc, (lds_void *)(dst + u * 1024), row * KROW + ch * 16, (uint32_t)jt * KROW);
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        constexpr int CPR = VROW / 16, RPI = 1024 / VROW;
        const int row = u * RPI + lane / CPR;
        const int ch = (lane % CPR) ^ dswz<VROW>(row);
        dma16nt(vrsrc, (lds_void *)(dst + KTB + u * 1024), row * VROW + ch * 16,
                (uint32_t)(jt / kDT) * VTB);
      }
    };
    // per-lane operand offsets: K row kb*32 + c32 and V^T row 32dt + c32
    // share the swizzle of row c32
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = c32 * KROW + (((2 * ks + hl) ^ dswz<KROW>(c32)) << 4);
    int voff[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) voff[q4] = KTB + c32 * VROW + (((2 * q4 + hl) ^ dswz<VROW>(c32)) << 4);

    auto compute = [&](const char *stg, int jt) {
      f32x16 S[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          S[kb] = M::mma(*(const s16x8 *)(stg + koff[ks] + kb * 32 * KROW), qf[ks], S[kb]);
      // element e of S^T[kb] is key jt + 32kb + 8(e/4) + 4hl + e%4 of this lane's column
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = jt + 32 * kb + (e >> 2) * 8 + 4 * hl + (e & 3);
          if (j >= jlim) S[kb][e] = -INFINITY;
          mx = fmaxf(mx, S[kb][e]);
        }
      mx = half_max(mx);
      const float mt = mx * c;
      if (wave_any(mt > m_run + kTau)) {
        const float mn = fmaxf(m_run, mt);
        const float al = __builtin_amdgcn_exp2f(m_run - mn);
        lsum *= al;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) O[dt][e] *= al;
        m_run = mn;
      }
      const float nm = -m_run;
      // P^T (B operand), 16 keys per MFMA in the packed order: group q4 is
      // registers 8(q4 % 2) .. +7 of S^T[q4 / 2]
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x16 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = __builtin_amdgcn_exp2f(fmaf(S[q4 >> 1][8 * (q4 & 1) + e], c, nm));
          lsum += pb[e];
        }
        const s16x8 P = M::pack(pb, 0);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          O[dt] = M::mma(*(const s16x8 *)(stg + voff[q4] + dt * 32 * VROW), P, O[dt]);
      }
    };
    // tile t + 1 streams into the other stage (last read by tile t - 1, whose
    // operands were consumed before its MFMAs) while tile t is computed
    const int ntile = (jend - j0 + kDT - 1) / kDT;
    issue(j0, 0);
    for (int t = 0; t < ntile; ++t) {
      if (t + 1 < ntile) {
        issue(j0 + (t + 1) * kDT, (t + 1) & 1);
        __builtin_amdgcn_s_waitcnt(dwait_vm(NK + NV));  // tile t has landed
      } else {
        __builtin_amdgcn_s_waitcnt(dwait_vm(0));
      }
      compute(ring + (t & 1) * SB, j0 + t * kDT);
    }
  }

  // the staging ring and the partials below share the LDS
  __syncthreads();
  // Fold the waves' partials in LDS: m = max m_w, weights 2^(m_w - m),
  // O = sum w O_w / sum w l_w.  Then one partial per workgroup.
  const float lt = half_sum(lsum);
  {
    float *orow = sO + (wave * 32 + c32) * sorow<D>();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *(float4 *)(orow + 32 * dt + 8 * rg + 4 * hl) =
            make_float4(O[dt][4 * rg], O[dt][4 * rg + 1], O[dt][4 * rg + 2], O[dt][4 * rg + 3]);
    if (hl == 0) {
      sM[wave * 32 + c32] = m_run;
      sL[wave * 32 + c32] = lt;
    }
  }
  __syncthreads();
  {
    constexpr int TPC = 2 * kDW;   // threads per column: 32 columns over 64*kDW threads
    constexpr int PER = D / TPC;   // outputs per thread
    const int t = threadIdx.x;
    const int cc = t / TPC, d0 = (t % TPC) * PER;
    const int ccol = blockIdx.y * 32 + cc;
    float mw = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < kDW; ++w) mw = fmaxf(mw, sM[w * 32 + cc]);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kDW; ++w) {
      const float lw = sL[w * 32 + cc];
      const float wt = lw > 0.f ? __builtin_amdgcn_exp2f(sM[w * 32 + cc] - mw) : 0.f;
      L += wt * lw;
      const float *src = sO + (w * 32 + cc) * sorow<D>() + d0;
#pragma unroll
      for (int e = 0; e < PER; e += 4) {
        const float4 x = *(const float4 *)(src + e);
        acc[e] += wt * x.x;
        acc[e + 1] += wt * x.y;
        acc[e + 2] += wt * x.z;
        acc[e + 3] += wt * x.w;
      }
    }
    if (ccol < ncols) {
      const int hq = kvh * G + ccol / p.nq;
      const int prow = (b * p.Hq + hq) * p.nq + ccol % p.nq;
      const int pidx = r * p.splits + split;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float *dst = p.po + ((int64_t)pidx * rows + prow) * D + d0;
#pragma unroll
      for (int e = 0; e < PER; e += 4)
        *(float4 *)(dst + e) =
            make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
      if (t % TPC == 0) {
        const int64_t mi = (int64_t)pidx * rows + prow;
        p.pm[mi] = L > 0.f ? mw * kLn2 : -INFINITY;
        p.pl[mi] = L;
      }
    }
  }
}

// Fold the P partials of one output row: m = max m_p, w_p = l_p e^{m_p - m},
// l = sum w_p, O = sum w_p O_p / l; then O in the output dtype and
// LSE = m + ln l ((0, -inf) for a row that saw no key).
template <typename T>
__global__ void __launch_bounds__(256) decode_reduce_kernel(const float *__restrict__ po,
                                                            const float *__restrict__ pm,
                                                            const float *__restrict__ pl, int P,
                                                            int rows, int d, T *__restrict__ out,
                                                            float *__restrict__ lse) {
  __shared__ float w[kMaxP];
  __shared__ float4 red4[256];
  __shared__ float red[256];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  float mx = -INFINITY;
  for (int q = t; q < P; q += 256) {
    const int64_t i = (int64_t)q * rows + row;
    if (pl[i] > 0.f) mx = fmaxf(mx, pm[i]);
  }
  red[t] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float ls = 0.f;
  for (int q = t; q < P; q += 256) {
    const int64_t i = (int64_t)q * rows + row;
    const float wq = pl[i] > 0.f ? pl[i] * expf(pm[i] - M) : 0.f;
    w[q] = wq;
    ls += wq;
  }
  red[t] = ls;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const float L = red[0];
  // float4 columns c4 = t % (d/4), partial slices t / (d/4)
  const int d4 = d / 4, c4 = t % d4, slice = t / d4, nsl = 256 / d4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = slice; q < P; q += nsl) {
    const float4 x = *(const float4 *)(po + ((int64_t)q * rows + row) * d + 4 * c4);
    const float wq = w[q];
    acc.x += wq * x.x;
    acc.y += wq * x.y;
    acc.z += wq * x.z;
    acc.w += wq * x.w;
  }
  red4[t] = acc;
  __syncthreads();
  if (slice == 0) {
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sl = 0; sl < nsl; ++sl) {
      const float4 x = red4[sl * d4 + c4];
      sum.x += x.x;
      sum.y += x.y;
      sum.z += x.z;
      sum.w += x.w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T *o = out + (int64_t)row * d + 4 * c4;
    o[0] = (T)(sum.x * inv);
    o[1] = (T)(sum.y * inv);
    o[2] = (T)(sum.z * inv);
    o[3] = (T)(sum.w * inv);
    if (c4 == 0) lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
  }
}

template <int D, bool BF16>
hipError_t launch_decode_d(const DecodeParams &p, hipStream_t s) {
  constexpr size_t lds = decode_lds_bytes<D>();
  // more than 64 KB of LDS per workgroup must be opted into, once per process
  // (a function-local static: initialised once even with several host threads)
  static const hipError_t attr =
      lds > 65536 ? hipFuncSetAttribute((const void *)decode_kernel<D, BF16>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
                  : hipSuccess;
  if (attr != hipSuccess) return attr;
  dim3 grid((unsigned)(p.R * p.B * p.Hkv * p.splits), (unsigned)p.col_blocks);
  hipLaunchKernelGGL((decode_kernel<D, BF16>), grid, dim3(kDW * 64), lds, s, p);
  return hipGetLastError();
}

}  // namespace

// Partials of the allocation-free decode entry point.  The array's name is a
// host-side stand-in on the host: kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device (each device holds
// its own copy) and kept for the life of the process.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams &p, int dtype, void *o, float *lse, hipStream_t s) {
  const int rows = p.B * p.Hq * p.nq;
  if (rows == 0) return hipSuccess;
  if (p.P > kMaxP) return hipErrorInvalidValue;
  hipError_t e;
  if (dtype == RA_DT_BF16)
    e = p.d == 64 ? launch_decode_d<64, true>(p, s) : launch_decode_d<128, true>(p, s);
  else
    e = p.d == 64 ? launch_decode_d<64, false>(p, s) : launch_decode_d<128, false>(p, s);
  if (e != hipSuccess) return e;
  if (dtype == RA_DT_BF16)
    hipLaunchKernelGGL(decode_reduce_kernel<__bf16>, dim3(rows), dim3(256), 0, s, p.po, p.pm,
                       p.pl, p.P, rows, p.d, (__bf16 *)o, lse);
  else
    hipLaunchKernelGGL(decode_reduce_kernel<_Float16>, dim3(rows), dim3(256), 0, s, p.po, p.pm,
                       p.pl, p.P, rows, p.d, (_Float16 *)o, lse);
  return hipGetLastError();
}

}  // namespace ra
