// elementwise.hip -- the bandwidth-bound kernels of the ring path: the
// online-softmax combine of two partials, the final cast + log-sum-exp, the
// token <-> slot index maps and the row gather/scatter between the original
// token order and rank shards.
//
// Page citations (page title and section):
//  * combine: Thai Ring Attention guide, technical-insight section (running
//    maximum and normaliser; earlier partial sums rescaled when a larger
//    maximum appears) and the German guide "Sequenzparallelität und
//    Ringaufmerksamkeit", FAQ (this makes the blockwise result equal full
//    attention);
//  * index maps: highthink.cn Ring Attention article, section "Zig Zag Ring
//    Attention 通信和计算重叠" (interleaved assignment: rank r holds tokens
//    r, r+R, r+2R, ...) and the German guide, "Tiefer Einblick" (contiguous
//    runs).
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

// One thread per 4 consecutive floats of a row; d/4 threads share a row.
// Reads O_a, O_b (8d bytes), writes O (4d), plus the row's (m, l) pairs.  The
// O rows are touched once: non-temporal loads and stores stream them past the
// caches (plain streaming reads top out ~10 % lower on MI355X).
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) merge_kernel(float *__restrict__ o_acc,
                                                    float *__restrict__ m_acc,
                                                    float *__restrict__ l_acc,
                                                    const float *__restrict__ o_blk,
                                                    const float *__restrict__ m_blk,
                                                    const float *__restrict__ l_blk, int64_t rows,
                                                    int d4, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int64_t row = tid / d4;
  const int q = (int)(tid - row * d4);
  const float ma = m_acc[row], mb = m_blk[row];
  const float la = l_acc[row], lb = l_blk[row];
  const float m = fmaxf(ma, mb);
  float4 r;
  float l;
  if (m == -INFINITY) {  // both partials empty: stay the identity (0, -inf, 0)
    r = make_float4(0.f, 0.f, 0.f, 0.f);
    l = 0.f;
  } else {
    const float wa = (ma == -INFINITY) ? 0.f : la * __expf(ma - m);
    const float wb = (mb == -INFINITY) ? 0.f : lb * __expf(mb - m);
    l = wa + wb;
    const float inv = 1.f / l;
    const float ca = wa * inv, cb = wb * inv;
    const f32x4 a = __builtin_nontemporal_load((const f32x4 *)o_acc + tid);
    const f32x4 b = __builtin_nontemporal_load((const f32x4 *)o_blk + tid);
    r.x = ca * a.x + cb * b.x;
    r.y = ca * a.y + cb * b.y;
    r.z = ca * a.z + cb * b.z;
    r.w = ca * a.w + cb * b.w;
  }
  const f32x4 rv = {r.x, r.y, r.z, r.w};
  __builtin_nontemporal_store(rv, (f32x4 *)o_acc + tid);
  if (q == 0) {
    m_acc[row] = m;
    l_acc[row] = l;
  }
  (void)rows;
}

template <typename T>
__device__ __forceinline__ T cast_out(float x);
template <>
__device__ __forceinline__ __bf16 cast_out<__bf16>(float x) {
  return (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
}
template <>
__device__ __forceinline__ _Float16 cast_out<_Float16>(float x) {
  return (_Float16)x;  // round to nearest even
}
template <>
__device__ __forceinline__ float cast_out<float>(float x) {
  return x;
}

template <typename T>
__global__ void __launch_bounds__(256) finalize_kernel(const float *__restrict__ o_acc,
                                                       const float *__restrict__ m,
                                                       const float *__restrict__ l,
                                                       T *__restrict__ out, float *__restrict__ lse,
                                                       int d4, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int64_t row = tid / d4;
  const int q = (int)(tid - row * d4);
  const float4 a = ((const float4 *)o_acc)[tid];
  T *o = out + tid * 4;
  o[0] = cast_out<T>(a.x);
  o[1] = cast_out<T>(a.y);
  o[2] = cast_out<T>(a.z);
  o[3] = cast_out<T>(a.w);
  if (q == 0) {
    const float lv = l[row];
    lse[row] = lv > 0.f ? m[row] + __logf(lv) : -INFINITY;
  }
}

// The same for d % 8 == 0 and a 16-byte aligned output: one thread per 8
// floats of a row, read with two non-temporal 16-byte loads and written as
// one 16-byte store of 16-bit values (two for fp32 output), all streaming.
template <typename T>
__global__ void __launch_bounds__(256) finalize8_kernel(const float *__restrict__ o_acc,
                                                        const float *__restrict__ m,
                                                        const float *__restrict__ l,
                                                        T *__restrict__ out,
                                                        float *__restrict__ lse, int d8,
                                                        int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int64_t row = tid / d8;
  const int q = (int)(tid - row * d8);
  const f32x4 a = __builtin_nontemporal_load((const f32x4 *)o_acc + 2 * tid);
  const f32x4 b = __builtin_nontemporal_load((const f32x4 *)o_acc + 2 * tid + 1);
  if constexpr (sizeof(T) == 4) {
    __builtin_nontemporal_store(a, (f32x4 *)out + 2 * tid);
    __builtin_nontemporal_store(b, (f32x4 *)out + 2 * tid + 1);
  } else {
    typedef T t8 __attribute__((ext_vector_type(8)));
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    t8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = cast_out<T>(a[e]);
      r[4 + e] = cast_out<T>(b[e]);
    }
    __builtin_nontemporal_store(__builtin_bit_cast(u4, r), (u4 *)out + tid);
  }
  if (q == 0) {
    const float lv = l[row];
    lse[row] = lv > 0.f ? m[row] + __logf(lv) : -INFINITY;
  }
}

__global__ void layout_kernel(int layout, int64_t S, int32_t R, int64_t n, int32_t *fwd,
                              int32_t *inv) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= S) return;
  const int64_t r = p / n, j = p - r * n;
  const int64_t c = n >> 1;  // zig-zag chunk length
  int64_t t;
  if (layout == RA_LAYOUT_CONTIGUOUS)
    t = p;
  else if (layout == RA_LAYOUT_STRIPED)
    t = j * R + r;
  else
    t = j < c ? r * c + j : (2 * (int64_t)R - 1 - r) * c + (j - c);
  fwd[p] = (int32_t)t;
  if (inv) inv[t] = (int32_t)p;
}

// One thread per 16-byte chunk (vector path) or element (scalar path) of a
// shard row.  Shard row (k, b, h, j) <-> token row fwd[(rank0+k)*n + j].
template <typename U>
__global__ void move_kernel(bool gather, const U *__restrict__ src, U *__restrict__ dst,
                            const int32_t *__restrict__ fwd, int64_t BH, int64_t S, int64_t n,
                            int64_t row_units, int32_t rank0, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int64_t u = tid % row_units;
  const int64_t shard_row = tid / row_units;  // ((k*BH) + bh)*n + j
  const int64_t j = shard_row % n;
  const int64_t kbh = shard_row / n;
  const int64_t bh = kbh % BH;
  const int64_t k = kbh / BH;
  const int64_t tok = fwd[(rank0 + k) * n + j];
  const int64_t orig = (bh * S + tok) * row_units + u;
  if (gather)
    dst[tid] = src[orig];
  else
    dst[orig] = src[tid];
}

// The 16-byte path of the same move on a 2-D grid: blockIdx.y is the shard
// slab kbh = k * BH + bh (uniform, so its split is scalar work), x runs over
// the n * ru 16-byte units of the slab.  Every unit is read and written once:
// non-temporal loads and stores.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) move16_kernel(bool gather, const u32x4v *__restrict__ src,
                                                     u32x4v *__restrict__ dst,
                                                     const int32_t *__restrict__ fwd, int64_t BH,
                                                     int64_t S, int64_t n, uint32_t ru,
                                                     int32_t rank0) {
  const uint32_t x = blockIdx.x * 256u + threadIdx.x;  // unit within the slab (< n * ru < 2^32)
  if ((int64_t)x >= n * ru) return;
  const int64_t kbh = blockIdx.y;
  const int64_t k = kbh / BH, bh = kbh - k * BH;
  const uint32_t j = x / ru, u = x - j * ru;
  const int64_t tok = fwd[(rank0 + k) * n + j];
  const int64_t sh = kbh * n * ru + x;
  const int64_t orig = (bh * S + tok) * ru + u;
  if (gather)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + orig), dst + sh);
  else
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + sh), dst + orig);
}

inline unsigned blocks_for(int64_t total) { return (unsigned)((total + 255) / 256); }

}  // namespace

// The K/V hand-off between hops: a plain copy, run on the side stream next to
// the block kernel.  A small grid (the copy has a whole hop to finish) and
// non-temporal 16-byte loads and stores that stream past the caches, so the
// copy neither takes many compute units nor evicts the K/V tiles the block
// kernel's workgroups share in L2.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyGrid = 64, kCopyUnroll = 4;
__global__ void __launch_bounds__(256) copy16_kernel(const u32x4 *__restrict__ src,
                                                     u32x4 *__restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * stride < n16; i += kCopyUnroll * stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_merge(float *o_acc, float *m_acc, float *l_acc, const float *o_blk,
                        const float *m_blk, const float *l_blk, int64_t rows, int32_t d,
                        hipStream_t s) {
  const int64_t total = rows * (d / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(blocks_for(total)), dim3(256), 0, s, o_acc, m_acc, l_acc,
                     o_blk, m_blk, l_blk, rows, d / 4, total);
  return hipGetLastError();
}

hipError_t launch_finalize(const float *o_acc, const float *m, const float *l, void *out,
                           float *lse, int dtype, int64_t rows, int32_t d, hipStream_t s) {
  const int64_t total = rows * (d / 4);
  if (total == 0) return hipSuccess;
  if (d % 8 == 0 && (uintptr_t)out % 16 == 0) {
    const int64_t t8 = rows * (d / 8);
    if (dtype == RA_DT_BF16)
      hipLaunchKernelGGL(finalize8_kernel<__bf16>, dim3(blocks_for(t8)), dim3(256), 0, s, o_acc,
                         m, l, (__bf16 *)out, lse, d / 8, t8);
    else if (dtype == RA_DT_FP16)
      hipLaunchKernelGGL(finalize8_kernel<_Float16>, dim3(blocks_for(t8)), dim3(256), 0, s, o_acc,
                         m, l, (_Float16 *)out, lse, d / 8, t8);
    else
      hipLaunchKernelGGL(finalize8_kernel<float>, dim3(blocks_for(t8)), dim3(256), 0, s, o_acc, m,
                         l, (float *)out, lse, d / 8, t8);
    return hipGetLastError();
  }
  if (dtype == RA_DT_BF16)
    hipLaunchKernelGGL(finalize_kernel<__bf16>, dim3(blocks_for(total)), dim3(256), 0, s, o_acc, m,
                       l, (__bf16 *)out, lse, d / 4, total);
  else if (dtype == RA_DT_FP16)
    hipLaunchKernelGGL(finalize_kernel<_Float16>, dim3(blocks_for(total)), dim3(256), 0, s, o_acc,
                       m, l, (_Float16 *)out, lse, d / 4, total);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, dim3(blocks_for(total)), dim3(256), 0, s, o_acc, m,
                       l, (float *)out, lse, d / 4, total);
  return hipGetLastError();
}

hipError_t launch_layout_permute(int layout, int64_t S, int32_t R, int32_t *fwd, int32_t *inv,
                                 hipStream_t s) {
  if (S == 0) return hipSuccess;
  hipLaunchKernelGGL(layout_kernel, dim3(blocks_for(S)), dim3(256), 0, s, layout, S, R, S / R,
                     fwd, inv);
  return hipGetLastError();
}

hipError_t launch_layout_move(bool gather, const void *src, void *dst, const int32_t *fwd,
                              int32_t elem_bytes, int64_t B, int64_t H, int64_t S, int64_t d,
                              int32_t R, int32_t rank0, int32_t n_ranks, hipStream_t s) {
  const int64_t n = S / R;
  const int64_t row_bytes = d * elem_bytes;
  const int64_t rows = (int64_t)n_ranks * B * H * n;
  if (rows == 0 || row_bytes == 0) return hipSuccess;
  const bool vec = (row_bytes % 16 == 0) && ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
  const int64_t ru16 = row_bytes / 16, slabs = (int64_t)n_ranks * B * H;
  if (vec && slabs <= 65535 && n * ru16 < (int64_t)1 << 31) {
    const dim3 grid((unsigned)((n * ru16 + 255) / 256), (unsigned)slabs);
    hipLaunchKernelGGL(move16_kernel, grid, dim3(256), 0, s, gather, (const u32x4v *)src,
                       (u32x4v *)dst, fwd, B * H, S, n, (uint32_t)ru16, rank0);
  } else if (vec) {
    const int64_t ru = row_bytes / 16, total = rows * ru;
    hipLaunchKernelGGL(move_kernel<uint4>, dim3(blocks_for(total)), dim3(256), 0, s, gather,
                       (const uint4 *)src, (uint4 *)dst, fwd, B * H, S, n, ru, rank0, total);
  } else if (elem_bytes == 8) {
    const int64_t total = rows * d;
    hipLaunchKernelGGL(move_kernel<uint64_t>, dim3(blocks_for(total)), dim3(256), 0, s, gather,
                       (const uint64_t *)src, (uint64_t *)dst, fwd, B * H, S, n, d, rank0, total);
  } else if (elem_bytes == 4) {
    const int64_t total = rows * d;
    hipLaunchKernelGGL(move_kernel<uint32_t>, dim3(blocks_for(total)), dim3(256), 0, s, gather,
                       (const uint32_t *)src, (uint32_t *)dst, fwd, B * H, S, n, d, rank0, total);
  } else if (elem_bytes == 2) {
    const int64_t total = rows * d;
    hipLaunchKernelGGL(move_kernel<uint16_t>, dim3(blocks_for(total)), dim3(256), 0, s, gather,
                       (const uint16_t *)src, (uint16_t *)dst, fwd, B * H, S, n, d, rank0, total);
  } else {
    const int64_t total = rows * d;
    hipLaunchKernelGGL(move_kernel<uint8_t>, dim3(blocks_for(total)), dim3(256), 0, s, gather,
                       (const uint8_t *)src, (uint8_t *)dst, fwd, B * H, S, n, d, rank0, total);
  }
  return hipGetLastError();
}

// The ring's hand-off copy for long hops, shaped to run beside the hop's kernels
// instead of taking compute units from them: one-wave workgroups of 16 VGPRs fit
// in the registers the attention kernels leave free on each SIMD (two of their
// waves hold 496 of the 512), so a copy wave shares a SIMD's issue slots and
// the memory system but displaces no attention workgroup.  Each workgroup
// copies one contiguous run of 1 KB units, two units in flight, with
// non-temporal loads and stores.  Alone it moves 3.5-4.6 TB/s of reads plus
// writes; next to a short, memory-heavy hop (512-token blocks) it costs more
// than the 64-workgroup copy above, which those hops take instead.
constexpr int kThinGrid = 1024;
__global__ void __launch_bounds__(64) copy16_thin_kernel(const u32x4 *__restrict__ src,
                                                         u32x4 *__restrict__ dst, int64_t n16) {
  const int64_t units = (n16 + 63) >> 6;
  const int64_t per = (units + gridDim.x - 1) / gridDim.x;
  const int64_t u0 = (int64_t)blockIdx.x * per;
  const int64_t u1 = u0 + per < units ? u0 + per : units;
  int64_t i = (u0 << 6) + threadIdx.x;
  const int64_t iend = (u1 << 6) < n16 ? (u1 << 6) : n16;
  for (; i + 64 < iend; i += 128) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + 64);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + 64);
  }
  if (i < iend) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_handoff_copy(void *dst, const void *src, size_t bytes, hipStream_t s,
                               bool thin) {
  if (!thin) return launch_copy(dst, src, bytes, s);
  if (bytes == 0) return hipSuccess;
  if (((uintptr_t)dst | (uintptr_t)src | bytes) & 15)
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t units = (n16 + 63) / 64;
  const unsigned grid = (unsigned)(units < kThinGrid ? units : kThinGrid);
  hipLaunchKernelGGL(copy16_thin_kernel, dim3(grid), dim3(64), 0, s, (const u32x4 *)src,
                     (u32x4 *)dst, n16);
  return hipGetLastError();
}

// One wave sleeping `n` times for s_sleep's longest step (64 x 127 clocks):
// a bounded stall that widens the windows between the ring's two streams.
__global__ void __launch_bounds__(64) delay_kernel(int n) {
  for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
}

hipError_t launch_delay(int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, s, n);
  return hipGetLastError();
}

hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s, int max_grid) {
  if (bytes == 0) return hipSuccess;
  if (((uintptr_t)dst | (uintptr_t)src | bytes) & 15)
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t need = (n16 + 255) / 256;
  const int64_t cap = max_grid > 0 ? max_grid : kCopyGrid;
  const unsigned grid = (unsigned)(need < cap ? need : cap);
  hipLaunchKernelGGL(copy16_kernel, dim3(grid), dim3(256), 0, s, (const u32x4 *)src, (u32x4 *)dst,
                     n16);
  return hipGetLastError();
}

}  // namespace ra
