// issue_mix.hip -- what the matrix cores of gfx950 sustain next to the rest of
// an attention kernel's instruction mix.  Each wave issues 32x32x16 bf16 MFMAs
// on four independent accumulators and, per MFMA, optionally
//   - the softmax work of one score element: an FMA, an exponential and an add
//     (independent chains, as in the kernel), and
//   - LDS operand reads of 16 bytes per lane feeding the MFMA's A operand,
//     either one per MFMA or one per two MFMAs, read four steps ahead,
// with operands that either stay constant or change (random bf16 values, as
// real data: the chip's clock, and so its MFMA rate, depends on how much the
// data toggles).  One or two waves per SIMD (256 or 512 threads, one
// workgroup per CU).  Reports TFLOP/s against the 2.5 PFLOP/s dense bf16
// peak, the shader clock (s_memtime against the 100 MHz s_memrealtime), and
// the MFMA pipe's busy share at that clock.  A second kernel does the same with
// 16x16x32 bf16 MFMAs (half the FLOPs each), where one score element's softmax
// work comes every two MFMAs and a fragment can feed two, three or four of them
// (32, 48 or 64 queries per wave).  Only in-bounds LDS accesses; each thread
// writes one float of output.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kLdsBytes = 65536;  // the region the operand reads cover

// NL: LDS operand reads per two MFMAs (0, 1 or 2); SOFTMAX: one FMA, exp and
// add per MFMA; RAND: operands from random data (else constant)
template <int NL, bool SOFTMAX, bool RAND>
__global__ void mix_kernel(float *out, unsigned long long *clk, float y, float z, int iters) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsBytes / 16; i += blockDim.x) {
    unsigned h = (unsigned)i * 2654435761u + 12345u, w[4];
    for (int k = 0; k < 4; ++k) {
      h ^= h >> 13;
      h *= 0x5bd1e995u;
      h ^= h >> 15;
      // two bf16 values in [0.5, 2) with random sign and mantissa
      w[k] = RAND ? (((0x3f00u | ((h >> 24) & 0x80u)) | ((h >> 16) & 0x7fu)) << 16) |
                        (0x3f00u | ((h >> 8) & 0xffu))
                  : 0x3f803f80u;
    }
    ((uint4 *)lds)[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __syncthreads();
  const int lane = tid & 63;
  const int base = ((tid >> 6) & 3) * 16384 + lane * 16;  // 16 KB per SIMD, 1 KB per read
  s16x8 fr[4];
  for (int u = 0; u < 4; ++u) fr[u] = *(const s16x8 *)(lds + base + u * 1024);
  const s16x8 b = *(const s16x8 *)(lds + base + 8192);
  const s16x8 a0 = *(const s16x8 *)(lds + base + 9216);
  const s16x8 a1 = *(const s16x8 *)(lds + base + 10240);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  f32x16 acc[4];
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
  float xf[8], xe[8], xa[8];
  for (int u = 0; u < 8; ++u) {
    xf[u] = tid * 0.001f + u;
    xe[u] = 0.01f * u;
    xa[u] = u;
  }
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) {
      s16x8 av = (mm & 1) ? a1 : a0;
      if (NL == 2) {  // one read per MFMA, consumed four steps later
        av = fr[mm & 3];
        fr[mm & 3] = *(const s16x8 *)(lds + base + ((mm + (it >> 2)) & 7) * 1024);
      } else if (NL == 1) {  // one read per two MFMAs, each fragment feeds both
        av = fr[(mm >> 1) & 3];
        if (mm & 1) fr[(mm >> 1) & 3] = *(const s16x8 *)(lds + base + ((mm + (it >> 2)) & 7) * 1024);
      }
      acc[mm & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                            __builtin_bit_cast(bf16x8, b),
                                                            acc[mm & 3], 0, 0, 0);
      if (SOFTMAX) {
        const int j = mm & 7;
        xf[j] = fmaf(xf[j], y, z);
        xe[j] = __builtin_amdgcn_exp2f(xe[j]);
        xa[j] = xa[j] + xe[(j + 3) & 7];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 16; ++r) s += acc[m][r];
  for (int u = 0; u < 8; ++u) s += xf[u] + xe[u] + xa[u];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// 16x16x32 MFMAs on four accumulators; one FMA, exp and add every two MFMAs
// (the softmax work per FLOP of the 32x32x16 kernel's SOFTMAX rows); one
// 16-byte LDS read every LDP MFMAs, each fragment feeding LDP of them.
template <int LDP>
__global__ void __launch_bounds__(768) mix16_kernel(float *out, unsigned long long *clk, float y,
                                                    float z, int iters) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsBytes / 16; i += blockDim.x) {
    unsigned h = (unsigned)i * 2654435761u + 12345u, w[4];
    for (int k = 0; k < 4; ++k) {
      h ^= h >> 13;
      h *= 0x5bd1e995u;
      h ^= h >> 15;
      w[k] = (((0x3f00u | ((h >> 24) & 0x80u)) | ((h >> 16) & 0x7fu)) << 16) |
             (0x3f00u | ((h >> 8) & 0xffu));
    }
    ((uint4 *)lds)[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __syncthreads();
  const int lane = tid & 63;
  const int base = ((tid >> 6) & 3) * 16384 + lane * 16;  // <= 50,160: reads end below 64 KB
  s16x8 fr[4];
  for (int u = 0; u < 4; ++u) fr[u] = *(const s16x8 *)(lds + base + u * 1024);
  const s16x8 b = *(const s16x8 *)(lds + base + 8192);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  f32x4 acc[4];
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 4; ++r) acc[m][r] = 0.f;
  float xf[8], xe[8], xa[8];
  for (int u = 0; u < 8; ++u) {
    xf[u] = tid * 0.001f + u;
    xe[u] = 0.01f * u;
    xa[u] = u;
  }
  int rd = 0;
  for (int it = 0; it < iters; it += 12) {
#pragma unroll
    for (int mm = 0; mm < 12; ++mm) {
      const s16x8 av = fr[(mm / LDP) & 3];
      if (mm % LDP == LDP - 1)  // the fragment's last use: read its successor
        fr[(mm / LDP) & 3] = *(const s16x8 *)(lds + base + ((rd + mm) & 7) * 1024);
      acc[mm & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                            __builtin_bit_cast(bf16x8, b),
                                                            acc[mm & 3], 0, 0, 0);
      if ((mm & 1) == 0) {
        const int j = (mm >> 1) & 7;
        xf[j] = fmaf(xf[j], y, z);
        xe[j] = __builtin_amdgcn_exp2f(xe[j]);
        xa[j] = xa[j] + xe[(j + 3) & 7];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    rd += 5;
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 4; ++r) s += acc[m][r];
  for (int u = 0; u < 8; ++u) s += xf[u] + xe[u] + xa[u];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

constexpr int kGrid = 256;  // one workgroup per CU (its LDS allows no second)

typedef void (*MixKernel)(float *, unsigned long long *, float, float, int);

void run_kernel(MixKernel kern, double flop_per_mfma, const char *name, int threads, int iters,
                float *out, unsigned long long *clk) {
  const size_t lds = 100 * 1024;
  if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds) != hipSuccess) {
    printf("%s: hipFuncSetAttribute failed\n", name);
    exit(1);
  }
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  hipLaunchKernelGGL(kern, dim3(kGrid), dim3(threads), lds, 0, out, clk, 1.0001f, 0.5f, iters);
  (void)hipEventRecord(e0);
  const int reps = 3;
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(kern, dim3(kGrid), dim3(threads), lds, 0, out, clk, 1.0001f, 0.5f, iters);
  (void)hipEventRecord(e1);
  if (hipEventSynchronize(e1) != hipSuccess) {
    printf("%s: kernel failed\n", name);
    exit(1);
  }
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  ms /= reps;
  unsigned long long c[2 * kGrid];
  (void)hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost);
  double mhz = 0.0;
  for (int i = 0; i < kGrid; ++i) mhz += (double)c[2 * i] / (double)c[2 * i + 1];
  mhz = mhz / kGrid * 100.0;
  const double flop = flop_per_mfma * iters * (threads / 64) * kGrid;
  const double tf = flop / ms / 1e9;
  printf("| %-40s | %d | %.1f | %.3f | %.0f | %.3f |\n", name, threads / 256, tf, tf / 2500.0, mhz,
         tf / (2500.0 * mhz / 2400.0));
  fflush(stdout);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
}

// the 32x32x16 kernel issues four MFMAs per unit of iters
template <int NL, bool SOFTMAX, bool RAND>
void run(const char *name, int threads, int iters, float *out, unsigned long long *clk) {
  run_kernel(mix_kernel<NL, SOFTMAX, RAND>, 2.0 * 32 * 32 * 16 * 4.0, name, threads, iters, out,
             clk);
}

// the 16x16x32 kernel issues one MFMA per unit of iters (a multiple of 12)
template <int LDP>
void run16(const char *name, int threads, int iters, float *out, unsigned long long *clk) {
  run_kernel(mix16_kernel<LDP>, 2.0 * 16 * 16 * 32, name, threads, iters, out, clk);
}

int main() {
  float *out = nullptr;
  unsigned long long *clk = nullptr;
  if (hipMalloc(&out, kGrid * 1024 * sizeof(float)) != hipSuccess ||
      hipMalloc(&clk, kGrid * 2 * sizeof(unsigned long long)) != hipSuccess) {
    printf("hipMalloc failed\n");
    return 1;
  }
  const int it = 200000;
  printf("| per MFMA | waves per SIMD | TFLOP/s | of 2.5 PF | clock MHz | MFMA busy at that clock |\n");
  printf("|---|---|---|---|---|---|\n");
  run<0, false, false>("MFMA only, constant operands", 256, it, out, clk);
  run<0, false, false>("MFMA only, constant operands", 512, it / 2, out, clk);
  run<0, false, true>("MFMA only, random operands", 256, it, out, clk);
  run<0, false, true>("MFMA only, random operands", 512, it / 2, out, clk);
  run<0, true, true>("+ fma, exp, add", 512, it / 2, out, clk);
  run<1, false, true>("+ 1/2 LDS read", 512, it / 2, out, clk);
  run<2, false, true>("+ 1 LDS read", 512, it / 2, out, clk);
  run<1, true, true>("+ fma, exp, add + 1/2 LDS read", 512, it / 2, out, clk);
  run<2, true, true>("+ fma, exp, add + 1 LDS read", 512, it / 2, out, clk);
  run<1, true, true>("+ fma, exp, add + 1/2 LDS read", 256, it, out, clk);
  run<2, true, true>("+ fma, exp, add + 1 LDS read", 256, it, out, clk);
  // 16x16x32: per wave the FLOPs of the two-wave 32x32x16 rows (2 x 4 x it / 2 MFMAs of
  // half the size), rounded down to whole 12-MFMA steps
  const int it16 = (it * 4 / 12) * 12;
  run16<2>("16x16x32 + fma, exp, add per 2 + 1/2 LDS read", 512, it16, out, clk);
  run16<3>("16x16x32 + fma, exp, add per 2 + 1/3 LDS read", 512, it16, out, clk);
  run16<4>("16x16x32 + fma, exp, add per 2 + 1/4 LDS read", 512, it16, out, clk);
  run16<3>("16x16x32 + fma, exp, add per 2 + 1/3 LDS read", 768, it16, out, clk);
  (void)hipFree(out);
  (void)hipFree(clk);
  return 0;
}
