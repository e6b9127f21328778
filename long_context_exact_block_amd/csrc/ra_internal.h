// ra_internal.h -- declarations shared by the host side of libra.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ra.h"

namespace ra {

// A batch of nz (query shard, K/V block) problems with one shape, launched
// together.  Problem z uses
//   q          = q + z*q_zstride
//   k          = k + ((kv_idx0 + z) % kv_idx_mod) * kv_zstride
//   v          = v + ((kv_idx0 + z) % kv_idx_mod) * kv_vzstride
//   qgid(i)    = qg_add + z*qg_z + i*q_step
//   kgid(j)    = kg_add + ((kg_s0 + z) % kg_smod)*kg_mult + j*k_step
// or, when zz_c > 0 (zig-zag ids, two chunks of zz_c tokens per rank), with
// rank = q_rank0 + z for queries and (kg_s0 + z) % kg_smod for keys:
//   gid(j)     = rank*zz_c + j                    (j < zz_c)
//              = (2*zz_R - 1 - rank)*zz_c + j - zz_c  (j >= zz_c)
//   o, m, l    = + z*o_zstride / z*ml_zstride
// which covers one public block call (nz = 1) and one ring hop over all
// computed ranks (z = rank index, block index and key ids follow the ring).
struct BatchParams {
  const void *q, *k, *v;
  int64_t q_zstride, kv_zstride, kv_vzstride;
  int32_t kv_idx0, kv_idx_mod;
  int64_t qs_b, qs_h, qs_t;
  int64_t ks_b, ks_h, ks_t;
  int64_t vs_b, vs_h, vs_t;
  int32_t B, Hq, Hkv, nq, nk, d, nz;
  float scale;
  int32_t causal;
  int64_t qg_add, qg_z, q_step;
  int64_t kg_add, kg_mult, k_step;
  int32_t kg_s0, kg_smod;
  float *o;
  int64_t o_zstride, os_b, os_h, os_t;
  float *m, *l;
  int64_t ml_zstride;
  // 0: write this block's partial (O normalised, m, l).
  // 1: continue the running state stored in o/m/l (same format) and write it
  //    back -- online softmax carried across hops.
  int32_t accumulate;
  // V layout: 0 = rows [token][d] (strides vs_*); 1 = packed transposed
  // blocks from pack_v (vs_b, vs_h as given, vs_t = the packed row length).
  int32_t v_packed;
  // 1: the stored m is the exact row maximum of the scores seen (a block
  // partial).  0: it may be any reference maximum the stored l is relative
  // to (a running state between hops; m + ln l is the same).
  int32_t exact_m;
  int32_t zz_c, zz_R, q_rank0;
  // In-kernel hand-off (the ring's FORWARD mode, 16-bit packed path): with
  // fwd = 1, problem z also writes the K block and the packed V block it reads
  // to slot z + 1 of the receive buffers fk / fv (laid out like k / v, slot s
  // at + s*kv_zstride / s*kv_vzstride), and with fwd_wrap the last problem to
  // slot 0; every workgroup writes its share of the block's 64-key tiles.
  void *fk, *fv;
  int32_t fwd, fwd_wrap;
};

// Packed V: for each (b, h) n_pad/64 tiles of [d][64] (n_pad = n rounded up
// to 64), position q of tile T's row c holding key 64T + perm16(q) (the 2nd
// and 3rd groups of four keys of every 16 swapped), zero past n.  This is the
// key order in which the PV product consumes probabilities, so every operand
// read is 16 bytes, and a 64-key V^T tile is one contiguous block.
constexpr int kPackAlign = 64;
// The packed-V kernel addresses a (b, h) slice of packed V and a 64-row K tile
// with 32-bit byte offsets: bound the packed row length and the K row stride.
constexpr int64_t kMaxPackedKeys = int64_t(1) << 23;
constexpr int64_t kMaxKRowStride = int64_t(1) << 22;
inline int64_t packed_n(int64_t n) { return (n + kPackAlign - 1) / kPackAlign * kPackAlign; }
hipError_t launch_pack_v(const void *v, void *vp, int elt, int64_t BH, int64_t H, int64_t n,
                         int64_t d, int64_t vs_b, int64_t vs_h, int64_t vs_t, hipStream_t s);
hipError_t launch_block_fwd_packed(const BatchParams &p, int dtype, hipStream_t s);

hipError_t launch_block_fwd(const BatchParams &p, int dtype, hipStream_t s);

// Decode: nq new queries per (b, query head) against a KV cache split over R
// ranks, rank r holding tokens r*n .. r*n + n - 1.  Every wave streams its own
// range of wave_keys keys of one (rank, b, kv head) for one block of 32 query
// columns (column c = head-in-group * nq + query); the waves of a workgroup
// fold their results into one partial (O normalised, m, l), and
// decode_reduce folds the P partials of every row.
constexpr int kDecodeWaves = 2;  // waves per decode workgroup (each streams its own keys)
struct DecodeParams {
  const void *q;  // [B][Hq][nq][d]
  const void *k;  // [R][B][Hkv][n][d]
  const void *v;  // packed: [R][B][Hkv][n_pad/64][d][64]
  int32_t B, Hq, Hkv, nq, n, d, R;
  int64_t n_pad;
  float scale;
  int32_t causal;
  int64_t q_gid0;     // token of query i: q_gid0 + i
  int32_t splits;     // key ranges per (rank, b, kv head), kDecodeWaves waves each
  int32_t wave_keys;  // keys per wave (a multiple of 32)
  int32_t col_blocks; // ceil(Hq/Hkv * nq / 32)
  int32_t P;          // partials per row: R * splits
  float *po, *pm, *pl;  // [P][rows][d], [P][rows], [P][rows]; rows = B*Hq*nq
};
hipError_t launch_decode(const DecodeParams &p, int dtype, void *o, float *lse,
                         hipStream_t s);
// Device-resident scratch of the allocation-free decode entry point: one
// array of kDecodeScratchBytes per device (devices 0 .. kMaxScratchDevices-1),
// its address looked up on the current device's first use.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t decode_scratch(void **ptr);
hipError_t launch_merge(float *o_acc, float *m_acc, float *l_acc, const float *o_blk,
                        const float *m_blk, const float *l_blk, int64_t rows, int32_t d,
                        hipStream_t s);
hipError_t launch_finalize(const float *o_acc, const float *m, const float *l, void *out,
                           float *lse, int dtype, int64_t rows, int32_t d, hipStream_t s);
hipError_t launch_layout_permute(int layout, int64_t S, int32_t R, int32_t *fwd, int32_t *inv,
                                 hipStream_t s);
// device-to-device copy on stream s (a small grid of at most max_grid workgroups,
// 0: the default 64; non-temporal; falls back to hipMemcpyAsync for pointers
// or sizes that are not 16-byte multiples)
hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s, int max_grid = 0);
// the ring's hand-off copy: thin -- one-wave workgroups small enough to run
// beside the attention kernels, for long hops -- or launch_copy
hipError_t launch_handoff_copy(void *dst, const void *src, size_t bytes, hipStream_t s, bool thin);
// a bounded sleep of n steps (~64 x 127 clocks each) on stream s; n <= 0: nothing
hipError_t launch_delay(int n, hipStream_t s);
hipError_t launch_layout_move(bool gather, const void *src, void *dst, const int32_t *fwd,
                              int32_t elem_bytes, int64_t B, int64_t H, int64_t S, int64_t d,
                              int32_t R, int32_t rank0, int32_t n_ranks, hipStream_t s);

// Backward of a batch of (query shard, K/V block) problems.  `a` carries the
// forward's addressing (q, k, v rows, contiguous per problem, global ids, z
// batching); the rest:
//   dout        like q (same strides)
//   qT, doT     packed (ra_pack_v layout) per query problem z: q_zstride_p
//   kT          packed per K/V block (block index as for k): kT_zstride
//   nl, nD      fp32 per query row: + z*ml_zstride, [b][h][i]; nl = -lse log2(e)
//               (-inf for a row with no key), nD = -<dO, O>, both from launch_bwd_prep
//   dq          fp32 accumulator like q rows: + z*dq_zstride, [b][h][i][d]
//   dk, dv      fp32 accumulators per K/V block: + kv*dk_zstride, [b][kvh][j][d]
// Each problem z adds its contributions; within a launch no two problems
// share a K/V block or a query shard.
struct BwdParams {
  BatchParams a;
  const void *dout;
  const void *qT, *doT, *kT;
  int64_t qT_zstride, kT_zstride;
  const float *nl, *nD;
  float *dq, *dk, *dv;
  int64_t dq_zstride, dk_zstride;
};
hipError_t launch_bwd_prep(const void *o, const void *dout, const float *lse, float *nD,
                           float *nl, int dtype, int64_t rows, int32_t d, hipStream_t s);
// parts: kBwdKV (the dK and dV kernels), kBwdQ (the dQ kernel) or both
constexpr int kBwdKV = 1, kBwdQ = 2, kBwdAll = 3;
hipError_t launch_bwd(const BwdParams &p, int dtype, hipStream_t s, int parts = kBwdAll);
hipError_t launch_zero(float *x, int64_t n, hipStream_t s);  // n % 4 == 0
hipError_t launch_cast(const float *x, void *y, int dtype, int64_t n, hipStream_t s);

// Per-thread detail text for ra_last_error().
void set_error(const char *fmt, ...);
void clear_error();

}  // namespace ra
