/*
 * ra.h -- C ABI of the MI355X (gfx950) ring-attention library (libra.so).
 *
 * The library computes exact causal / non-causal attention the way a ring of
 * R ranks does it: every rank keeps its query shard, key/value blocks travel
 * hop by hop, and each arriving block's partial attention is folded into a
 * running (O, m, l) with online softmax.  On one GPU the ring is emulated:
 * all computed ranks run in one launch per hop and the hop-to-hop K/V
 * hand-off is an on-device copy on a second HIP stream, overlapped with the
 * compute of the current hop.
 *
 * Page citations (page title and section):
 *  [ZZ] highthink.cn repost of the context-parallelism / Ring Attention
 *       article, section "Zig Zag Ring Attention 通信和计算重叠": ring of
 *       ranks, K/V passed to the next rank while the current block is
 *       computed, causal rule, interleaved token assignment.
 *  [DE] aiunderstanding.org "Sequenzparallelität und Ringaufmerksamkeit",
 *       "Tiefer Einblick" and FAQ: contiguous split, online softmax with
 *       running max and sum, blockwise result equals full attention, only
 *       K/V move while queries stay.
 *  [TH] Thai version of that guide, technical-insight section: running
 *       maximum, running normaliser, rescaling of earlier partial sums.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device pointers; "host" are host
 *    pointers.  The caller allocates and frees every buffer.
 *  - `stream` arguments are hipStream_t values passed as void* (NULL is the
 *    null stream).  Calls are asynchronous: they return once the work is
 *    enqueued.  Argument validation happens on the host before anything is
 *    enqueued; on a non-OK status nothing was enqueued.
 *  - A HIP launch/copy failure returns RA_ERR_HIP; ra_last_error() then
 *    holds the HIP error text.  Faults inside kernels surface at the
 *    caller's next synchronisation.  No C++ exception crosses the ABI.
 *  - Outputs never alias inputs (ra_merge updates its accumulator in place).
 *  - No floating-point atomics are used: results are bitwise reproducible
 *    for identical arguments on the same device.
 *  - Element dtypes: bf16 and fp16 (16-bit MFMA path), fp32 (fp32 MFMA path).
 *    Head dimension d must be 64 or 128.  Rows (the last, d-long dimension)
 *    must be contiguous and 16-byte aligned.
 */
#ifndef RA_H_
#define RA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ra_stream; /* a hipStream_t */

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1, /* null pointer, bad enum value, bad scalar          */
  RA_ERR_SHAPE = 2,       /* sizes inconsistent (S % R, Hq % Hkv, d, ranks...)  */
  RA_ERR_DTYPE = 3,       /* unknown dtype                                      */
  RA_ERR_ALIGNMENT = 4,   /* pointer or row stride not 16-byte aligned          */
  RA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required         */
  RA_ERR_UNSUPPORTED = 6, /* valid request this build does not implement        */
  RA_ERR_HIP = 7          /* a HIP runtime call failed                          */
} ra_status;

typedef enum { RA_LAYOUT_CONTIGUOUS = 0, RA_LAYOUT_STRIPED = 1, RA_LAYOUT_ZIGZAG = 2 } ra_layout;
typedef enum { RA_DT_BF16 = 0, RA_DT_FP16 = 1, RA_DT_FP32 = 2 } ra_dtype;
/* How the next K/V block reaches a rank. COPY: an on-device copy on the copy
 * stream into the rank's receive buffer (the emulated link); SWAP: the rank
 * reads the resident block in place (no transfer; an upper bound); FORWARD:
 * as COPY, but on hops too short for the copy to hide beside the block kernel
 * (ra_handoff_thin returns 0: the copy would compete with the kernel for
 * memory), a block whose next holder is a computed rank is written to that
 * rank's receive buffer by the block kernel itself, from the tiles it loads
 * while it computes (each workgroup writes its share; no copy kernel and no
 * second stream for those blocks -- in a ring over several GPUs these would be
 * stores into the peer's buffer).  Long hops, blocks entering from ranks that
 * are not computed, and the fp32 path are copied as in COPY; ra_ring_bwd
 * treats FORWARD as COPY.  All three give bitwise equal results. */
typedef enum { RA_HANDOFF_COPY = 0, RA_HANDOFF_SWAP = 1, RA_HANDOFF_FORWARD = 2 } ra_handoff;
/* How each hop's partial is folded. FUSED: the block kernel continues the
 * running online softmax from the accumulator; SEPARATE: ra_block_fwd writes
 * the hop's partial and ra_merge folds it in. */
typedef enum { RA_MERGE_FUSED = 0, RA_MERGE_SEPARATE = 1 } ra_merge_mode;

/* Library version (major*10000 + minor*100 + patch). */
int ra_version(void);
/* Static text for a status code. */
const char *ra_status_string(ra_status s);
/* Detail of the last non-OK status returned on this host thread ("" if none). */
const char *ra_last_error(void);

/*
 * ra_layout_permute -- token <-> slot index maps of a sequence split over R
 * ranks.  Slot p = r*n + j is local position j of rank r (n = S/R).
 *   RA_LAYOUT_CONTIGUOUS ([DE] "Tiefer Einblick": each rank owns a contiguous
 *     run of tokens):           fwd[p] = p
 *   RA_LAYOUT_STRIPED ([ZZ] interleaved assignment, rank r holds r, r+R,
 *     r+2R, ...):               fwd[r*n + j] = j*R + r
 *   RA_LAYOUT_ZIGZAG ([ZZ] and [DE] "Zukunft" name a zig-zag assignment; read
 *     as 2R chunks of c = S/(2R) tokens, rank r holding chunk r then chunk
 *     2R-1-r, which gives every rank the same causal work):
 *                               fwd[r*n + j] = r*c + j            (j < c)
 *                               fwd[r*n + j] = (2R-1-r)*c + j - c  (j >= c)
 *   inv[fwd[p]] = p.
 * fwd, inv: device int32[S] (inv may be NULL).  Requires S % R == 0 (S % 2R
 * == 0 for zig-zag), 1 <= R, S < 2^31.  Errors: RA_ERR_INVALID_ARG,
 * RA_ERR_SHAPE, RA_ERR_HIP.
 */
ra_status ra_layout_permute(int32_t layout, int64_t S, int32_t R, int32_t *fwd,
                            int32_t *inv, ra_stream stream);

/*
 * ra_layout_gather -- move rows from the original token order into rank
 * shards using a map from ra_layout_permute ([ZZ], [DE]: each rank holds the
 * Q, K and V rows of its own tokens).
 *   x    device [B][H][S][d] elements of elem_bytes each (original order)
 *   fwd  device int32[S] (slot -> token)
 *   x_sh device [n_ranks][B][H][n][d], shard k holding rank rank0+k:
 *        x_sh[k][b][h][j] = x[b][h][fwd[(rank0+k)*n + j]]
 * elem_bytes in {1, 2, 4, 8}; (d*elem_bytes) % 16 == 0 and 16-byte aligned
 * pointers give the vector path, anything else a scalar path.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE, RA_ERR_HIP.
 */
ra_status ra_layout_gather(const void *x, void *x_sh, const int32_t *fwd, int32_t elem_bytes,
                           int64_t B, int64_t H, int64_t S, int64_t d, int32_t R, int32_t rank0,
                           int32_t n_ranks, ra_stream stream);

/*
 * ra_layout_scatter -- inverse of ra_layout_gather for the ranks given:
 *   x[b][h][fwd[(rank0+k)*n + j]] = x_sh[k][b][h][j]
 * Rows of x owned by other ranks are left untouched.  Same arguments and
 * errors as ra_layout_gather (x is the output here).
 */
ra_status ra_layout_scatter(const void *x_sh, void *x, const int32_t *fwd, int32_t elem_bytes,
                            int64_t B, int64_t H, int64_t S, int64_t d, int32_t R,
                            int32_t rank0, int32_t n_ranks, ra_stream stream);

/*
 * ra_block_fwd -- partial attention of one query shard against one K/V block:
 * the work a rank does when a block arrives ([DE] "Tiefer Einblick": partial
 * attention per arriving block; [TH]: running max and normaliser).
 *
 * For batch b, query head h (K/V head g = h / (Hq/Hkv)) and local query i,
 * the allowed keys are A = { j : !causal || kgid(j) <= qgid(i) } with
 * qgid(i) = q_gid0 + i*q_gid_step and kgid(j) = k_gid0 + j*k_gid_step
 * ([ZZ]: a token attends only to tokens not after it; the diagonal is
 * included).  With s_j = scale * <q_i, k_j> (fp32 accumulation of products of
 * the input dtype):
 *   m = max_{j in A} s_j (natural units, scale included)
 *   l = sum_{j in A} exp(s_j - m)          (fp32, from unrounded p)
 *   O = sum_{j in A} exp(s_j - m) v_j / l  (p rounded to the input dtype for
 *                                           the PV product; fp32 accumulate)
 * A row with no allowed key gets O = 0, m = -inf, l = 0.
 *
 * Layout: q element (b,h,i,c) at q + b*q_stride[0] + h*q_stride[1]
 * + i*q_stride[2] + c (element strides); likewise k, v with Hkv heads and
 * n_k rows, and o (fp32) with o_stride.  With v_packed = 1, v is the output
 * of ra_pack_v for (B, Hkv, n_k, d) and v_stride is ignored; that path reads
 * V with plain 16-byte loads and is the fast one.  m, l are dense fp32 [B][Hq][n_q].
 * All device pointers.  Requires Hq % Hkv == 0, d in {64,128}, n_q, n_k >= 0,
 * the global-id steps >= 1, 16-byte aligned rows.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE, RA_ERR_DTYPE, RA_ERR_ALIGNMENT,
 * RA_ERR_HIP.
 */
typedef struct {
  const void *q, *k, *v;
  int32_t dtype; /* ra_dtype */
  int32_t v_packed; /* 0: v rows with v_stride; 1: v from ra_pack_v (bf16/fp16 only) */
  int32_t B, Hq, Hkv, n_q, n_k, d;
  int64_t q_stride[3], k_stride[3], v_stride[3];
  float scale;
  int32_t causal;
  int64_t q_gid0, q_gid_step, k_gid0, k_gid_step;
  float *o;
  int64_t o_stride[3];
  float *m, *l;
} ra_block_args;

ra_status ra_block_fwd(const ra_block_args *a, ra_stream stream);

/*
 * ra_pack_v -- repack V rows for the fast PV path of ra_block_fwd (the ring
 * does this itself).  v: device [B][H][n][d] with element strides v_stride
 * (d contiguous, 16-byte aligned rows); vp: device, ra_packed_v_bytes bytes.
 * Packed layout: per (b, h), n_pad/64 tiles (n_pad = n rounded up to 64),
 * each a [d][64] array: tile T, row c, position q holds V[b][h][key][c] with
 * key = 64T + q except that within every 16 positions the 2nd and 3rd groups
 * of four keys are swapped (the order in which the probability matrix feeds
 * the PV product); zero where key >= n.  A 64-key tile of V^T is one
 * contiguous d*128-byte block.  bf16 / fp16 only.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE, RA_ERR_DTYPE, RA_ERR_ALIGNMENT,
 * RA_ERR_HIP.
 */
size_t ra_packed_v_bytes(int32_t dtype, int32_t B, int32_t H, int32_t n, int32_t d);
ra_status ra_pack_v(const void *v, void *vp, int32_t dtype, int32_t B, int32_t H, int32_t n,
                    int32_t d, const int64_t v_stride[3], ra_stream stream);

/*
 * ra_merge -- online-softmax combine of two partials of the same rows, in
 * place on the accumulator ([TH]: rescale the earlier partial sums when a
 * larger maximum appears; [DE] FAQ: blockwise equals full attention):
 *   m = max(m_a, m_b); w_a = l_a e^{m_a-m}; w_b = l_b e^{m_b-m};
 *   l = w_a + w_b;     O = (w_a O_a + w_b O_b) / l
 * (0, -inf, 0) is the identity; two empty rows stay (0, -inf, 0).
 * o_*: device fp32 [rows][d] contiguous; m_*, l_*: device fp32 [rows].
 * d % 4 == 0, 16-byte aligned o pointers.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE, RA_ERR_ALIGNMENT, RA_ERR_HIP.
 */
ra_status ra_merge(float *o_acc, float *m_acc, float *l_acc, const float *o_blk,
                   const float *m_blk, const float *l_blk, int64_t rows, int32_t d,
                   ra_stream stream);

/*
 * ra_handoff_copy -- the K/V hand-off between hops (highthink.cn article,
 * section on Zig Zag Ring Attention: each rank passes the K/V it holds to its
 * ring successor while attending to the current block): a device-to-device
 * copy of `bytes` bytes on `stream`, in either of the two forms the rings
 * issue on their copy stream, with non-temporal loads and stores:
 *   thin = 1: one-wave workgroups of 16 VGPRs that fit in the registers the
 *     attention kernels leave free, so they run beside them without
 *     displacing their workgroups.  The rings use it where ra_handoff_thin
 *     says so.
 *   thin = 0: 64 workgroups of 256 threads, for short, memory-heavy hops.
 * dst, src: device pointers, not overlapping; 16-byte aligned pointers and a
 * multiple of 16 bytes take the kernels, anything else falls back to
 * hipMemcpyAsync.  Asynchronous.
 * Errors: RA_ERR_INVALID_ARG (thin not 0 or 1; null pointer with bytes > 0),
 * RA_ERR_HIP.
 */
ra_status ra_handoff_copy(void *dst, const void *src, size_t bytes, int32_t thin,
                          ra_stream stream);

/*
 * ra_handoff_thin -- which hand-off copy form the rings use for a hop
 * (instrumentation: lets a benchmark time the copies alone in that form).
 * Returns 1 (thin) when the hop's estimated MFMA time -- `work` times 4 d flop
 * per allowed (query, key) pair and query head, `pairs_heads` of them, at
 * 1.3 PFLOP/s; work = 1 for the forward, 3.2 for the backward's kernels -- is
 * at least half the time the hop's `moved_bytes` (read plus written) take at
 * 1 TB/s; else 0.  Host-only arithmetic: no device call, no error.
 */
int32_t ra_handoff_thin(double moved_bytes, double pairs_heads, int32_t d, double work);

/*
 * ra_finalize -- running state to outputs: out = O rounded to nearest even
 * in `dtype`, lse = m + ln(l) (fp32, natural log; -inf for an empty row).
 * o_acc device fp32 [rows][d]; out device [rows][d] of dtype; m, l, lse
 * device fp32 [rows].  Errors as ra_merge, plus RA_ERR_DTYPE.
 */
ra_status ra_finalize(const float *o_acc, const float *m, const float *l, void *out,
                      float *lse, int32_t dtype, int64_t rows, int32_t d, ra_stream stream);

/*
 * ra_ring_fwd -- the whole ring on one GPU ([ZZ]: every rank keeps its Q
 * chunk, passes its K/V chunk to the next rank and receives the previous
 * rank's, until every query has met every key; the transfer overlaps the
 * compute of the current block).
 *
 * Computed query ranks r = rank0 .. rank0+n_ranks-1 (all R, or a single
 * rank's share; rank0 + n_ranks <= R).  At hop h = 0..R-1 rank r holds the block of source rank
 * s = (r - h) mod R.  Global token ids follow `layout` (contiguous: rank r,
 * local j -> r*n + j; striped: j*R + r; zig-zag: the two chunks of
 * ra_layout_permute, n even).
 *   q_sh  device [n_ranks][B][Hq][n][d]   query shards of the computed ranks
 *   k_sh, v_sh device [R][B][Hkv][n][d]   every source rank's K/V shard (on
 *         one GPU they stand in for the other ranks' memory)
 *   o     device [n_ranks][B][Hq][n][d] in dtype
 *   lse   device fp32 [n_ranks][B][Hq][n] (natural log)
 * handoff COPY: before hop h+1 each rank's receive buffer is filled, on the
 * `copy` stream, with the block its ring predecessor holds at hop h, while
 * the `compute` stream runs hop h; events order the two streams (no
 * write-after-read on the double buffer).  SWAP reads blocks in place.
 * FORWARD (16-bit dtypes, hops too short for the thin copy): hop h's block
 * kernel writes the block of computed rank r to the receive buffer of
 * computed rank r+1 (on a full ring, rank rank0+n_ranks-1's to rank0) as it
 * streams it; only blocks whose sender is not computed go through the copy
 * stream (none when n_ranks = R).  Hop h+1 reads the buffer hop h wrote and
 * hop h-1 read, on the same stream.  On other hops FORWARD is COPY.
 * The copy stream first waits for work already on the compute stream; the
 * compute stream waits for the copy stream before the call's last kernel,
 * so everything is complete when `compute` is.  Passing the same stream
 * twice is allowed (serialised, same results).
 * The workspace (device, ra_ring_fwd_workspace_size bytes, 256-byte
 * aligned) holds the packed V blocks (16-bit dtypes; see ra_pack_v), the
 * two receive buffers and the fp32 running state.
 * COPY, SWAP and FORWARD give bitwise-identical outputs; FUSED and SEPARATE
 * agree to rounding.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE, RA_ERR_DTYPE, RA_ERR_ALIGNMENT,
 * RA_ERR_WORKSPACE, RA_ERR_HIP.
 */
typedef struct {
  const void *q_sh, *k_sh, *v_sh;
  int32_t dtype;  /* ra_dtype */
  int32_t R, rank0, n_ranks;
  int32_t B, Hq, Hkv, n, d;
  float scale;
  int32_t causal;
  int32_t layout;     /* ra_layout */
  int32_t handoff;    /* ra_handoff */
  int32_t merge_mode; /* ra_merge_mode */
  void *o;
  float *lse;
  /* Instrumentation, not part of the computation: an optional host array of
   * 2*R hipEvent_t created by the caller (or NULL).  Event 2h is recorded on
   * `compute` right before hop h's block kernel and event 2h+1 right after
   * it, so a caller can time the block kernel on the stream it runs on.
   * Results do not depend on it. */
  void **hop_events;
} ra_ring_args;

/* Bytes of workspace ra_ring_fwd needs for these arguments (0 on invalid
 * arguments; ra_last_error() says why). */
size_t ra_ring_fwd_workspace_size(const ra_ring_args *a);

ra_status ra_ring_fwd(const ra_ring_args *a, void *workspace, size_t workspace_bytes,
                      ra_stream compute, ra_stream copy);

/*
 * ra_block_bwd -- gradient contributions of one query shard x one K/V block:
 * the unit of work of one hop of the backward ring (training is the pages'
 * headline use; they give no backward algorithm, so this is the derivative
 * of the forward: p = exp(s - lse), dP = dO v, D = <dO, O>, dS = p(dP - D),
 * dQ += scale dS k, dK += scale dS^T q, dV += p^T dO).  lse and O are the
 * forward's outputs over the WHOLE sequence (not this block's partial), so
 * the contributions of all blocks add up to the full gradients.
 *   q, o, dout  device [B][Hq][n_q][d] in dtype, contiguous
 *   k, v        device [B][Hkv][n_k][d] in dtype, contiguous
 *   lse         device fp32 [B][Hq][n_q] (natural log, as ra_finalize writes)
 *   ids, scale, causal as in ra_block_args
 *   dq          device fp32 [B][Hq][n_q][d]; dk, dv device fp32 [B][Hkv][n_k][d]:
 *               the call ADDS this pair's contributions (dk, dv summed over
 *               the query heads of a K/V head)
 * 16-bit dtypes, d in {64, 128}.  The workspace (ra_block_bwd_workspace_size
 * bytes, 256-byte aligned) holds transposed copies of q, dout, k, and D and
 * -lse log2(e) per query row.
 * Deterministic (no atomics).  Asynchronous on `stream`.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE, RA_ERR_DTYPE, RA_ERR_ALIGNMENT,
 * RA_ERR_WORKSPACE, RA_ERR_UNSUPPORTED, RA_ERR_HIP.
 */
typedef struct {
  const void *q, *k, *v, *o, *dout;
  int32_t dtype;
  int32_t B, Hq, Hkv, n_q, n_k, d;
  float scale;
  int32_t causal;
  int64_t q_gid0, q_gid_step, k_gid0, k_gid_step;
  const float *lse;
  float *dq, *dk, *dv;
} ra_block_bwd_args;

size_t ra_block_bwd_workspace_size(const ra_block_bwd_args *a);
ra_status ra_block_bwd(const ra_block_bwd_args *a, void *workspace, size_t workspace_bytes,
                       ra_stream stream);

/*
 * ra_ring_bwd -- the backward pass over the whole ring on one GPU: every
 * computed query rank r meets the block of source rank s = (r - h) mod R at
 * hop h (as in ra_ring_fwd) and adds that pair's gradient contributions; dQ
 * stays with its rank, dK/dV belong to the block and travel with it ([ZZ]:
 * each rank passes on what it holds while it computes).
 *   q_sh, k_sh, v_sh, R, rank0, n_ranks, B, Hq, Hkv, n, d, scale, causal,
 *   layout: as in ra_ring_args (16-bit dtypes only)
 *   handoff COPY: before hop h+1 each computed rank's receive buffers are
 *     filled on the `copy` stream with what its ring predecessor held at hop
 *     h: K, V and the transposed K while hop h computes, then the block's
 *     fp32 dK/dV accumulators once hop h's kernels are done (they arrive
 *     while hop h+1's dQ kernel runs); a block leaving the computed ranks
 *     (or the ring's end) puts its accumulators back home.  SWAP reads and
 *     accumulates every block in place.  Both give bitwise-identical results.
 *     FORWARD is handled as COPY here.
 *     Stream ordering as in ra_ring_fwd (same stream twice is allowed).
 *   o_sh, dout_sh  device [n_ranks][B][Hq][n][d]: the forward's O and the
 *                  upstream gradient of the computed ranks
 *   lse            device fp32 [n_ranks][B][Hq][n]: the forward's LSE
 *   dq_sh          device [n_ranks][B][Hq][n][d] in dtype (written)
 *   dk_sh, dv_sh   device [R][B][Hkv][n][d] in dtype (written): gradients of
 *                  every source block from the computed query ranks
 * Workspace: ra_ring_bwd_workspace_size bytes, 256-byte aligned (transposed
 * copies of Q, dO, K; D and -lse log2(e) per query row; fp32 accumulators;
 * with COPY the two receive buffers).  Asynchronous on the streams.
 * Errors: as ra_ring_fwd, plus RA_ERR_UNSUPPORTED for fp32.
 */
typedef struct {
  const void *q_sh, *k_sh, *v_sh, *o_sh, *dout_sh;
  const float *lse;
  int32_t dtype;
  int32_t R, rank0, n_ranks;
  int32_t B, Hq, Hkv, n, d;
  float scale;
  int32_t causal;
  int32_t layout;
  int32_t handoff; /* ra_handoff */
  void *dq_sh, *dk_sh, *dv_sh;
} ra_ring_bwd_args;

size_t ra_ring_bwd_workspace_size(const ra_ring_bwd_args *a);
ra_status ra_ring_bwd(const ra_ring_bwd_args *a, void *workspace, size_t workspace_bytes,
                      ra_stream compute, ra_stream copy);

/*
 * ra_decode_fwd -- nq new query tokens against a KV cache split over R ranks:
 * rank r holds the contiguous run of tokens r*n .. r*n + n - 1 ([DE]
 * "Tiefer Einblick": contiguous split; "Reale Umsetzung": serving long
 * contexts).  Every rank's run yields partial attention of the new queries
 * (several partials per run on one GPU), and all partials of a row are
 * folded with the online-softmax combine of ra_merge ([TH]; [DE] FAQ).
 *   q   device [B][Hq][nq][d]   new queries, contiguous
 *   k   device [R][B][Hkv][n][d] the cache shards, contiguous
 *   v   device, the shards' V in the packed layout: ra_pack_v applied to V
 *       seen as [R*B][Hkv][n][d] (ra_packed_v_bytes(dtype, R*B, Hkv, n, d))
 *   query i is token q_gid0 + i; causal: it attends to cache tokens <= its
 *   own (the new tokens' own K/V are expected in the cache); otherwise to all
 *   o   device [B][Hq][nq][d] in dtype; lse device fp32 [B][Hq][nq]
 *   (natural log; a row that sees no key gets O = 0, LSE = -inf)
 * Grouped heads: query head h uses K/V head h / (Hq/Hkv).  16-bit dtypes
 * only; d in {64, 128}; 1 <= nq and (Hq/Hkv)*nq <= 256; n <= 2^23; R <= 512.
 * The workspace (ra_decode_fwd_workspace_size bytes, 256-byte aligned)
 * holds the fp32 partials.  Asynchronous on `stream`.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE, RA_ERR_DTYPE, RA_ERR_ALIGNMENT,
 * RA_ERR_WORKSPACE, RA_ERR_UNSUPPORTED, RA_ERR_HIP.
 */
typedef struct {
  const void *q, *k, *v;
  int32_t dtype; /* ra_dtype: RA_DT_BF16 or RA_DT_FP16 */
  int32_t R, B, Hq, Hkv, nq, n, d;
  float scale;
  int32_t causal;
  int64_t q_gid0;
  void *o;
  float *lse;
} ra_decode_args;

size_t ra_decode_fwd_workspace_size(const ra_decode_args *a);
ra_status ra_decode_fwd(const ra_decode_args *a, void *workspace, size_t workspace_bytes,
                        ra_stream stream);

/*
 * ra_decode_fwd_noalloc -- ra_decode_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, kernels and results (bitwise) as
 * ra_decode_fwd, but the fp32 partials live in a device array the library
 * holds per GPU (32 MiB each, kept until the process ends; the address is
 * looked up on a device's first call).  The call allocates nothing.
 * Arguments whose partials (ra_decode_fwd_workspace_size) exceed 32 MiB are
 * rejected with RA_ERR_UNSUPPORTED; the 1M-token cache with 32 query heads
 * over 8 K/V heads and 4 new tokens needs about 2 MiB.  Every call on a GPU
 * uses that GPU's one array, so calls that overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller;
 * nothing in the array needs to start at zero.
 * Errors: as ra_decode_fwd, except RA_ERR_WORKSPACE.
 */
ra_status ra_decode_fwd_noalloc(const ra_decode_args *a, ra_stream stream);

/*
 * ra_causal_work -- per-rank count of allowed causal (query, key) pairs over
 * the whole ring, W[r] for r < R (host int64 array of R entries), from the
 * same block classification the kernels use ([ZZ]: the interleaved layout
 * exists to even out this count across ranks).  Host-only, synchronous.
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_SHAPE.
 */
ra_status ra_causal_work(int32_t layout, int64_t S, int32_t R, int64_t *W);

/*
 * ra_cached_events -- diagnostic: how many HIP events the library holds.  The
 * ring drivers lease their events from a per-device cache behind a mutex and
 * hand them back when the call returns, so the count grows only with the
 * number of ring calls that ever ran at the same time, never per call or per
 * host thread.  Host-only.
 */
size_t ra_cached_events(void);

#ifdef __cplusplus
}
#endif
#endif /* RA_H_ */
