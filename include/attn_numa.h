/*
 * attn_numa: NUMA-aware FlashAttention-2 style attention forward for MI355X
 * (gfx950), C ABI.
 *
 * The operation is scaled dot-product attention, S = Q K^T, P = softmax(S /
 * sqrt(d)), O = P V, per head ("Optimizing Attention on GPUs by Exploiting GPU
 * Architectural NUMA Effects", digest page, §4 equation), computed by one
 * workgroup per (batch, query head, row block of attn_block_m() rows) that
 * streams all of that head's K and V with an online softmax (same page, §3
 * Figure 4).  Which
 * workgroup takes which row block is set by one of four workgroup-ID remaps
 * (same page, §2 Q2, §3 Figure 10 and the before/after table, §7 Figures 3
 * and 11).
 *
 * Conventions for every entry point:
 *   - Return value: 0 on success, a negative ATTN_E* code otherwise; nothing
 *     is launched when validation fails.  attn_strerror(code) describes it.
 *   - No entry point allocates, frees or synchronises device memory.  The
 *     caller owns every buffer.  Device work is enqueued on `stream` (a
 *     hipStream_t; NULL = the null stream) and the call returns once it is
 *     enqueued.
 *   - Thread-safe: the only shared state is a per-device cache of device
 *     attributes filled on first use.
 */
#ifndef ATTN_NUMA_H
#define ATTN_NUMA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define ATTN_OK 0
#define ATTN_E_NULL (-1)        /* a required pointer is NULL */
#define ATTN_E_SHAPE (-2)       /* B, H_Q, H_KV or N <= 0, H_Q % H_KV != 0,
                                   or a size beyond the 32-bit limits below */
#define ATTN_E_HEAD_DIM (-3)    /* d <= 0, d > 128 or d % 8 != 0 */
#define ATTN_E_MAPPING (-4)     /* mapping not in 0..15 */
#define ATTN_E_ALIGN (-5)       /* a device pointer is not 16-byte aligned */
#define ATTN_E_HIP (-6)         /* HIP runtime or launch error */
#define ATTN_E_NO_DEVICE (-7)   /* no HIP device is visible */
#define ATTN_E_SCRATCH (-8)     /* attn_fwd_split_noalloc: the workspace would
                                   not fit ATTN_SCRATCH_BYTES */

/* Workgroup remap modes (digest page §3 before/after table, §5). */
#define ATTN_MAP_NAIVE_BLOCK_FIRST 0    /* id order, heads fastest */
#define ATTN_MAP_NAIVE_HEAD_FIRST 1     /* id order, row blocks fastest */
#define ATTN_MAP_SWIZZLED_BLOCK_FIRST 2 /* chiplet swizzle, heads fastest */
#define ATTN_MAP_SWIZZLED_HEAD_FIRST 3  /* chiplet swizzle, blocks fastest:
                                           one ACC per XCD at a time */
/* Added to any mode: row blocks from the last to the first (longest first
   under a causal mask) and, in head-first order, the query heads of an ACC
   that share a row block adjacent.  Not on the pages: concurrent workgroups
   of a causal ACC then stay close together in the K/V stream, which keeps
   the swizzled head-first L2 hit rate up (measured in the design notes). */
#define ATTN_MAP_LONGEST_FIRST 4
/* Added to ATTN_MAP_SWIZZLED_HEAD_FIRST (ignored by the other modes): the
   work-balanced fallback.  The pages leave open what happens when the XCD
   count does not divide the ACC count (digest §7, key implementation
   details, item 1; the commentary page's H_Q = 12 example).  It acts only
   on XCDs whose slice holds part of an ACC that a slice boundary splits,
   and keeps every XCD's ACCs: a split ACC's (row block, head) units are laid
   out in folded order (longest, shortest, second longest, ...) before the
   slices cut it, so under a causal mask each XCD's share of the work is
   within one row block of the mean; and on such an XCD a piece runs merged
   with the adjacent whole ACC, longest row block first, so the XCD's
   longest workgroups do not start last. */
#define ATTN_MAP_BALANCED_SPLIT 8

/*
 * attn_fwd: attention forward pass.
 *
 * Passage: digest page §4 equation (the result) and §3 Figure 4 (the
 * row-block tiling: one workgroup per attn_block_m() = 256 query rows of a
 * head, reading all of that head's K and V).
 *
 *   q    device, bf16 [B][H_Q][N][d], contiguous, read only
 *   k    device, bf16 [B][H_KV][N][d], contiguous, read only
 *   v    device, bf16 [B][H_KV][N][d], contiguous, read only
 *   o    device, bf16 [B][H_Q][N][d], contiguous, written (every element)
 *   lse  device, fp32 [B][H_Q][N], written, may be NULL: natural-log
 *        logsumexp of the scaled (and masked) scores of each query row
 *   B, H_Q, H_KV, N, d   shape; H_Q % H_KV == 0; query head h reads KV head
 *        h / (H_Q / H_KV); 8 <= d <= 128 with d % 8 == 0 (d <= 64 runs a
 *        64-wide tile, else a 128-wide one); B*H_Q*ceil(N/256) < 2^31 and
 *        N*d*2 <= 2^31 - 2^16 bytes per head
 *   causal  0: every key; 1: query row i sees keys 0..i (top-left aligned)
 *   mapping ATTN_MAP_* (0..3), optionally | ATTN_MAP_LONGEST_FIRST and/or
 *          | ATTN_MAP_BALANCED_SPLIT (0..15); the XCD count used is
 *          attn_num_xcd()
 *   stream  hipStream_t or NULL
 *
 * Arithmetic: bf16 inputs, fp32 scores, softmax statistics and accumulators;
 * P is rounded to bf16 (nearest-even) before P V; O is rounded to bf16.
 * O and lse do not depend on `mapping` (bit-identical across modes).
 * Errors: ATTN_E_NULL (q, k, v or o NULL), ATTN_E_SHAPE, ATTN_E_HEAD_DIM,
 * ATTN_E_MAPPING, ATTN_E_ALIGN (q, k, v, o or lse), ATTN_E_NO_DEVICE,
 * ATTN_E_HIP (launch failed; attn_strerror(ATTN_E_HIP) has the HIP text).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H_Q, int H_KV, int N, int d, int causal, int mapping,
             void* stream);

/*
 * attn_fwd_split: attention of N_q query rows over N_kv keys, optionally with
 * the keys split into num_splits ranges computed by separate workgroups and
 * merged (split-KV, e.g. decode with N_q = 1).
 *
 * Passage: the per-head attention of attn_fwd (digest page §4 equation, §3
 * Figure 4); the split and merge are the decode reduction of the "Fused
 * Grouped-Query Attention" page (each shard computes attention over its KV
 * range; the partial results are reduced into the output), in (O, lse) form:
 * lse = ln sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
 *
 *   q, o   device, bf16 [B][H_Q][N_q][d];  k, v  device, bf16 [B][H_KV][N_kv][d]
 *   lse    device, fp32 [B][H_Q][N_q] or NULL
 *   causal 1: bottom-right aligned, query row i sees keys 0 .. i + N_kv - N_q
 *          (the attn_fwd mask when N_q == N_kv; every key when N_q == 1).
 *          A row that sees no key gets O = 0 and lse = -inf.
 *   num_splits >= 1.  Split s covers keys [s c, min((s+1) c, N_kv)) with
 *          c = attn_split_chunk(N_kv, num_splits); a split past the keys is
 *          empty.  With num_splits == 1 the result goes straight to o and lse
 *          and o_ws, lse_ws are ignored (may be NULL); then the call equals
 *          attn_fwd when N_q == N_kv (bit-identical).
 *   o_ws   device, fp32 [num_splits][B][H_Q][N_q][d], caller-owned workspace:
 *          split s's output normalised over its keys (0 for rows that see
 *          none of them).  Used when num_splits > 1.
 *   lse_ws device, fp32 [num_splits][B][H_Q][N_q]: split s's natural-log
 *          logsumexp (-inf for rows that see none of its keys).
 *   Other arguments and limits as attn_fwd (N_q and N_kv each obey N's
 *   limits; B*H_Q*ceil(N_q/256)*num_splits < 2^31).
 * Launches the attention kernel, then (num_splits > 1) the merge kernel, on
 * `stream`.  Errors: as attn_fwd; ATTN_E_NULL also for a NULL workspace with
 * num_splits > 1, ATTN_E_ALIGN for a misaligned one.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int H_Q, int H_KV, int N_q, int N_kv,
                   int d, int causal, int num_splits, float* o_ws,
                   float* lse_ws, int mapping, void* stream);

/*
 * attn_fwd_split_noalloc: attn_fwd_split without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * The same computation and kernels as attn_fwd_split (results are
 * bit-identical to it); the split partials (o_ws, lse_ws of attn_fwd_split)
 * live in a fixed device array of ATTN_SCRATCH_BYTES that the library owns:
 * each GPU it runs on holds one such array from the first call on that GPU
 * until the process ends.  The call itself allocates nothing (no hipMalloc,
 * no allocating library routine).
 *
 *   q, k, v, o, lse, B, H_Q, H_KV, N_q, N_kv, d, causal, num_splits,
 *   mapping, stream   as attn_fwd_split.
 * Needs num_splits * B * H_Q * N_q * (d + 1) * 4 bytes (rounded up to 256
 * between the two parts) <= ATTN_SCRATCH_BYTES when num_splits > 1; larger
 * calls return ATTN_E_SCRATCH before touching the device.  Every call
 * overwrites all of the scratch it uses before reading it, so nothing has to
 * be cleared between calls; calls that overlap on one GPU (e.g. on two
 * streams) share the array and race, so the caller serialises them.
 * Errors: as attn_fwd_split; ATTN_E_SCRATCH; ATTN_E_HIP also when the
 * array's device address cannot be obtained.
 */
#define ATTN_SCRATCH_BYTES (32 * 1024 * 1024)
int attn_fwd_split_noalloc(const void* q, const void* k, const void* v,
                           void* o, float* lse, int B, int H_Q, int H_KV,
                           int N_q, int N_kv, int d, int causal,
                           int num_splits, int mapping, void* stream);

/*
 * attn_split_chunk: keys per split for attn_fwd_split, ceil(N_kv /
 * num_splits) rounded up to a multiple of 32 (whole key tiles).  Needs no
 * GPU.  Errors: ATTN_E_SHAPE for N_kv <= 0 or num_splits < 1.
 */
int attn_split_chunk(int N_kv, int num_splits);

/*
 * attn_merge: merge num_splits partial results into one (the same reduction
 * as attn_fwd_split; also usable for partial results computed elsewhere,
 * e.g. per device).
 *
 *   o_parts   device, fp32 [num_splits][B][H_Q][N_q][d], read only
 *   lse_parts device, fp32 [num_splits][B][H_Q][N_q] (natural log; -inf for
 *             a part with no keys), read only
 *   o         device, bf16 [B][H_Q][N_q][d], written
 *   lse       device, fp32 [B][H_Q][N_q], written, may be NULL
 * A row whose parts are all -inf gets O = 0 and lse = -inf.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_HEAD_DIM, ATTN_E_ALIGN,
 * ATTN_E_NO_DEVICE, ATTN_E_HIP.
 */
int attn_merge(const float* o_parts, const float* lse_parts, int num_splits,
               int B, int H_Q, int N_q, int d, void* o, float* lse,
               void* stream);

/*
 * attn_bwd: gradients dQ, dK, dV of sum(dO * O) for the attention of
 * attn_fwd (FlashAttention-2 style: P is recomputed from q, k and the
 * forward's lse), with the same workgroup remap as the forward pass.
 *
 * Passage: digest page, Q3 results table and the §3 "Backward pass"
 * paragraph (the paper's Figure 16: the remaps applied to FA2's backward
 * kernel); the equations are the chain rule of the §4 equation:
 * dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with D = rowsum(dO * O),
 * dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d); with GQA a KV head's dK, dV
 * sum over its query heads.
 *
 *   q, o, dout  device, bf16 [B][H_Q][N][d], read only (o: attn_fwd's output)
 *   k, v        device, bf16 [B][H_KV][N][d], read only
 *   lse         device, fp32 [B][H_Q][N], read only: attn_fwd's lse (natural log)
 *   dq          device, bf16 [B][H_Q][N][d], written (every element)
 *   dk, dv      device, bf16 [B][H_KV][N][d], written (every element)
 *   ws          device, fp32 [B][H_Q][2][N], caller-owned workspace: per
 *               (batch, query head) -lse * log2(e) of its rows, then -D
 *               (minus rowsum(dO * O)); overwritten
 *   B, H_Q, H_KV, N, d, causal   as attn_fwd (the same mask); also
 *               B*H_Q*ceil(N/128) < 2^31
 *   mapping     ATTN_MAP_* (0..15) as attn_fwd: the dK/dV kernel maps
 *               (batch, KV head, 128-key block) with the remap's row blocks
 *               counted from the last key block (the fewest query rows under
 *               a causal mask), the dQ kernel (batch, query head, 128-row block)
 *   stream      hipStream_t or NULL
 * Launches three kernels on `stream` (D and lse2 per row; dK and dV; dQ).
 * Arithmetic: bf16 inputs, fp32 scores and accumulators; P and dS are rounded
 * to bf16 (nearest-even) before the products that use them; outputs are
 * rounded to bf16.  Deterministic: every output element is reduced by one
 * workgroup in a fixed order, so results do not depend on `mapping`.
 * Errors: ATTN_E_NULL (any pointer NULL), ATTN_E_SHAPE, ATTN_E_HEAD_DIM,
 * ATTN_E_MAPPING, ATTN_E_ALIGN (any pointer), ATTN_E_NO_DEVICE, ATTN_E_HIP.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* lse, void* dq, void* dk, void* dv,
             float* ws, int B, int H_Q, int H_KV, int N, int d, int causal,
             int mapping, void* stream);

/*
 * attn_wg_map: the remap table the kernel uses, computed on the host.
 *
 * Passage: digest page §2 Q1 (dispatch to XCD w mod X), §2 Q2 and §7
 * Figures 3 and 11 (the swizzles), §3 Figure 10.
 *
 *   out_host  host, int32 [W][3], W = B*H_Q*ceil(N/attn_block_m()); row w
 *             receives the
 *             (batch, query head, row block) that workgroup w computes when
 *             the chip has num_xcd XCDs.  Caller-owned.
 *   num_xcd   >= 1 (pass attn_num_xcd() for the device's value)
 * H_KV is validated like attn_fwd (the ACC structure depends on it) but the
 * table itself does not.  Needs no GPU.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE (also num_xcd < 1), ATTN_E_MAPPING.
 */
int attn_wg_map(int mapping, int B, int H_Q, int H_KV, int N, int num_xcd,
                int32_t* out_host);

/*
 * attn_block_m: query rows per workgroup (the row-block height, 256), so
 * that a caller can size the tables of attn_wg_map and attn_probe_placement:
 * W = B * H_Q * ceil(N / attn_block_m()).  The pages tile rows by 128
 * (digest page §4); 256 rows per workgroup halve the K/V tile traffic per
 * CU on MI355X.  Needs no GPU.
 */
int attn_block_m(void);

/*
 * attn_num_xcd: XCDs of the current device (8 on MI355X in SPX mode), the
 * count attn_fwd swizzles over.
 *
 * Passage: digest page, §2 Q1 (the dispatcher hands workgroup w to XCD
 * w mod X) and §7 Figure 11, where this count is the NUM_XCD constant of
 * the swizzle.  Read from hipDeviceAttributeNumberOfXccs.  The environment
 * variable ATTN_NUM_XCD (an integer 1..64) overrides it.  Returns the count
 * (>= 1) or a negative ATTN_E_* code (ATTN_E_NO_DEVICE without a GPU).
 */
int attn_num_xcd(void);

/*
 * attn_probe_placement: where the hardware ran each workgroup.
 *
 * Launches the attention grid for this shape and mapping with a kernel that
 * does no attention: workgroup w writes, at dev_out[4*w .. 4*w+3], the XCC
 * id register it ran on and the (batch, query head, row block) the remap
 * gives it.  Checks the dispatch model of digest page §2 Q1 on the device.
 *
 *   dev_out  device, int32 [W][4], W as in attn_wg_map, caller-owned.
 * Errors: as attn_fwd (ATTN_E_NULL for dev_out).
 */
int attn_probe_placement(int mapping, int B, int H_Q, int H_KV, int N,
                         int32_t* dev_out, void* stream);

/*
 * attn_strerror: text for an ATTN_E_* code; for ATTN_E_HIP, the calling
 * thread's last HIP error.  The pointer stays valid until the next call on
 * the same thread.
 *
 * Passage: none.  The pages define no host interface; this is the error
 * reporting of the C boundary around the kernels (plain int codes, no
 * exceptions across the ABI).  Unknown codes return a generic text.
 */
const char* attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_NUMA_H */
