/*
 * fa_fwd.h -- C ABI of the MI355X (gfx950) exact-attention forward library
 * (libfa_fwd.so).
 *
 * The operation is the FlashAttention forward pass dissected by the pages
 * "FlashAttention core algorithm: forward pass" (the Hopper kernel's
 * consumer loop: per query tile S = Q K^T, online softmax with the scale
 * folded into softmax_scale_log2, O += P V, then the epilogue's store or
 * store_zero) and "Dissecting the SM_120 Microarchitecture" (section 11.2,
 * FlashAttention bottleneck analysis, Fig. 12).  For every sequence b,
 * query head h and query row i:
 *
 *   g    = h / (heads_q / heads_kv)                      grouped-query heads
 *   A_i  = { j < sk_b : not causal or j <= i + sk_b - sq_b }   bottom-right
 *   s_ij = softmax_scale * q_i . k_j                    (q_descale*k_descale
 *                                                        folded in for fp8)
 *   O_i  = sum_{j in A_i} softmax_j(s_i) v_j             (times v_descale)
 *   LSE_i = ln sum_{j in A_i} exp(s_ij)
 *   A_i empty: O_i = 0, LSE_i = -inf    (the epilogue's store_zero rule)
 *
 * Data types: without descales Q, K, V are bf16; with descales they are OCP
 * fp8 e4m3 ("e4m3fn") codes.  O is always bf16 (round to nearest even), LSE
 * always fp32.
 *
 * Layouts (contiguous, no strides):
 *   Q [total_q][heads_q][head_dim]     K [total_k][heads_kv][head_dim]
 *   V [total_k][heads_kv][head_dim_v]  O [total_q][heads_q][head_dim_v]
 *   LSE [heads_q][total_q]
 *   cu_seqlens == NULL: total_q = batch*seqlen_q, total_k = batch*seqlen_k.
 *   cu_seqlens != NULL: int32[2*(batch+1)]; cu_seqlens[0..batch] are the
 *     query offsets, cu_seqlens[batch+1 .. 2*batch+1] the key offsets of a
 *     packed batch (the page's SeqlenInfo: per-sequence offsets and
 *     lengths); total_q = cu_seqlens[batch], total_k = cu_seqlens[2*batch+1]
 *     (LSE rows are total_q long); seqlen_q / seqlen_k are then the largest
 *     sequence lengths (they size the launch grid).  Offsets must be
 *     non-decreasing, start at 0 and every length must be <= the maximum
 *     passed: the array lives on the device, where fa_fwd does not read it
 *     on the host, so this is the caller's contract -- fa_check_cu_seqlens
 *     checks a host copy of it (the Python binding always does).
 *
 * Ownership: every pointer belongs to the caller; the library allocates no
 * device memory and keeps no per-call state (it caches one device-property
 * query per device).  Calls are asynchronous on `stream`; a device fault
 * surfaces at the caller's next synchronisation.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Codes FA_ERR_NULL .. FA_ERR_UNSUPPORTED are decided on the
 * host before any HIP call. */
#define FA_OK 0
#define FA_ERR_NULL (-1)        /* a required pointer is NULL                       */
#define FA_ERR_INVALID (-2)     /* bad sizes, heads_q % heads_kv != 0, bad scale     */
#define FA_ERR_UNSUPPORTED (-3) /* head_dim not in {64,128}, head_dim_v != head_dim,
                                   or no tile plan fits the device                   */
#define FA_ERR_DEVICE (-4)      /* not a gfx950 device, or the launch failed         */

/* Input type selector for the planner (fa_fwd itself infers it from
 * `descales`). */
#define FA_DTYPE_BF16 0
#define FA_DTYPE_E4M3 1

/*
 * fa_fwd -- launch the forward pass on `stream` (a hipStream_t; NULL is the
 * null stream).
 *
 *   q, k, v     device pointers, layouts above (bf16, or e4m3 codes when
 *               descales != NULL)
 *   o           device pointer, bf16 [total_q][heads_q][head_dim_v] (output)
 *   lse         device pointer, fp32 [heads_q][total_q] (output)
 *   batch, heads_q, heads_kv   > 0, heads_q % heads_kv == 0
 *   seqlen_q, seqlen_k         >= 0 (maxima when cu_seqlens != NULL)
 *   cu_seqlens  NULL or device int32[2*(batch+1)] (see above)
 *   head_dim, head_dim_v       64 or 128, equal
 *   softmax_scale              finite and > 0 (usually 1/sqrt(head_dim))
 *   causal      0: every key of the sequence; 1: bottom-right causal mask
 *   descales    NULL (bf16 inputs) or device float[3] = {q, k, v} descale
 *               factors of e4m3 inputs: q*k descale multiplies the scores,
 *               v descale the output
 *
 * q, o and lse may be NULL only when seqlen_q == 0, k and v only when
 * seqlen_k == 0 (for a packed batch these are the maxima, so no sequence has
 * a query row, or a key, to read).
 *
 * Returns FA_OK or a negative code (fa_strerror).  Rows of a sequence with
 * no admissible key get O = 0 and LSE = -inf; nothing is written for
 * sequences with no query.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
           int heads_q, int heads_kv, int seqlen_q, int seqlen_k, const int* cu_seqlens,
           int head_dim, int head_dim_v, float softmax_scale, int causal, const float* descales,
           void* stream);

/* Text for a return code (static storage, never NULL).  FA_ERR_UNSUPPORTED
 * is the answer of the tile screen ("FlashAttention on SM120 reusing the SM80
 * forward", section on can_implement: a configuration whose buffers do not
 * fit is refused before launch); rows without an admissible key are not an
 * error but the epilogue's store_zero case ("FlashAttention core algorithm:
 * forward pass", epilogue). */
const char* fa_strerror(int code);

/*
 * fa_check_cu_seqlens -- host-side check of a packed batch's offsets (the
 * contract stated with the layouts above), on a HOST copy of the int32
 * array of 2*(batch+1) entries:
 *   cu[0] == 0 and cu[batch+1] == 0; both halves non-decreasing;
 *   every query length cu[b+1]-cu[b] <= seqlen_q, every key length
 *   cu[batch+2+b]-cu[batch+1+b] <= seqlen_k;
 *   cu[batch] == rows_q (the rows of Q, O and of each LSE row) and
 *   cu[2*batch+1] <= rows_k (the rows of K and V).
 * Pure host function.  Returns FA_OK, FA_ERR_NULL (cu_host NULL) or
 * FA_ERR_INVALID (batch <= 0, negative sizes, or a violated condition).
 * A call that passes this check cannot make fa_fwd read or write outside
 * Q/K/V/O/LSE buffers of those row counts.
 */
int fa_check_cu_seqlens(const int* cu_host, int batch, int seqlen_q, int seqlen_k,
                        int64_t rows_q, int64_t rows_k);

/* ---- KV cache ------------------------------------------------------------ */

/*
 * fa_fwd_kvcache -- append new keys/values to a KV cache, then run the
 * forward pass over the cache: the AppendKV step of "FlashAttention core
 * algorithm: forward pass" (the producer loop loads the new K/V before the
 * tile's K/V when AppendKV is enabled), read as the usual cached forward:
 *
 *   1. for every sequence b and j < seqlen_new, rows k_new[b][j] and
 *      v_new[b][j] are copied to k_cache[b][cache_seqlens[b] + j] and
 *      v_cache[b][cache_seqlens[b] + j] (positions outside
 *      [0, cache_capacity) are skipped);
 *   2. fa_fwd over Q [batch][seqlen_q][heads_q][head_dim] (fixed length) and
 *      the first sk_b = clamp(cache_seqlens[b] + seqlen_new, 0,
 *      cache_capacity) rows of sequence b's cache, with bottom-right causal
 *      alignment when causal = 1 (the last query sees the last key).
 *
 *   k_cache, v_cache   device, [batch][cache_capacity][heads_kv][head_dim]
 *                      (bf16, or e4m3 codes when descales != NULL); updated
 *                      in place
 *   k_new, v_new       device, [batch][seqlen_new][heads_kv][head_dim]
 *   cache_seqlens      device int32[batch]: rows already in each cache
 *                      (read, not updated: the caller advances it)
 *   q, o, lse, batch, heads, head dims, softmax_scale, causal, descales
 *                      as for fa_fwd, with total_q = batch * seqlen_q
 *
 * The append runs as its own kernel on `stream` before the attention
 * kernel.  Returns FA_OK or a negative code; argument errors are reported
 * before anything is launched or written.  k_new / v_new may be NULL when
 * seqlen_new == 0, the caches when cache_capacity == 0.
 */
int fa_fwd_kvcache(const void* q, void* k_cache, void* v_cache, const void* k_new,
                   const void* v_new, void* o, float* lse, int batch, int heads_q, int heads_kv,
                   int seqlen_q, int seqlen_new, int cache_capacity, const int* cache_seqlens,
                   int head_dim, int head_dim_v, float softmax_scale, int causal,
                   const float* descales, void* stream);

/* ---- tile / occupancy screening (host functions) -------------------------- */

/*
 * Capacity figures of a device, as the shared-memory screen of "FlashAttention
 * on SM120 reusing the SM80 forward" (section on can_implement and the
 * appendix table of per-SM / per-block shared memory) uses them.  On gfx950
 * the "shared memory" is the LDS: 160 KiB per compute unit, all of it
 * available to one workgroup.
 */
typedef struct fa_device_limits {
  int64_t lds_bytes_per_block; /* largest allocation one workgroup may hold  */
  int64_t lds_bytes_per_cu;    /* total shared by resident workgroups        */
  int num_cus;                 /* compute units (SMs)                         */
  int simds_per_cu;            /* 4 on gfx950                                 */
  int regs_per_simd_lane;      /* VGPR+AGPR per lane per SIMD (512 on gfx950) */
  int max_waves_per_simd;      /* hardware wave slots per SIMD                */
} fa_device_limits_t;

/* One candidate tile configuration, in the page's terms. */
typedef struct fa_tile_config {
  int tile_m;      /* query rows per block                                */
  int tile_n;      /* keys per main-loop step                             */
  int head_dim;    /* D                                                   */
  int head_dim_v;  /* Dv                                                  */
  int elem_bytes;  /* bytes per Q/K/V element (2 bf16, 1 fp8)             */
  int kv_stages;   /* K/V buffers (1 single-stage, 2 double-stage)        */
  int q_in_regs;   /* 1: Q lives in registers after the prologue, so its
                      buffer shares space with V (max instead of sum)     */
} fa_tile_config_t;

typedef struct fa_screen {
  int64_t smem_bytes; /* Q + stages*(K + V), or K*stages + max(Q, V*stages) */
  int fits;           /* smem_bytes <= lds_bytes_per_block                  */
  int blocks_per_cu;  /* floor(lds_bytes_per_cu / smem_bytes) when it fits  */
} fa_screen_t;

/* The page's byte accounting and fit verdict for one configuration.
 * Returns FA_OK, FA_ERR_NULL or FA_ERR_INVALID (non-positive sizes). */
int fa_smem_screen(const fa_tile_config_t* cfg, const fa_device_limits_t* dev, fa_screen_t* out);

/* The gfx950 (MI355X) figures used when a planner call passes dev == NULL. */
int fa_gfx950_limits(fa_device_limits_t* out);

/* The plan fa_fwd would launch for a shape. */
typedef struct fa_plan {
  int tile_m;            /* query rows per workgroup                          */
  int tile_n;            /* keys per main-loop iteration                      */
  int waves;             /* wavefronts per workgroup                          */
  int kv_stages;         /* LDS buffers for K/V                               */
  int64_t lds_bytes;     /* LDS per workgroup, as the kernel lays it out      */
  int wg_per_cu;         /* resident workgroups per CU (LDS and VGPR limits)  */
  int vgprs_per_lane;    /* VGPR+AGPR budget per lane the kernel is built for */
  int64_t num_workgroups;/* grid size                                         */
  int m_tiles;           /* query tiles (tile_m rows) per (sequence, head)    */
  int kernel_variant;    /* index of the compiled kernel                      */
  int query_tiles;       /* 32-row query tiles per wave                       */
  int heads_per_workgroup; /* query heads sharing one workgroup's K/V staging  */
  int schedule;          /* 1 to 5 (see fa_fwd_plan)                          */
} fa_plan_t;

/*
 * fa_fwd_plan -- choose the kernel configuration for a shape: the
 * can_implement screen of "FlashAttention on SM120 reusing the SM80 forward"
 * (buffers against the per-block and per-CU shared-memory capacity, blocks per
 * CU) carried on to gfx950's LDS and register file, plus the choice of
 * schedule.  Host function, no HIP call; its inputs are the arguments and the
 * process-wide schedule override of fa_set_schedule (0, the default, leaves
 * the choice to the rules below).  dev == NULL means gfx950.  Returns FA_OK,
 * FA_ERR_NULL, FA_ERR_INVALID or FA_ERR_UNSUPPORTED (nothing fits `dev`).
 *
 * Schedules:
 *   1  4 waves, one 32-row query tile each: 128 rows of one query head per
 *      workgroup, two waves per SIMD (every shape, bf16 and fp8);
 *   2  bf16: 4 waves with two query tiles each: 256 rows of one head, one wave
 *      per SIMD holding the full register file, every LDS operand read
 *      feeding two matrix instructions;
 *   3  bf16, heads_q / heads_kv even, or odd for fixed lengths (varlen ==
 *      0): 8 waves in two groups of four, 128 rows of two query heads that
 *      share a KV head, or (odd heads_q / heads_kv, e.g. 1) two adjacent
 *      128-row query tiles of one head (tile_m 256),
 *      one K/V staging for both groups, the groups alternating matrix-core
 *      and softmax phases (ping-pong);
 *   4  bf16, heads_q / heads_kv * seqlen_q <= 32 (decode): the (query head,
 *      row) pairs of one KV head in the 32 columns of one tile, one workgroup
 *      per (sequence, KV head) whose 4 waves split the key range and merge
 *      their partial softmax states at the end;
 *   5  forced only, where 3 applies: schedule 3's work items walked by
 *      resident workgroups (a persistent launch: num_workgroups = the CUs, a
 *      whole number per XCD, at most the number of items), each taking its
 *      XCD's items in the order of schedule 3's grid, zig-zag in windows of
 *      twice the workgroups per XCD, and loading the next item's query rows
 *      into an LDS stage (lds_bytes includes it) during the current item --
 *      the persistent tile scheduler of "FlashAttention core algorithm:
 *      forward pass" (producer loop: the next work tile fetched before the
 *      epilogue).  It computes what schedule 3 computes; it measures slower
 *      on gfx950, where the hardware dispatcher already hands out schedule
 *      3's workgroups heaviest first as CUs free up.
 * The plan uses 4 where it applies, else 3 where it applies, head_dim is 128
 * and its grid has at least one workgroup per CU (`dev->num_cus`; smaller
 * grids finish first on schedule 1's finer tiles; without causal masking,
 * more than half a workgroup per CU suffices), from 2048 query rows (1024
 * without causal masking)
 * unless its grid is a single round (one workgroup per CU), with tile pairs
 * under causal masking only from 6144 query rows or for a single round, and
 * not for a single causal round over at most 8 (sequence, KV head) pairs;
 * else 1, unless fa_set_schedule forces one.
 */
int fa_fwd_plan(int dtype, int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                int varlen, int head_dim, int head_dim_v, int causal,
                const fa_device_limits_t* dev, fa_plan_t* out);

/*
 * fa_set_schedule -- tuning override of the planner's schedule choice (for
 * benchmarking and for tests that run every schedule on the same shapes).
 * 0 restores the automatic choice; 1, 2, 3, 4 or 5 forces that schedule in every
 * later fa_fwd / fa_fwd_kvcache / fa_fwd_plan call of the process wherever it
 * applies (schedule 1 elsewhere).  All schedules compute the same function to
 * within rounding, but not bit for bit: the reference maximum that the
 * softmax rescales against is updated per wave, and waves hold different rows
 * in different schedules.  The setting is a process-wide atomic; calls already
 * launched are unaffected.  Returns FA_OK, or FA_ERR_INVALID for any other
 * value.
 */
int fa_set_schedule(int schedule);

/*
 * fa_set_exp2_offload -- exp2 offload ("Dissecting the SM_120
 * Microarchitecture", section 11.2, Fig. 12, first remedy for the
 * softmax-bound tile): in the ping-pong schedule (3), evaluate every 4th or
 * 8th exponential of P with a Cody-Waite reduction and a degree-3 polynomial
 * on the FMA pipe instead of the transcendental unit (relative error below
 * 7.5e-5, under the bf16 rounding of P).  0 (the default) turns it off.  On
 * gfx950 it measures slower (the vector ALU, not the transcendental unit, is
 * the contended resource), so it is a tuning and study switch.  Process-wide
 * atomic like fa_set_schedule.  Returns FA_OK, or FA_ERR_INVALID for values
 * other than 0, 4 and 8.
 */
int fa_set_exp2_offload(int every);

/*
 * fa_set_fp8_exact_scores -- precision switch of the e4m3 path.  The pages fold
 * the q and k descales into the exp2 scale and run S = Q K^T on the fp8
 * tensor unit ("FlashAttention core algorithm: forward pass", FP8 branch of
 * the consumer loop).  gfx950's fp8 matrix instruction keeps only about
 * 13-14 bits below the largest product of each dot product it sums, so a row
 * whose few largest scores come from products far above the others (scores
 * of about 50 and more) carries an LSE error of about 1e-4 of those scores.
 * 1 runs S = Q K^T on the bf16 matrix instruction instead, from Q and K
 * widened exactly from e4m3 to bf16 (P V stays on fp8); 0 (the default)
 * keeps the fp8 product.  Same results otherwise; slower (the widening of
 * every K operand runs on the vector ALU, and the bf16 product at half the
 * fp8 rate).  Process-wide atomic like fa_set_schedule; calls already
 * launched are unaffected.  Returns FA_OK, or FA_ERR_INVALID for values
 * other than 0 and 1.
 */
int fa_set_fp8_exact_scores(int on);

/* Library version: major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
