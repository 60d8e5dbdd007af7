/*
 * mha_fwd.h -- C ABI of the fused multi-head-attention forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  For every sequence b of a ragged batch, every query head
 * h and every query row i of that sequence:
 *
 *     S[i, j] = sigma * (q[i, h, :Dn] . k[j, g, :Dn] + q_rope[i, h, :] . k_rope[j, g, :])
 *     O[i, h, :] = sum_j softmax_j(S[i, .]) v[j, g, :]          over visible keys j
 *     LSE[h, i] = ln sum_j exp(S[i, j])                          over visible keys j
 *
 * with g = h / (num_heads / num_kv_heads) (grouped-query attention) and key j
 * visible to query i iff j < L_b and, when causal, j <= i (indices local to
 * the sequence; queries and keys share one length per sequence).
 *
 * The pages this follows (the Modular API pages "SM100AttentionSMem",
 * "TMAProducerPipeline" and "MHATileScheduler" for an SM100 flash-attention
 * kernel) give the pieces: Q/K split into a "nope" part and a separately
 * typed "rope" part and an optional per-token scale for Q and K
 * (SM100AttentionSMem, Parameters); per-batch sequence-length offsets
 * (MHATileScheduler, Required methods: get_current_work_info); a per-row
 * correction buffer for the online softmax (SM100AttentionSMem, Methods:
 * correction_smem).  The signature itself is this library's own.
 *
 * Conventions for every entry point below:
 *   - tensor pointers are DEVICE pointers to contiguous, token-major ("THD")
 *     arrays; the caller owns them; the library keeps no reference after the
 *     call returns;
 *   - calls are asynchronous on `stream` (a hipStream_t, passed as void*;
 *     NULL = the null stream); outputs are valid once the stream reaches
 *     them;
 *   - on any nonzero status nothing has been launched and the outputs are
 *     untouched; mha_fwd_last_error() returns a message for the calling
 *     thread's last nonzero status.
 */
#ifndef MHA_FWD_H_
#define MHA_FWD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  F32: q, k, v, q_rope, k_rope and o are float32.
 * BF16: all of them are bfloat16.  FP8_E4M3: q and k are OCP E4M3 codes
 * ("fn", largest finite 448) with float32 per-token scales; v, o are
 * bfloat16 (SM100AttentionSMem, Parameters: qkv_dtype, scale_dtype_).
 * FP8_E4M3 decodes the codes to bfloat16 (exactly) for the Q K^T products,
 * which the bf16 matrix instruction sums with float32-grade accuracy.
 * FP8_E4M3_FASTACC takes the same inputs but runs Q K^T on the fp8 matrix
 * instruction at twice the rate; that instruction sums its 64 products
 * keeping only about 13 bits below the largest one (measured on gfx950:
 * error up to 2^-13 of the sum of the products' magnitudes), so a score
 * can be off by about 1e-4 of sigma * sum_d |q_d k_d|, and the LSE of rows
 * with large scores by more than 1e-3. */
typedef enum {
  MHA_DTYPE_F32 = 0,
  MHA_DTYPE_BF16 = 1,
  MHA_DTYPE_FP8_E4M3 = 2,
  MHA_DTYPE_FP8_E4M3_FASTACC = 3
} mha_dtype_t;

typedef enum {
  MHA_OK = 0,
  MHA_ERR_INVALID_ARG = 1,  /* a pointer, size or flag is malformed            */
  MHA_ERR_UNSUPPORTED = 2,  /* (dtype, Dn, Dr, Dv) outside the compiled set      */
  MHA_ERR_HIP = 3           /* a HIP runtime call or launch failed               */
} mha_status_t;

/*
 * mha_fwd -- O and LSE for a ragged batch of sequences.
 *
 *   q           [T, num_heads, head_dim_nope]      element type per `dtype`
 *   k           [T, num_kv_heads, head_dim_nope]
 *   v           [T, num_kv_heads, v_dim]           float32 (F32) or bfloat16
 *   o           [T, num_heads, v_dim]   written;   float32 (F32) or bfloat16
 *   lse         [num_heads, T] float32, written;   natural log, softmax scale
 *               included
 *   cu_seqlens  [batch + 1] int32: cu_seqlens[0] = 0, nondecreasing, the
 *               token offset of each sequence (MHATileScheduler, Required
 *               methods: the optional pointer of per-batch sequence length
 *               offsets).  T = cu_seqlens[batch].  Not checked on the host
 *               (that would need a device sync).
 *   batch       number of sequences, >= 1
 *   max_seqlen  >= every sequence length; sizes the work table (num_heads *
 *               batch * ceil(max_seqlen / block_m) entries, block_m = 32
 *               for float32 and 256 for bf16 / fp8).  0 means every
 *               sequence is empty: the scalar arguments are still checked,
 *               but nothing is read, written or launched and the tensor
 *               pointers may be NULL.  When a length breaks this bound, the
 *               device refuses the whole call and writes nothing (O and LSE
 *               keep what they held; the status is only visible on the
 *               device, as the lengths are not read on the host).
 *   num_heads, num_kv_heads   query and key/value heads; num_heads must be a
 *               multiple of num_kv_heads
 *   head_dim_nope, head_dim_rope, v_dim   Dn, Dr (0 = no rope part), Dv
 *   q_rope      [T, num_heads, head_dim_rope], k_rope [T, num_kv_heads,
 *               head_dim_rope]: the rope part of Q and K, already rotated,
 *               bfloat16 (float32 for F32; bfloat16 also under FP8_E4M3,
 *               where q_scale / k_scale scale the nope product only:
 *               S = sigma (q_scale k_scale q_nope . k_nope + q_rope . k_rope)).
 *               NULL iff head_dim_rope == 0 (SM100AttentionSMem, Parameters:
 *               rope_dtype_, its own element type; Methods: q_rope_smem).
 *   causal      0: every key of the sequence is visible; 1: key j visible to
 *               query i iff j <= i
 *   softmax_scale  sigma; <= 0 selects 1/sqrt(head_dim_nope + head_dim_rope)
 *   dtype       an mha_dtype_t
 *   q_scale     [T, num_heads] float32, k_scale [T, num_kv_heads] float32:
 *               dequantisation scales, value = code * scale, one per (token,
 *               head) row, >= 0 (SM100AttentionSMem, Methods: q_scale_smem,
 *               k_scale_smem).  Required iff dtype is FP8_E4M3 or
 *               FP8_E4M3_FASTACC, else NULL.
 *   stream      hipStream_t or NULL
 *
 * Alignment: q, k, v, o, q_rope and k_rope must be 16-byte aligned (the
 * kernels move them in 16-byte units), lse, cu_seqlens, q_scale and k_scale
 * 4-byte aligned; MHA_ERR_INVALID_ARG otherwise (checked on the host, before
 * any HIP call).
 *
 * Compiled set (MHA_ERR_UNSUPPORTED otherwise):
 *   F32      (Dn, Dr, Dv) in {(64,0,64), (128,0,128), (128,64,128)}
 *   BF16     (Dn, Dr, Dv) in {(64,0,64), (128,0,128), (128,64,128)}
 *   FP8_E4M3, FP8_E4M3_FASTACC  (Dn, Dr, Dv) in {(128,0,128), (128,64,128)}
 *
 * Key splits of its own (BF16 and FP8_E4M3): where the longest work items
 * would set the run time (few, long items for the device's CUs, e.g. one
 * long causal sequence with few heads), mha_fwd runs them as
 * mha_fwd_splitkv would, with mha_fwd_auto_splits(batch, max_seqlen,
 * num_heads, causal, v_dim, CUs) key ranges and the partials in its
 * workspace (O rounded to bfloat16, LSE in float32), and merges them; O and
 * LSE agree with the unsplit run up to that rounding of the partial O and
 * float32 rounding of the merge.  Never with fewer than 16 key blocks
 * (max_seqlen <= 960).
 *
 * Small float32 calls (batch <= 64, and no more (sequence, head, q-tile)
 * items of the max_seqlen grid than one full launch has workgroups) skip the
 * scheduler: workgroup i takes item i directly, with no prepass launch and
 * no workspace; the refusal above holds the same.
 *
 * The library owns a workspace per (device, stream): the work table and
 * queue counters of the persistent scheduler, and the partials of its own
 * key splits.  It is allocated on the first call for that pair (so the first
 * call must not be inside a HIP graph capture) and grown when a larger
 * problem arrives.  Calls on one stream are ordered and may follow each other
 * freely; calls on two streams use two workspaces.
 */
int mha_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
            int32_t num_heads, int32_t num_kv_heads,
            int32_t head_dim_nope, int32_t head_dim_rope, int32_t v_dim,
            const void* q_rope, const void* k_rope,
            int32_t causal, float softmax_scale, int32_t dtype,
            const float* q_scale, const float* k_scale, void* stream);

/*
 * mha_fwd_noalloc -- mha_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as mha_fwd, except:
 *
 *   - the scheduler workspace is a fixed 16 MiB device array inside the
 *     library (one copy per GPU, held until the process ends), so no call
 *     allocates or frees device memory; a call whose work table would not
 *     fit (16 bytes per work item -- num_heads * batch * ceil(max_seqlen /
 *     block_m), block_m 256 for bf16 / fp8 and 32 for float32 -- plus 4 bytes
 *     per (sequence, KV head) and 2.3 KB) returns MHA_ERR_INVALID_ARG with a
 *     message giving both sizes, before any launch;
 *   - it never splits keys by itself (mha_fwd's own splits keep float32
 *     partials in its allocated workspace); with one split its output is
 *     mha_fwd's bit for bit;
 *   - the first call on a device looks the array up for that device
 *     (hipGetSymbolAddress; no allocation);
 *   - every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (two streams, or two host threads) race and must be ordered by
 *     the caller.  Each call's scheduler prepass rewrites all of the state it
 *     reads, so calls in sequence need no clearing.
 */
int mha_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                    int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim_nope, int32_t head_dim_rope, int32_t v_dim,
                    const void* q_rope, const void* k_rope,
                    int32_t causal, float softmax_scale, int32_t dtype,
                    const float* q_scale, const float* k_scale, void* stream);

/* Message for the calling thread's last nonzero status ("" if none).  The
 * string is owned by the library and valid until the thread's next call. */
const char* mha_fwd_last_error(void);

/* 1 if (dtype, Dn, Dr, Dv) is in the compiled set, else 0.  No HIP call. */
int mha_fwd_supported(int32_t dtype, int32_t head_dim_nope,
                      int32_t head_dim_rope, int32_t v_dim);

/*
 * mha_fwd_kernel_info -- launch facts of the kernel that mha_fwd would use for
 * (dtype, Dn, Dr, Dv) on the current device: *block_m = query rows per work
 * item, *blocks_per_cu = workgroups resident per compute unit (its register
 * and LDS footprint allow), *grid = workgroups of the persistent launch
 * before clamping to the number of work items, *lds_bytes = static LDS per
 * workgroup.  Any output pointer may be NULL.  Returns MHA_ERR_UNSUPPORTED
 * outside the compiled set, MHA_ERR_HIP if the device cannot be queried.
 */
int mha_fwd_kernel_info(int32_t dtype, int32_t head_dim_nope, int32_t head_dim_rope,
                        int32_t v_dim, int32_t* block_m, int32_t* blocks_per_cu,
                        int32_t* grid, int32_t* lds_bytes);

/*
 * Measurement hook.  Registers two hipEvent_t handles (created by the
 * caller, who keeps ownership) that every following mha_fwd call made by the
 * same host thread records on its stream immediately before and after the
 * attention kernel, so that the kernel's own duration can be read without a
 * profiler (the scheduler prepass that precedes it is outside the pair);
 * mha_quantize_fp8 records the same pair around its kernel.
 * NULL, NULL switches the hook off; exactly one NULL is MHA_ERR_INVALID_ARG.
 * A call whose outputs are empty (max_seqlen == 0) records nothing.
 */
int mha_fwd_set_kernel_events(void* start_event, void* stop_event);

/*
 * mha_sched_visit -- diagnostic for the persistent tile scheduler
 * (MHATileScheduler, class description: the scheduler hands out work tiles
 * to workgroups and moves each one on to its next tile).  Builds the work
 * table exactly as mha_fwd
 * does for (cu_seqlens, batch, max_seqlen, num_heads, num_kv_heads, causal,
 * block_m) and runs `grid` workgroups (0 = the size mha_fwd would use for
 * this block_m) that only fetch work items and add 1 to
 * visits[h * (batch * tiles) + b * tiles + qtile], tiles =
 * ceil(max_seqlen / block_m).  visits is a caller-owned device int32 array of
 * num_heads * batch * tiles entries, zeroed by the caller.  block_m is 32 or
 * 256 (the float32 and bf16 / fp8 kernels' query tiles).  protocol 0
 * reserves the next item when the current one starts and reads its entry
 * after a workgroup barrier (as the float32 kernel does); protocol 1 reserves
 * it and reads its entry near the end of the current item, with workgroup
 * barriers in between (as the bf16 / fp8 kernel does; items with no key
 * blocks included).  Every
 * existing item must end with exactly one visit.  MHA_ERR_INVALID_ARG for a
 * protocol other than 0 or 1.
 */
int mha_sched_visit(const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                    int32_t num_heads, int32_t num_kv_heads, int32_t causal,
                    int32_t block_m, int32_t grid, int32_t protocol, int32_t* visits,
                    void* stream);

/*
 * mha_fwd_splitkv -- mha_fwd with the keys of every query tile cut into
 * num_splits ranges that run as separate work items, merged afterwards (more
 * work items when batch x heads x query tiles would leave compute units
 * idle).  The pages name the split count (SM100AttentionSMem, comptime
 * members: MiscMBarsType is built with the config's splitk_partitions) and
 * keep per-row softmax statistics (Methods: correction_smem); how the keys
 * are cut and merged is this library's:
 *
 *   - a query tile (256 rows) of sequence b sees nb = ceil(n / 64) key blocks
 *     of 64, n = min(L_b, 256 (qt + 1)) when causal, else L_b; split s of
 *     num_splits holds blocks [s p, min((s + 1) p, nb)), p = ceil(nb /
 *     num_splits) (possibly none);
 *   - each split writes its partial result for every row r of the tile:
 *     lse_partial[s, h, r] = ln sum_j exp(S[r, j]) and o_partial[s, r, h, :] =
 *     sum_j exp(S[r, j] - lse_partial[s, h, r]) v[j, g, :] over the visible keys
 *     j of the split (o 0, lse -inf when there are none);
 *   - mha_combine_splits then writes o and lse (bf16 o for BF16 / FP8).
 *
 * Arguments as for mha_fwd, plus:
 *   total_tokens  T = cu_seqlens[batch] (the caller's token count; the partial
 *                 layouts use it; rows at or past it are not written)
 *   num_splits    1 .. 64 (1: exactly mha_fwd, the partials are not used)
 *   o_partial     device float32 [num_splits, T, num_heads, v_dim], 16-byte
 *                 aligned, caller-owned scratch (written)
 *   lse_partial   device float32 [num_splits, num_heads, T] (written)
 * BF16 and FP8_E4M3 shapes only (F32: MHA_ERR_UNSUPPORTED).  Errors as for
 * mha_fwd; also MHA_ERR_INVALID_ARG for num_splits outside 1 .. 64, a
 * negative total_tokens, or NULL / misaligned partial buffers with
 * num_splits > 1.  The kernel-events hook brackets the attention kernel;
 * the merge follows it on the same stream.
 */
int mha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim_nope,
                    int32_t head_dim_rope, int32_t v_dim, const void* q_rope, const void* k_rope,
                    int32_t causal, float softmax_scale, int32_t dtype, const float* q_scale,
                    const float* k_scale, int32_t total_tokens, int32_t num_splits,
                    float* o_partial, float* lse_partial, void* stream);

/*
 * mha_combine_splits -- the log-sum-exp merge of partial attention results
 * over disjoint key sets (the second half of mha_fwd_splitkv; also merges
 * results computed elsewhere, e.g. on several devices):
 *
 *   lse[h, t] = ln sum_s exp(lse_partial[s, h, t])
 *   o[t, h, :] = sum_s exp(lse_partial[s, h, t] - lse[h, t]) o_partial[s, t, h, :]
 *
 * with the largest term factored out; a partial with lse -inf weighs 0; a
 * row whose partials are all -inf gets o = 0, lse = -inf.
 *   o_partial    device float32 [num_splits, total_tokens, num_heads, v_dim],
 *                16-byte aligned
 *   lse_partial  device float32 [num_splits, num_heads, total_tokens]
 *   o            device [total_tokens, num_heads, v_dim], float32 (out_dtype
 *                MHA_DTYPE_F32) or bfloat16 (MHA_DTYPE_BF16, RNE), 16-byte
 *                aligned (written)
 *   lse          device float32 [num_heads, total_tokens] (written)
 * num_splits 1 .. 64, v_dim 64 or 128 (else MHA_ERR_UNSUPPORTED).
 * HBM-bound: reads num_splits x (v_dim x 4 + 4), writes v_dim x {4, 2} + 4
 * bytes per (token, head).
 */
int mha_combine_splits(const float* o_partial, const float* lse_partial, int32_t num_splits,
                       int32_t total_tokens, int32_t num_heads, int32_t v_dim, int32_t out_dtype,
                       void* o, float* lse, void* stream);

/*
 * mha_fwd_auto_splits -- the number of key splits mha_fwd chooses for a
 * bf16 / fp8 problem (host arithmetic only, no device call).  With every
 * sequence taken at max_seqlen, nb = ceil(max_seqlen / 64) key blocks for
 * the longest work item and W = the blocks of all items (causal: q-tile t of
 * 256 rows sees min(nb, 4 (t + 1)) blocks) over `cus` compute units: 1 when
 * 4 nb <= 5 ceil(W / cus), else ceil(1.2 nb / ceil(W / cus)) capped at 8 and at
 * nb / 8 (at least 8 blocks per split), lowered until splits x batch x
 * max_seqlen x num_heads x v_dim x 4 bytes (the partial O in float32, as
 * mha_fwd_splitkv keeps it) fit in 1 GiB.
 * The split (SM100AttentionSMem, comptime members: MiscMBarsType takes the
 * config's splitk_partitions) is the pages'; this rule for choosing it is
 * the library's.  Returns >= 1; 1 for non-positive arguments.
 */
int mha_fwd_auto_splits(int32_t batch, int32_t max_seqlen, int32_t num_heads, int32_t causal,
                        int32_t v_dim, int32_t cus);

/*
 * mha_quantize_fp8 -- per-token fp8 quantisation of Q or K rows, the step in
 * front of the FP8_E4M3 path (whose Q and K are E4M3 codes with one float32
 * scale per token and head: SM100AttentionSMem, Parameters: scale_dtype_;
 * Methods q_scale_smem / k_scale_smem).  The pages do not say how the codes
 * are made; this library's reading, per row r of `cols` elements:
 *
 *     scales[r]   = amax_c |x[r, c]| / 448      (1 for a row of zeros)
 *     codes[r, c] = E4M3 code nearest to clamp(x[r, c] / scales[r], -448, 448),
 *                   ties to the even code
 *
 * with IEEE float32 division, so codes and scales are exact functions of x.
 * A [T, H, D] tensor is rows = T * H, cols = D; the results feed mha_fwd as
 * q / k and q_scale / k_scale directly.
 *
 *   x       device, rows x cols, contiguous; float32 (x_dtype MHA_DTYPE_F32)
 *           or bfloat16 (MHA_DTYPE_BF16); 16-byte aligned; finite values
 *           (NaN / Inf inputs give unspecified codes)
 *   codes   device uint8, rows x cols, written; 8-byte aligned
 *   scales  device float32, rows, written
 *   rows    >= 0 (0: nothing is launched), < 2^31
 *   cols    multiple of 8, 8 .. 512
 * MHA_ERR_INVALID_ARG for a NULL pointer (rows > 0), a misaligned pointer, an
 * unknown x_dtype or a size outside these ranges; MHA_ERR_HIP if the launch
 * fails.  HBM-bound: reads rows * cols * sizeof(x), writes rows * (cols + 4)
 * bytes.
 */
int mha_quantize_fp8(const void* x, int32_t x_dtype, int64_t rows, int32_t cols,
                     uint8_t* codes, float* scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MHA_FWD_H_ */
