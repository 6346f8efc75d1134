/*
 * rpa.h: paged, variable-length, causal attention with an additive relative
 * position bias, for AMD MI355X (gfx950).  C ABI of librpa.so.
 *
 * The operation is the one the Inkling FA4 relative-attention walkthrough
 * ("vllm中提取Inkling FA4 Relative Attention算子基础的base优化版本",
 * nxmr.cn/news/19446) wraps around flash_attn_varlen_func: sections
 * "_get_score_mod() 的内部" (the bias), "inkling_fa4_num_splits" (the split
 * planner) and "主函数 inkling_fa4_rel_attention" (arguments and layouts).
 * For request b with Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] query tokens
 * and Lk = cache_seqlens[b] keys, query row i (packed token
 * tok = cu_seqlens_q[b] + i) sits at absolute position qa = i + Lk - Lq and
 * q head h reads kv head h / (H / Hkv).  Key t < Lk lives at
 * key_cache[block_table[b, t / BS], t % BS, kv_head, :].  Key t is visible
 * when causal implies t <= qa, window_left >= 0 implies t >= qa - left and
 * window_right >= 0 implies t <= qa + right.  The logit of a visible key is
 *     s = softmax_scale * <q[tok, h], k[t]>
 *         + (0 <= qa - t < rel_extent ? rel_logits[tok, h, qa - t] : 0)
 * and out[tok, h] = sum_t softmax(s)_t v[t], lse[tok, h] = ln sum_t exp(s_t).
 * A row with no visible key gets out = 0 and lse = -inf.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major data
 *     on the current HIP device; the caller owns them.  The library
 *     allocates nothing and keeps no state between calls, except the static
 *     scratch array of rpa_attn_varlen_noalloc (below).
 *   - Calls are asynchronous: they validate host-visible arguments, enqueue
 *     kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *     return.  Any error status is returned BEFORE anything is enqueued,
 *     except RPA_ERR_HIP, which reports a failed launch.
 *   - Calls enqueue kernel launches only (no memset, copy, allocation or
 *     host read of device data) and size their grids from host arguments
 *     alone, so a call can be captured in a HIP graph and replayed after
 *     the device-resident lengths, block table and inputs change in place.
 *   - bf16 means IEEE bfloat16 bit patterns (uint16 storage); outputs are
 *     rounded to nearest even from fp32.
 *   - Results are bitwise repeatable for fixed inputs and num_splits.
 */
#ifndef RPA_H
#define RPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RPA_OK = 0,
  RPA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  RPA_ERR_SHAPE = -2,       /* inconsistent or negative sizes, or key positions
                               past 32 bits (max_pages_per_seq * block_size
                               + max_seqlen_q + rel_extent + 128 >= 2^31)        */
  RPA_ERR_UNSUPPORTED = -3, /* head_dim not 64/128, block_size not a multiple of 16,
                               or bf16 rel_logits misaligned or too wide (_ex)       */
  RPA_ERR_WORKSPACE = -4,   /* num_splits != 1 and the workspace is missing/small */
  RPA_ERR_HIP = -5          /* a HIP launch failed                                */
} rpa_status;

/* Largest num_splits accepted by rpa_attn_varlen. */
#define RPA_MAX_SPLITS 128

/*
 * rpa_attn_varlen: the whole method in one call (attention kernel, plus the
 * split combine when num_splits > 1).
 *
 *   q              bf16 [num_tokens, num_heads, head_dim], queries packed by
 *                  cu_seqlens_q (already normalised / rotated by the caller).
 *   key_cache,
 *   value_cache    bf16 [num_blocks, block_size, num_kv_heads, head_dim].
 *   block_table    int32 [batch, max_pages_per_seq]; only the first
 *                  ceil(Lk / block_size) entries of a row are read and each
 *                  must lie in [0, num_blocks); padding may hold any value.
 *   cache_seqlens  int32 [batch]: Lk, the KV length INCLUDING this step's
 *                  query tokens (their K/V are already in the cache).
 *   cu_seqlens_q   int32 [batch + 1]: non-decreasing, cu[0] = 0,
 *                  cu[batch] = num_tokens.
 *   max_seqlen_q   must be >= every Lq.  It only bounds the launch grid: a
 *                  larger value changes nothing, a smaller one drops work.
 *   softmax_scale  multiplies <q, k>; the bias is added after scaling.  Any finite
 *                  value, including 0 and negative values; a scale below 2^-100 in
 *                  magnitude is treated as 0 (its q.k term changes no fp32 logit).
 *                  The prefill kernel carries the bias as bias / scale, so
 *                  |rel_logits| must stay below 2^27.
 *   causal         nonzero = bottom-right causal mask.
 *   window_left,
 *   window_right   sliding window; -1 leaves that side unbounded, and so does
 *                  any side that reaches past every key (left >=
 *                  max_pages_per_seq * block_size, right >= max_seqlen_q):
 *                  any value up to 2^31 - 1 is accepted.
 *   rel_extent     R >= 0; 0 means no bias (rel_logits may then be NULL).
 *   rel_logits     fp32 [num_tokens, num_heads, R].
 *   num_splits     S in [0, RPA_MAX_SPLITS].  S >= 1: each work item's
 *                  visible key range is cut into S contiguous chunks whose
 *                  partial results are merged by the log-sum-exp combine.
 *                  S = 0, balanced: when every request has Lq * G <= 16 (known
 *                  from max_seqlen_q), batch <= 2048 and rel_logits spans
 *                  less than 2 GiB, the 16-key blocks of the whole batch are
 *                  dealt out in equal contiguous shares, one per compute unit
 *                  of the current device (with 8 kv heads a block covers all
 *                  heads, else one (request, kv head) pair), and the pieces of
 *                  a request cut between shares are merged by the same
 *                  combine; otherwise S = 0 runs as S = 1.  rpa_choose_splits gives a
 *                  default.  Any S gives the same result up to fp32 rounding.
 *   workspace      device scratch of at least rpa_workspace_bytes(S, ...)
 *                  bytes when S != 1 (may be NULL when S == 1); holds split
 *                  partials, consumed within this call on `stream`.
 *   out            bf16 [num_tokens, num_heads, head_dim], written.
 *   lse            fp32 [num_tokens, num_heads] natural-log LSE, or NULL.
 *
 * Device-resident metadata (block_table, cache_seqlens, cu_seqlens_q) is not
 * checked; violating the preconditions above is undefined behaviour, except
 * that Lk < Lq (rows with negative qa) and Lk == 0 are defined (empty rows).
 * Supported: head_dim in {64, 128}; block_size a positive multiple of 16;
 * num_heads a multiple of num_kv_heads.
 */
int rpa_attn_varlen(const void *q, const void *key_cache, const void *value_cache,
                    const int32_t *block_table, int32_t max_pages_per_seq,
                    const int32_t *cache_seqlens, const int32_t *cu_seqlens_q,
                    int32_t batch, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t num_blocks, int32_t block_size,
                    int32_t max_seqlen_q, float softmax_scale, int causal,
                    int32_t window_left, int32_t window_right,
                    int32_t rel_extent, const float *rel_logits,
                    int32_t num_splits, void *workspace, size_t workspace_bytes,
                    void *out, float *lse, void *stream);

/*
 * rpa_workspace_bytes: scratch needed by rpa_attn_varlen for num_splits
 * partials: num_splits * num_tokens * num_heads * (head_dim + 1) * 4 bytes
 * (fp32 partial outputs and LSEs), rounded up to 256; 0 when num_splits == 1.
 * num_splits = 0 needs a fixed size for head_dim, whatever the batch:
 * 16 KiB of per-workgroup records plus 8192 * 16 * (head_dim + 1) * 4 bytes
 * of partials (two slots of eight kv heads for each of up to 512
 * workgroups; about 68 MB for head_dim 128).  Returns 0 for negative sizes.
 */
size_t rpa_workspace_bytes(int32_t num_splits, int32_t num_tokens, int32_t num_heads,
                           int32_t head_dim);

/*
 * rpa_split_combine: merge split partials (the phase-2 reduction of
 * partitioned attention, "paged_attention_v2_pytorch.py — BI-V100
 * PagedAttention V2", dev.modelhub.org.cn, with NORMALISED partials):
 *     M = max_s lse_s,  LSE = M + ln sum_s exp(lse_s - M),
 *     out = sum_s exp(lse_s - LSE) * o_s;
 * rows whose every lse_s is -inf give out = 0, lse = -inf.  A split whose
 * weight exp(lse_s - LSE) is 0 (lse_s = -inf: an empty chunk) is skipped, so
 * its partial_out row may hold any value, NaN included.  Every lse_s must be
 * finite or -inf (+inf and NaN are outside the contract).
 *
 *   partial_out  fp32 [num_splits, num_tokens, num_heads, head_dim]
 *   partial_lse  fp32 [num_splits, num_tokens, num_heads], natural log
 *   out          bf16 [num_tokens, num_heads, head_dim], written
 *   lse          fp32 [num_tokens, num_heads], written, or NULL
 * head_dim must be a positive multiple of 64 up to 256; num_splits in
 * [1, RPA_MAX_SPLITS].
 */
int rpa_split_combine(const float *partial_out, const float *partial_lse, int32_t num_splits,
                      int32_t num_tokens, int32_t num_heads, int32_t head_dim, void *out,
                      float *lse, void *stream);

/*
 * rpa_choose_splits: default num_splits for a batch (host only, no HIP call).
 * Same inputs as the walkthrough's inkling_fa4_num_splits (batch,
 * max_seqlen_q, heads, kv heads, max KV length, whether a window is set),
 * re-derived for a gfx950 with num_cus compute units (<= 0 means 256): work
 * items are (request, q-tile, kv head); a decode batch (max_seqlen_q * G <=
 * 16, at most 2048 requests, no window) gets 0, the balanced decode; other
 * batches are split until about two workgroups per CU exist, keeping at
 * least 512 keys per split; windowed (local) attention uses 1.
 * Returns a value in [0, RPA_MAX_SPLITS], or RPA_ERR_SHAPE for bad sizes.
 */
int rpa_choose_splits(int32_t batch, int32_t max_seqlen_q, int32_t num_heads,
                      int32_t num_kv_heads, int64_t max_seqlen_k, int is_local, int32_t num_cus);

/*
 * rpa_slot_mapping: the cache slot of every query token of a batch — the
 * slot_mapping of "vLLM V1 Attention — Part 2: 标准Attention后端实现"
 * (devpress.csdn.net), 附录O.1 Step 2.  Token j of request b (packed token
 * cu_seqlens_q[b] + j, Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b]) sits at
 * position pos = cache_seqlens[b] - Lq + j and gets the slot
 * block_table[b, pos / block_size] * block_size + pos % block_size, or -1
 * when pos < 0 (a request with fewer keys than queries).
 *
 *   block_table, max_pages_per_seq, cache_seqlens, cu_seqlens_q, batch,
 *   num_tokens, block_size   as for rpa_attn_varlen (device metadata is not
 *                            checked; block_size any positive value).
 *   slot_mapping             int64 [num_tokens], written.
 */
int rpa_slot_mapping(const int32_t *block_table, int32_t max_pages_per_seq, const int32_t *cache_seqlens,
                     const int32_t *cu_seqlens_q, int32_t batch, int32_t num_tokens, int32_t block_size,
                     int64_t *slot_mapping, void *stream);

/*
 * rpa_kv_cache_write: writes this step's keys and values into the paged
 * caches before attention — reshape_and_cache in "vLLM V1 Attention — Part
 * 2", 6.5 (FlashInferImpl.forward, step 2).  For every token t with
 * 0 <= s = slot_mapping[t] < num_blocks * block_size:
 *     key_cache[s / block_size, s % block_size] = key[t]
 *     value_cache[s / block_size, s % block_size] = value[t]
 * and other tokens write nothing (a negative slot is padding; a slot past the
 * cache is skipped rather than faulted).  Slots must be distinct; rows are
 * copied bit for bit.
 *
 *   key, value        bf16 [num_tokens, num_kv_heads, head_dim], 16-byte aligned.
 *   slot_mapping      int64 [num_tokens].
 *   key_cache,
 *   value_cache       bf16 [num_blocks, block_size, num_kv_heads, head_dim],
 *                     16-byte aligned, written in place.
 * num_kv_heads * head_dim must be a multiple of 8 (16-byte rows), else
 * RPA_ERR_UNSUPPORTED.
 */
int rpa_kv_cache_write(const void *key, const void *value, const int64_t *slot_mapping, int32_t num_tokens,
                       int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                       void *key_cache, void *value_cache, void *stream);

/*
 * FP8 KV cache.  "paged_attention_v2_pytorch.py — BI-V100 PagedAttention V2"
 * (dev.modelhub.org.cn) takes kv_cache_dtype, k_scale and v_scale and turns
 * the gathered cache rows into floats times their scale before the scores;
 * the TurboQuant chapter of "vLLM V1 Attention — Part 2" stores K/V as FP8
 * with a scale factor, quantised when written and dequantised when read.
 * Here the cache holds OCP E4M3 codes (uint8: 4 exponent bits with bias 7,
 * 3 mantissa bits, largest finite 448, S.1111.111 = NaN) with one k_scale
 * and one v_scale per cache (finite, > 0): code c stands for
 * e4m3(c) * scale.
 */

/*
 * rpa_attn_varlen_fp8: rpa_attn_varlen over E4M3 caches.  The result is the
 * definition above with k = e4m3(key code) * k_scale and
 * v = e4m3(value code) * v_scale: k_scale multiplies <q, k> only (the bias is
 * not scaled), v_scale the output only (not the LSE).
 *
 *   key_cache,
 *   value_cache   uint8 E4M3 codes [num_blocks, block_size, num_kv_heads, head_dim].
 *   k_scale,
 *   v_scale       finite and > 0, else RPA_ERR_SHAPE.
 * Every other argument, the supported sizes and the error behaviour are
 * those of rpa_attn_varlen (every split count and batch mix; the kernels
 * decode the codes to bf16 exactly as they stage each page).
 */
int rpa_attn_varlen_fp8(const void *q, const void *key_cache, const void *value_cache, float k_scale,
                        float v_scale, const int32_t *block_table, int32_t max_pages_per_seq,
                        const int32_t *cache_seqlens, const int32_t *cu_seqlens_q,
                        int32_t batch, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t num_blocks, int32_t block_size,
                        int32_t max_seqlen_q, float softmax_scale, int causal,
                        int32_t window_left, int32_t window_right,
                        int32_t rel_extent, const float *rel_logits,
                        int32_t num_splits, void *workspace, size_t workspace_bytes,
                        void *out, float *lse, void *stream);

/*
 * rpa_attn_varlen_ex: rpa_attn_varlen with every option of the path.
 *
 *   kv_e4m3        0: bf16 caches (k_scale, v_scale ignored); nonzero: E4M3
 *                  caches with k_scale, v_scale as for rpa_attn_varlen_fp8.
 *   rel_logits_bf16  0: rel_logits is fp32 [num_tokens, num_heads, R];
 *                  nonzero: bf16 of the same shape (half the bias bytes; the
 *                  values are widened exactly to fp32 where they are added).
 *                  bf16 rel_logits must start on a 4-byte boundary (they
 *                  are read as dwords), else RPA_ERR_UNSUPPORTED; so does a
 *                  batch with prefill rows (max_seqlen_q * num_heads /
 *                  num_kv_heads > 16) when (128 / G + 2) * num_heads * R * 2
 *                  bytes reach 2 GiB (G = num_heads / num_kv_heads): the
 *                  rows of one 128-row tile are read through one buffer
 *                  resource.
 *   alibi_slopes   NULL, or fp32 [num_heads] device array: the logit of key t
 *                  for a row at position qa of q head h gains
 *                  alibi_slopes[h] * (t - qa), added like the relative bias
 *                  (after softmax_scale; not scaled by it, nor by k_scale).
 *                  This is the ALiBi example of the FlexAttention chapter of
 *                  "vLLM V1 Attention — Part 2" (scores plus slopes times
 *                  (k_pos - q_pos)); the BI-V100 decode's form with the
 *                  absolute key position gives the same output and an LSE
 *                  larger by slope * qa.  Finite slopes of any sign; with
 *                  slopes the prefill kernel carries the bias as bias / scale,
 *                  so |slope * (t - qa)| must stay below 2^27 on visible keys.
 * Every other argument is that of rpa_attn_varlen; rpa_attn_varlen and
 * rpa_attn_varlen_fp8 are this call without slopes.
 */
int rpa_attn_varlen_ex(const void *q, const void *key_cache, const void *value_cache, int kv_e4m3,
                       float k_scale, float v_scale, const int32_t *block_table, int32_t max_pages_per_seq,
                       const int32_t *cache_seqlens, const int32_t *cu_seqlens_q,
                       int32_t batch, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t num_blocks, int32_t block_size,
                       int32_t max_seqlen_q, float softmax_scale, int causal,
                       int32_t window_left, int32_t window_right,
                       int32_t rel_extent, const void *rel_logits, int rel_logits_bf16,
                       const float *alibi_slopes, int32_t num_splits, void *workspace,
                       size_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * rpa_attn_varlen_noalloc: rpa_attn_varlen_ex without the workspace
 * arguments, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * It calls no allocating routine.  The workspace it needs (num_splits > 1
 * partials, or the balanced decode's records and partial slots) is a static
 * device array of RPA_NOALLOC_SCRATCH_BYTES that every GPU loading the
 * library holds until the process ends; its address is looked up once per
 * device, on that device's first call that needs it.
 *
 * Limit: the call returns RPA_ERR_WORKSPACE, before anything is enqueued,
 * when it needs more than RPA_NOALLOC_SCRATCH_BYTES: for num_splits > 1,
 * num_splits * num_tokens * num_heads * (head_dim + 1) * 4 bytes (rounded up
 * to 256); for the balanced decode (num_splits = 0 on a decode batch),
 * 16 KiB + (compute units of the device) * 16 * 16 * (head_dim + 1) * 4
 * bytes, about 34 MB for head_dim 128 on 256 compute units.  num_splits = 1
 * needs no workspace.
 *
 * Every call on one GPU shares that GPU's array, and nothing in it needs to
 * start at zero.  Calls that overlap on one GPU (on different streams, or
 * from different host threads without ordering) race on the array and give
 * undefined results; calls serialised on one stream do not.  Every other
 * argument, the result and the error behaviour are those of
 * rpa_attn_varlen_ex with the same num_splits.
 */
#define RPA_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
int rpa_attn_varlen_noalloc(const void *q, const void *key_cache, const void *value_cache, int kv_e4m3,
                            float k_scale, float v_scale, const int32_t *block_table,
                            int32_t max_pages_per_seq, const int32_t *cache_seqlens,
                            const int32_t *cu_seqlens_q, int32_t batch, int32_t num_tokens,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t num_blocks, int32_t block_size, int32_t max_seqlen_q,
                            float softmax_scale, int causal, int32_t window_left,
                            int32_t window_right, int32_t rel_extent, const void *rel_logits,
                            int rel_logits_bf16, const float *alibi_slopes, int32_t num_splits,
                            void *out, float *lse, void *stream);

/*
 * rpa_kv_cache_write_fp8: rpa_kv_cache_write into E4M3 caches.  Element x of
 * a key row is stored as the code of y = x / k_scale (one IEEE fp32
 * division): the nearest E4M3 value, ties to the even code; |y| >= 448
 * (infinity included) stores +-448; NaN stores a NaN code with x's sign.
 * Values use v_scale alike.  Slots, skipping and alignment are those of
 * rpa_kv_cache_write; the caches are uint8 [num_blocks, block_size,
 * num_kv_heads, head_dim], 8-byte aligned.  k_scale and v_scale must be
 * finite and > 0, else RPA_ERR_SHAPE.
 */
int rpa_kv_cache_write_fp8(const void *key, const void *value, const int64_t *slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                           float k_scale, float v_scale, void *key_cache, void *value_cache, void *stream);

/* rpa_status_string: static text for a status code (never NULL). */
const char *rpa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RPA_H */
