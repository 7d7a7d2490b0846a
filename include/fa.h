/*
 * fa.h -- C ABI of the fused exact-attention forward for AMD Instinct MI355X
 * (gfx950).
 *
 * Computes O = softmax(Q K^T * scale) V and the per-row natural-log
 * logsumexp LSE = ln sum_j exp(scale * <q_i, k_j>) in one fused tiled pass:
 * the N x N scores and probabilities never reach device memory.  The result is
 * the plain definition ("推理优化 | FlashAttention 1-4 详解", section
 * 原算法：标准 Attention 与显存瓶颈), reached with the online-softmax
 * recurrence of the same page (section Online Softmax 数学推导) and the
 * outputs named on "FlashAttention — IO 感知的精确注意力 kernel" (section 2.3,
 * step 5: O and the logsumexp are written back, nothing N x N).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is caller-owned DEVICE memory on the current HIP
 *     device.  The library never allocates or frees memory and keeps no state
 *     besides a per-device cache of the architecture check.
 *   - Inputs q, k, v (and the KV caches) are bfloat16, contiguous, with the
 *     head dimension innermost.  O is bfloat16 or float32 (fa_dtype); LSE is
 *     float32.
 *   - head_dim must be 64 or 128.  heads_kv must divide heads_q: query head h
 *     reads key/value head h / (heads_q / heads_kv) (grouped-query attention,
 *     "FlashAttention — IO 感知的精确注意力 kernel", section 1 capability table).
 *   - Causal masking is bottom-right aligned: query i of a sequence with Lq
 *     queries and Lk keys sees key j when j <= i + Lk - Lq (the lower triangle
 *     when Lq == Lk).  A query row that sees no key gets O = 0, LSE = -inf.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  They return after enqueueing.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Errors: every argument is validated before anything is enqueued; on a
 *     non-FA_OK return nothing was launched and outputs are untouched (except
 *     FA_ERR_HIP, which reports a failed launch).  fa_last_error() gives a
 *     detail string for the calling thread.
 *   - Thread safety: entry points are reentrant; the detail string is
 *     thread-local.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  FA_ERR_SHAPE = 2,     /* a size is non-positive, too large, or inconsistent */
  FA_ERR_HEADDIM = 3,   /* head_dim is not 64 or 128                         */
  FA_ERR_GQA = 4,       /* heads_kv does not divide heads_q                  */
  FA_ERR_DTYPE = 5,     /* unknown output dtype                              */
  FA_ERR_ARCH = 6,      /* the current device is not gfx950                  */
  FA_ERR_WORKSPACE = 7, /* workspace NULL or smaller than required           */
  FA_ERR_HIP = 8,       /* a HIP runtime call or launch failed               */
  FA_ERR_ARG = 9        /* another argument is out of range (scale, chunk)   */
} fa_status;

typedef enum fa_dtype {
  FA_DTYPE_BF16 = 0,
  FA_DTYPE_F32 = 1
} fa_dtype;

/*
 * fa_fwd -- attention forward for a batch of sequences.
 *
 * Fixed-length mode (cu_seqlens_q == NULL):
 *   q, o : [batch, seqlen_q, heads_q, head_dim]
 *   k, v : [batch, seqlen_k, heads_kv, head_dim]
 *   lse  : [batch, seqlen_q, heads_q]
 *   max_seqlen_q / max_seqlen_k are ignored.
 * Packed variable-length mode (cu_seqlens_q != NULL; "FlashAttention — IO 感知的
 * 精确注意力 kernel", section 1: sequences packed without padding through
 * cumulative offsets):
 *   cu_seqlens_q : device int32 [batch + 1], non-decreasing, cu_seqlens_q[0] = 0;
 *                  sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]).
 *   cu_seqlens_k : same for keys; NULL means "equal to cu_seqlens_q".
 *   q, o : [total_q, heads_q, head_dim];  k, v : [total_k, heads_kv, head_dim]
 *   lse  : [total_q, heads_q]
 *   max_seqlen_q must be >= every query length (it sizes the launch);
 *   max_seqlen_k must be >= every key length.  seqlen_q / seqlen_k are ignored.
 *   The offsets are read on the device; they are not validated there.
 * scale  : finite, > 0 (usually 1/sqrt(head_dim)); multiplies Q K^T in fp32.
 * causal : 0 or 1.
 * o_dtype: FA_DTYPE_BF16 or FA_DTYPE_F32 (O element type).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                 int head_dim, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                 int max_seqlen_q, int max_seqlen_k,
                 fa_dtype o_dtype, void* stream);

/*
 * fa_fwd_ext -- fa_fwd with the score variants the code-reading page lists as
 * compile-time switches beside causal masking ("FlashAttention — IO 感知的精
 * 确注意力 kernel", section 1 capability table: sliding window, ALiBi,
 * softcap).  Same tensors, layouts and rules as fa_fwd.  For query i and key
 * j of a sequence, with delta = Lk - Lq:
 *   x = scale * <q_i, k_j>
 *   softcap > 0          : x = softcap * tanh(x / softcap)
 *   alibi_slopes != NULL : x = x - slope[h] * |i + delta - j|
 *   admissible keys      : 0 <= j < Lk, j >= i + delta - window_left when
 *                          window_left >= 0, j <= i + delta + window_right
 *                          when window_right >= 0, and j <= i + delta when
 *                          causal (a negative window bound is open)
 *   O_i = softmax of x over the admissible keys, times V; lse natural log;
 *   a row without admissible keys gets O = 0 and lse = -inf.
 *   alibi_slopes        : device float32 [heads_q] (alibi_batch_stride = 0)
 *                         or [batch, heads_q] (alibi_batch_stride = heads_q).
 * Runs the pipelined forward's window instance, which visits only the key
 * tiles holding admissible keys (with ALiBi or a softcap, its instance that
 * transforms every score); with no variant set it equals fa_fwd, which pairs
 * causal tiles and is faster for that case.  The softcap and the distance
 * bias are computed in fp32 (tanh from one exp2 and one reciprocal).
 */
fa_status fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                     int head_dim, float scale, int causal,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     int max_seqlen_q, int max_seqlen_k, int window_left, int window_right,
                     float softcap, const float* alibi_slopes, int alibi_batch_stride,
                     fa_dtype o_dtype, void* stream);

/*
 * fa_fwd_fp8 -- the forward on FP8 inputs, both products on the FP8 matrix
 * cores (the first page's FlashAttention 3 notes, "推理优化 | FlashAttention
 * 1-4 详解", section FlashAttention 3 的硬件特性利用: FP8 matrix products in
 * the forward).  q, k, v hold OCP E4M3 codes (one byte each: 1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits, S.1111.111 = NaN, largest
 * finite 448), in fa_fwd's layouts; the real tensors are q_descale * q,
 * k_descale * k and v_descale * v.  Computes fa_fwd's O and lse of those real
 * tensors (same batching, varlen, causal and GQA rules), with these
 * differences:
 *   head_dim            : 128 only (FA_ERR_HEADDIM otherwise);
 *   q/k/v_descale       : finite and > 0 (FA_ERR_ARG otherwise);
 *   precision           : the scores are exact products of E4M3 values summed
 *                         by the FP8 matrix core (whose internal accumulation
 *                         is not exact fp32: measured errors reach about
 *                         2^-12 of the largest product in a 64-term sum);
 *                         the probabilities exp(s - r) are rounded to E4M3
 *                         before the product with V (r within 8 log2 units of
 *                         the row maximum), the row sum uses the unrounded
 *                         ones; O is scaled by v_descale in fp32.
 * Inputs containing NaN codes give NaN outputs.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                     int head_dim, float scale, float q_descale, float k_descale,
                     float v_descale, int causal, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, int max_seqlen_q, int max_seqlen_k,
                     fa_dtype o_dtype, void* stream);

/*
 * fa_decode_workspace_size -- bytes of float32 scratch that
 * fa_fwd_decode_splitkv needs for these sizes: the partial O and LSE that
 * every key chunk writes before the LSE-weighted merge ("FlashAttention — IO
 * 感知的精确注意力 kernel", section 2.3 step 3: split-KV for a short query;
 * section 7: each split keeps its partial result and a final step combines
 * them).  Per query row and split it holds head_dim + 1 floats.  chunk = 0
 * selects the built-in chunk size, which depends on heads_kv as well; the
 * size returned then covers every heads_kv that divides heads_q.  Returns 0
 * for invalid sizes.
 */
size_t fa_decode_workspace_size(int batch, int heads_q, int max_cache_len, int head_dim,
                                int chunk);

/*
 * fa_fwd_decode_splitkv -- one query per sequence against a KV cache, with the
 * keys split into chunks processed in parallel and merged by LSE weight
 * (split-KV for a short query and long keys, "FlashAttention — IO 感知的精确
 * 注意力 kernel", section 2.3 step 3 and the split-KV combine of section 7;
 * the query-head group is folded into the row dimension, section 4).
 *
 *   q, o          : [batch, heads_q, head_dim]
 *   k_cache, v_cache : [batch, max_cache_len, heads_kv, head_dim]
 *   cache_seqlens : device int32 [batch]; sequence b uses cache rows
 *                   [0, cache_seqlens[b]); values must lie in [0, max_cache_len]
 *                   (read on the device, not validated there).  Rows past the
 *                   length are never read.
 *   lse           : [batch, heads_q]
 *   chunk         : keys per split, a multiple of 128; 0 = built-in choice.
 *   workspace     : device memory of at least
 *                   fa_decode_workspace_size(batch, heads_q, max_cache_len,
 *                   head_dim, chunk) bytes, 16-byte aligned; contents on entry
 *                   are ignored, contents on return are unspecified.
 *   heads_q / heads_kv must be <= 32.
 * Enqueues the split kernel, then the combine, on `stream`.
 */
fa_status fa_fwd_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* cache_seqlens, void* o, float* lse,
                                int batch, int heads_q, int heads_kv, int max_cache_len,
                                int head_dim, float scale, int chunk,
                                void* workspace, size_t workspace_bytes,
                                fa_dtype o_dtype, void* stream);

/*
 * fa_decode_kvcache_workspace_size -- bytes of device scratch that
 * fa_fwd_decode_kvcache needs (a bf16 copy of the rotated queries, then the
 * split partials); max_cache_len is the per-sequence capacity.  Returns 0
 * for invalid sizes.  A call without rotary needs only
 * fa_decode_workspace_size(...) bytes.
 */
size_t fa_decode_kvcache_workspace_size(int batch, int heads_q, int max_cache_len,
                                        int head_dim, int chunk);

/*
 * fa_fwd_decode_kvcache -- one decode step against a KV cache that the call
 * updates in place, with rotary embedding applied to the new token in the
 * same call and the cache optionally paged ("FlashAttention — IO 感知的精确注
 * 意力 kernel", section 1: the KV-cache capability row (in-place append,
 * paged KV, split-KV decode) and the usage snippet's KV-cache call).  For
 * each sequence b, with t = cache_seqlens[b] tokens cached before the call:
 *   1. rotary (rotary_cos != NULL): q[b] and k_new[b] are rotated at
 *      position t.  Pair i of the first rotary_dim components, (i,
 *      i + rotary_dim/2) or (2i, 2i + 1) when rotary_interleaved, turns by
 *      the angle of table row t: (a, b) -> (a cos - b sin, b cos + a sin),
 *      computed in fp32 (products and sum rounded separately) and rounded to
 *      bf16.  q itself is not modified; the rotated copy is kept in the
 *      workspace.
 *   2. append (k_new != NULL): the (rotated) k_new[b] and v_new[b] are
 *      written to cache row t of sequence b.
 *   3. single-query attention over cache rows [0, t + (k_new != NULL)),
 *      split into chunks and merged as in fa_fwd_decode_splitkv.
 * cache_seqlens is read, never written: the caller advances it.
 *
 *   q, o             : [batch, heads_q, head_dim] bf16 / o_dtype
 *   k_new, v_new     : [batch, heads_kv, head_dim] bf16, or both NULL
 *   cache (block_table == NULL): k_cache, v_cache [batch, max_cache_len,
 *                      heads_kv, head_dim] bf16
 *   cache (paged): k_cache, v_cache [num_blocks, page_size, heads_kv,
 *                      head_dim]; block_table device int32 [batch,
 *                      max_blocks_per_seq]; logical row j of sequence b is
 *                      row j % page_size of block
 *                      block_table[b * max_blocks_per_seq + j / page_size].
 *                      page_size is a positive multiple of 128 and
 *                      max_cache_len must equal max_blocks_per_seq *
 *                      page_size.
 *   rotary_cos, rotary_sin : device fp32 [rotary_max_pos, rotary_dim / 2],
 *                      or both NULL; rotary_dim even, <= head_dim.
 *   lse              : [batch, heads_q] fp32
 *   workspace        : fa_decode_kvcache_workspace_size(batch, heads_q,
 *                      max_cache_len, head_dim, chunk) bytes, 16-byte
 *                      aligned; contents unspecified on return.
 * Device-side preconditions, not validated there: t + (k_new != NULL) <=
 * max_cache_len, t < rotary_max_pos, and every block id in [0, num_blocks).
 * A violation gives unspecified results but no out-of-bounds access: block
 * ids are clamped, a row outside the cache is not written, and a position
 * outside the table is not rotated.  Enqueues the append (when rotary or
 * k_new is given), the split kernel and the combine on `stream`.
 */
fa_status fa_fwd_decode_kvcache(const void* q, void* k_cache, void* v_cache,
                                const void* k_new, const void* v_new,
                                const int32_t* cache_seqlens, const int32_t* block_table,
                                int max_blocks_per_seq, int page_size, int num_blocks,
                                const float* rotary_cos, const float* rotary_sin,
                                int rotary_dim, int rotary_max_pos, int rotary_interleaved,
                                void* o, float* lse, int batch, int heads_q, int heads_kv,
                                int max_cache_len, int head_dim, float scale, int chunk,
                                void* workspace, size_t workspace_bytes, fa_dtype o_dtype,
                                void* stream);

/*
 * Bytes of device scratch that fa_fwd_decode_kvcache_noalloc holds on each
 * device it runs on (64 MiB).
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * fa_fwd_decode_kvcache_noalloc -- fa_fwd_decode_kvcache without a workspace
 * argument, for callers that cannot allocate device memory at the call: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the rotated queries and split partials go to
 * a scratch array that the library holds on every device it runs on, from
 * the first use there until the process ends.
 *   Arguments, layouts, results and errors: as fa_fwd_decode_kvcache, less
 *   workspace / workspace_bytes.  The call is bit-identical to
 *   fa_fwd_decode_kvcache with the same arguments.
 *   Limit: fa_decode_kvcache_workspace_size(batch, heads_q, max_cache_len,
 *   head_dim, chunk) -- for chunk = 0 an upper bound of the need -- must not
 *   exceed FA_NOALLOC_SCRATCH_BYTES; a call that needs more returns
 *   FA_ERR_WORKSPACE before touching the device.  (64 sequences x 32 query
 *   heads x 32768 cache rows x head_dim 128 with the built-in chunk needs
 *   about 24 MB.)
 *   Concurrency: every call on one device shares that device's scratch.
 *   Calls on one stream are ordered and safe; calls that can overlap on one
 *   device (different streams, or different host threads without ordering)
 *   race on it and give wrong results.  Nothing in the scratch needs to be
 *   cleared between calls.
 */
fa_status fa_fwd_decode_kvcache_noalloc(const void* q, void* k_cache, void* v_cache,
                                        const void* k_new, const void* v_new,
                                        const int32_t* cache_seqlens,
                                        const int32_t* block_table, int max_blocks_per_seq,
                                        int page_size, int num_blocks,
                                        const float* rotary_cos, const float* rotary_sin,
                                        int rotary_dim, int rotary_max_pos,
                                        int rotary_interleaved, void* o, float* lse,
                                        int batch, int heads_q, int heads_kv,
                                        int max_cache_len, int head_dim, float scale,
                                        int chunk, fa_dtype o_dtype, void* stream);

/*
 * fa_combine -- LSE-weighted merge of partial results computed over disjoint
 * key subsets (the block merge of the PKU lecture notes "FlashAttention",
 * section 6, written with logsumexps):
 *   M = max_s lse_part[r, s]
 *   lse[r] = M + ln sum_s exp(lse_part[r, s] - M)
 *   o[r, :] = sum_s exp(lse_part[r, s] - lse[r]) * o_part[r, s, :]
 * A split with lse_part = -inf is empty and contributes nothing (its o_part
 * values are not read).  All splits empty gives o = 0, lse = -inf.
 *   o_part   : float32 [rows, n_splits, head_dim], each split's normalised O
 *   lse_part : float32 [rows, n_splits]
 *   o        : [rows, head_dim] in o_dtype;  lse : float32 [rows]
 *   1 <= n_splits <= 4096.
 */
fa_status fa_combine(const float* o_part, const float* lse_part, int rows, int n_splits,
                     int head_dim, void* o, float* lse, fa_dtype o_dtype, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs: two fp32
 * arrays (rowsum(dO * O) and the logsumexp in base 2) of heads_q x
 * (batch * max_seqlen_q + 64) values.  For a fixed-length batch pass
 * max_seqlen_q = seqlen_q.  Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int batch, int heads_q, int max_seqlen_q);

/*
 * fa_bwd -- gradients of the scalar <dout, o> with respect to q, k and v for
 * the forward of fa_fwd (same shapes, layouts, scale, causal rule and varlen
 * conventions).  The backward keeps only o and lse from the forward and
 * recomputes P = exp(S scale - lse) tile by tile ("FlashAttention — IO 感知
 * 的精确注意力 kernel", section 4: the backward recomputes P from the saved
 * logsumexp and is split by key blocks; section 2.3: autograd saves q, k, v,
 * out and the logsumexp).  With D = rowsum(dout * o):
 *   dv = P^T dout,  dS = P * (dout v^T - D),  dq = scale dS k,
 *   dk = scale dS^T q;
 * a kv head receives the sum over the query heads of its group.
 *
 *   q, o, dout, dq : as q in fa_fwd;   k, v, dk, dv : as k in fa_fwd
 *   lse            : float32, the forward's natural-log logsumexp
 *   dq, dk, dv     : written in grad_dtype (bf16 or fp32); every row of the
 *                    batch is written, keys no query sees get zero.
 *   workspace      : device memory of at least fa_bwd_workspace_size(batch,
 *                    heads_q, varlen ? max_seqlen_q : seqlen_q) bytes,
 *                    4-byte aligned; contents on entry are ignored.
 *   varlen         : max_seqlen_q / max_seqlen_k must bound every sequence.
 * Bitwise deterministic: dq is computed by its own pass, not by atomic adds.
 * Enqueues three kernels on `stream`.  Errors as fa_fwd, plus
 * FA_ERR_WORKSPACE for a missing, short or misaligned workspace.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int batch, int heads_q,
                 int heads_kv, int seqlen_q, int seqlen_k, int head_dim, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int max_seqlen_q,
                 int max_seqlen_k, fa_dtype grad_dtype, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * The error channel of this interface.  No passage of the pages defines
 * error reporting: these two calls compute nothing of the method and only
 * describe the status codes the entry points above return.
 *
 * fa_status_string -- static, human-readable name of a status code
 * ("FA_ERR_UNKNOWN" for a value outside fa_status).  Never NULL.
 */
const char* fa_status_string(fa_status status);

/*
 * fa_last_error -- detail of the last non-FA_OK status returned on the
 * calling thread (empty string if none).  The string is owned by the
 * library, thread-local, and valid until the next call on that thread.
 */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
