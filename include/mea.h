/*
 * mea.h -- C ABI of the fused memory-efficient attention forward and backward
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (for every packed sequence b and query head h):
 *
 *   out[t, h, :] = sum_j softmax_j(scale * q[t, h, :] . k[j, g(h), :] + bias) v[j, g(h), :]
 *
 * where j runs over the keys of sequence b only (block-diagonal mask over
 * packed variable-length sequences: "Cómo construir transformadores con
 * memoria eficiente con xFormers ..." (7minutos.es), section 4, and "How to
 * Build Memory-Efficient Transformers with xFormers ..." (yifor-blog),
 * optimisation item 1), the scores are the scaled dot products of the
 * self-attention snippet on "multi query attention代码" (cidian.kuaisou.com),
 * g(h) = h / (Hq / Hkv) is the shared key/value head of query head h
 * (grouped-query attention: the GQA definition and the enable_gqa /
 * repeat_interleave check on "group query attention gqa", and the BMGHK
 * layout of the tutorial's section 5), and the bias is
 *   - ALiBi (yifor-blog, item 3): -slope[h] * |(r + L_k - L_q) - j| for query
 *     row r of the sequence, positions local to the sequence;
 *   - causal (yifor-blog, item 5): -inf where j > r + L_k - L_q (the queries
 *     are the last L_q positions of the sequence, so a single query sees its
 *     whole key history).
 * A row with no allowed key gets out = 0 and lse = -inf.
 *
 * The N x N score matrix is never written to memory: scores are produced
 * tile by tile on the matrix cores and folded into an online softmax.  A call
 * whose longest query sequence has one token (max_seqlen_q == 1, the decode
 * case) cuts the concatenated key axis [0, total_k) of all sequences into
 * equal pieces processed in parallel, one partial result per (piece,
 * sequence it touches), and merges each sequence's partials by their
 * log-sum-exp (the split-K scheme named in section 1 of
 * "大模型推理加速终极指南：xformers如何让Transformer性能飙升300%"
 * (zizhi168.cn)).
 *
 * Layouts (row-major, contiguous, element = 16-bit float of `dtype`):
 *   q, out       [total_q, Hq, D]
 *   k, v         [total_k, Hkv, D]
 *   lse          [Hq, total_q] float32 (natural log)
 *   seqstart_q   int32 [num_seqs + 1]: sequence b owns query rows
 *                seqstart_q[b] .. seqstart_q[b+1]-1; same for seqstart_k.
 *   alibi_slopes float32 [Hq] (per query head) or NULL for no ALiBi.
 *
 * Ownership: every pointer argument is caller-owned DEVICE memory (q, k, v,
 * out, lse, seqstart_q, seqstart_k, alibi_slopes, workspace).  The library
 * allocates no memory in a call, keeps no caller pointer after a call
 * returns, and has no global mutable state apart from the thread-local error
 * text, per-device caches of the compute-unit count and of the address of
 * mea_fwd_noalloc's fixed scratch array, and that array (see there).
 *
 * Execution: the work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising.  Faults during
 * execution surface at the caller's next synchronisation, as for any HIP
 * kernel.  Calls on different streams may run concurrently; calls sharing a
 * workspace buffer must be ordered by the caller.
 *
 * Errors: arguments are validated before anything is enqueued; a non-OK
 * status means nothing was launched and no output byte was written (except
 * MEA_ERR_HIP, a launch failure reported by the HIP runtime).
 * mea_last_error() returns a thread-local description of the last non-OK
 * status of the calling thread.
 */
#ifndef MEA_H_
#define MEA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEA_ABI_VERSION 10

#if defined(__GNUC__)
#define MEA_EXPORT __attribute__((visibility("default")))
#else
#define MEA_EXPORT
#endif

typedef enum {
  MEA_OK = 0,
  MEA_ERR_INVALID = 1,      /* malformed argument (null pointer, bad sizes, workspace too small) */
  MEA_ERR_UNSUPPORTED = 2,  /* well-formed but outside what the kernels implement */
  MEA_ERR_HIP = 3           /* the HIP runtime refused a launch */
} mea_status_t;

typedef enum {
  MEA_F16 = 0,   /* IEEE binary16 in and out; scores and softmax in float32 */
  MEA_BF16 = 1   /* bfloat16 in and out; scores and softmax in float32 */
} mea_dtype_t;

/*
 * mea_fwd -- attention forward over packed sequences (definition above).
 *
 *   q, k, v        device inputs, layouts above, 16-byte aligned.
 *   out            device output [total_q, Hq, D], 16-byte aligned.  Rows of
 *                  sequences with L_q = 0 do not exist; every other row is
 *                  written.
 *   lse            device output [Hq, total_q] float32, or NULL to skip it.
 *   seqstart_q/k   device int32 [num_seqs + 1].  Preconditions (not checked:
 *                  checking would need a device synchronisation):
 *                  seqstart_*[0] == 0, non-decreasing, seqstart_q[num_seqs]
 *                  == total_q, seqstart_k[num_seqs] == total_k, and every
 *                  sequence length <= max_seqlen_q (resp. max_seqlen_k).
 *                  Violations read or write out of bounds.
 *   num_seqs       >= 0; 0 (or total_q == 0) is a no-op returning MEA_OK.
 *   total_q        number of packed query rows (the lse row stride).
 *   total_k        number of packed key/value rows (sizes the workspace).
 *   max_seqlen_q/k upper bounds of the per-sequence lengths (sizes the grid).
 *   Hq, Hkv        query / key-value heads; Hq % Hkv == 0.
 *   D              head dimension, 64 or 128 (q, k and v share it).
 *   dtype          MEA_F16 or MEA_BF16 (all of q, k, v, out).
 *   causal         0 or 1.
 *   alibi_slopes   device float32 [Hq] or NULL.
 *   scale          finite and > 0 (1/sqrt(D) is the usual choice).
 *   workspace      device scratch of at least mea_fwd_workspace_size(...)
 *                  bytes, 256-byte aligned; may be NULL when that size is 0.
 *                  Its contents on entry do not matter and are clobbered.
 *   stream         hipStream_t to enqueue on.
 *
 * Returns MEA_ERR_INVALID for: a NULL seqstart pointer, a NULL q or out with
 * total_q > 0, a NULL k or v with total_k > 0 (k and v are never read when
 * there are no keys; every query row then gets out = 0 and lse = -inf); negative
 * sizes; Hq or Hkv <= 0 or Hq % Hkv != 0; total_q > 0 with max_seqlen_q == 0;
 * causal not 0/1; a workspace smaller than required.
 * Returns MEA_ERR_UNSUPPORTED for: D not 64/128; dtype not listed; a
 * non-finite or non-positive scale; a pointer not aligned as stated;
 * num_seqs > 65535; max_seqlen_k * Hkv * D * 2 >= 2^31 (one sequence's
 * key/value rows are addressed with 32-bit byte offsets).
 *
 * Numerics: Q K^T runs on the matrix cores in the input dtype with float32
 * accumulation; the softmax is float32; the softmax weights enter P V as
 * IEEE halves, with bfloat16 V re-encoded as halves, which is exact for
 * 2^-14 <= |v| <= 65504.  Wherever a block of bfloat16 V holds a larger
 * magnitude, or only magnitudes below 2^-14 (where the re-encoding would
 * lose precision), that block keeps bfloat16 V and bfloat16 weights instead
 * (prefill: a 64-key tile, and then the whole query tile that reads it;
 * decode: a 32-key block of one wave), so any finite bfloat16 V is served.
 * out is rounded to nearest even from float32.
 */
MEA_EXPORT mea_status_t mea_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     const int32_t* seqstart_q, const int32_t* seqstart_k, int32_t num_seqs,
                     int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                     int32_t Hkv, int32_t D, mea_dtype_t dtype, int32_t causal,
                     const float* alibi_slopes, float scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * mea_fwd_mixed -- mea_fwd on a mixed batch of prefills and decode steps, as a
 * serving engine batches requests of different lengths (section 4 of the
 * 7minutos.es tutorial names vLLM-style batching as the use of packed
 * sequences): the first num_prefill_seqs sequences are prefills (any number
 * of queries), the remaining ones decode steps of exactly one query each.
 * Computes exactly what mea_fwd computes on the whole batch, but serves the
 * two parts with their own kernels, one after the other on `stream`: the
 * prefills with the tiled prefill kernels, the decode steps with the
 * split-KV kernels over their own keys (mea_fwd sends a batch with any
 * sequence of more than one query wholly to the prefill kernels, where a
 * decode step fills one row of a 64-token tile and one workgroup walks its
 * whole key history).
 *   num_prefill_seqs     sequences 0 .. num_prefill_seqs - 1 are the prefills
 *   prefill_total_q/k    seqstart_q[num_prefill_seqs] and
 *                        seqstart_k[num_prefill_seqs] (host copies)
 *   decode_max_seqlen_k  an upper bound of the decode sequences' key counts
 *   max_seqlen_q/k       as for mea_fwd (max_seqlen_q bounds the prefills)
 *   workspace            mea_fwd_mixed_workspace_size(...) bytes: the prefill
 *                        part's V^T images, then (256-byte aligned) the decode
 *                        part's partials
 * Other arguments, ownership and errors as for mea_fwd, plus MEA_ERR_INVALID
 * when num_prefill_seqs is outside [0, num_seqs], prefill_total_q/k outside
 * [0, total_q/k], decode_max_seqlen_k outside [0, max_seqlen_k], or total_q -
 * prefill_total_q differs from the number of decode sequences.  Preconditions
 * as for mea_fwd, plus: every decode sequence has exactly one query, and the
 * prefill_total_q/k values equal the device seqstart entries.
 */
MEA_EXPORT mea_status_t mea_fwd_mixed(const void* q, const void* k, const void* v, void* out, float* lse,
                                      const int32_t* seqstart_q, const int32_t* seqstart_k, int32_t num_seqs,
                                      int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int32_t num_prefill_seqs, int32_t prefill_total_q, int32_t prefill_total_k,
                                      int32_t decode_max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                                      mea_dtype_t dtype, int32_t causal, const float* alibi_slopes, float scale,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of mea_fwd_mixed (0 for arguments it would reject, or when
 * nothing is needed): the prefill part's mea_fwd_workspace_size-style V^T
 * images for sequences 0 .. num_prefill_seqs - 1 (prefill_total_k keys), then,
 * rounded up to 256 bytes, the decode part's partials for the other sequences
 * (total_k - prefill_total_k keys, pieces chosen as mea_default_chunk_keys
 * does for that key count).  Pure host function. */
MEA_EXPORT size_t mea_fwd_mixed_workspace_size(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q,
                                               int32_t max_seqlen_k, int32_t num_prefill_seqs,
                                               int32_t prefill_total_k, int32_t decode_max_seqlen_k, int32_t Hq,
                                               int32_t Hkv, int32_t D);

/*
 * mea_fwd_noalloc -- mea_fwd for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, computation and errors, without the
 * workspace.  The scratch it needs (the V^T tile images of a prefill call,
 * the float32 partials of a decode call: mea_fwd_workspace_size with the
 * same sizes and chunk_keys = 0) lives in one fixed device array of
 * MEA_NOALLOC_SCRATCH_BYTES per GPU, part of the library's device code:
 * every GPU the library runs on holds it until the process ends.  The call
 * allocates nothing and calls no hipMalloc or hipFree.
 *   stream   must belong to the current device (MEA_ERR_INVALID otherwise).
 * Returns MEA_ERR_UNSUPPORTED when the call needs more than
 * MEA_NOALLOC_SCRATCH_BYTES of scratch (mea_fwd with a caller workspace has
 * no such limit), and everything mea_fwd returns.
 * Every call on one GPU uses that GPU's one array: calls that may overlap on
 * one GPU (different streams, different host threads) race and must be
 * ordered by the caller.  The array keeps the last call's contents; no call
 * depends on them.
 */
#define MEA_NOALLOC_SCRATCH_BYTES (32u << 20)
MEA_EXPORT mea_status_t mea_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                        const int32_t* seqstart_q, const int32_t* seqstart_k, int32_t num_seqs,
                                        int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                                        int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                                        mea_dtype_t dtype, int32_t causal, const float* alibi_slopes, float scale,
                                        void* stream);

/*
 * mea_fwd_splitkv -- mea_fwd for the decode case (max_seqlen_q must be 1)
 * with the piece length of the key axis forced to `chunk_keys` (a positive
 * multiple of 32) instead of the library's choice.  The result does not
 * depend on the piece length beyond float32 rounding; this entry point exists
 * to test that.
 * Same arguments, ownership and errors as mea_fwd, plus MEA_ERR_INVALID for a
 * bad chunk_keys or max_seqlen_q != 1.
 */
MEA_EXPORT mea_status_t mea_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* seqstart_q, const int32_t* seqstart_k,
                             int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                             int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                             mea_dtype_t dtype, int32_t causal, const float* alibi_slopes,
                             float scale, void* workspace, size_t workspace_bytes, void* stream,
                             int32_t chunk_keys);

/*
 * mea_fwd_paged -- mea_fwd with K and V held in a paged cache.  Section 4 of
 * the 7minutos.es tutorial names vLLM-style batching of requests of
 * different lengths as the use of packed sequences; engines of that kind keep
 * K and V in pages addressed through a block table.  Computes exactly what
 * mea_fwd computes on the sequences' keys gathered into the packed layout.
 *   k_cache, v_cache  [num_pages, page_size, Hkv, D], 16-bit float of dtype
 *   block_table       int32 [num_seqs, max_blocks] device array: entry
 *                     [b, i] is the page holding keys i*page_size ..
 *                     (i+1)*page_size - 1 of sequence b
 *   seqstart_k        as for mea_fwd: the logical key offsets (sequence b
 *                     has seqstart_k[b+1] - seqstart_k[b] keys; total_k is
 *                     their sum), used for the work split only
 * page_size must be a positive multiple of 64.  Rows of a sequence's last
 * page past its length are never read.  Every block_table entry a sequence
 * uses should be in [0, num_pages); the table is device memory and is not
 * checked on the host, but the kernels never dereference an entry outside
 * that range (nor a block past max_blocks): its keys and values read as
 * zeros, so the call touches no memory outside the cache, and that
 * sequence's result is meaningless.
 * Workspace: mea_fwd_workspace_size with the same sizes.  Same ownership and
 * errors as mea_fwd, plus MEA_ERR_INVALID for a NULL block_table, a
 * non-positive page_size, num_pages or max_blocks, or max_blocks *
 * page_size < max_seqlen_k, and MEA_ERR_UNSUPPORTED for a page_size that is
 * not a multiple of 64 or a page of 2 GiB or more.
 */
MEA_EXPORT mea_status_t mea_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* out,
                           float* lse, const int32_t* seqstart_q, const int32_t* seqstart_k,
                           const int32_t* block_table, int32_t num_seqs, int32_t total_q,
                           int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int32_t page_size, int32_t num_pages, int32_t max_blocks, int32_t Hq,
                           int32_t Hkv, int32_t D, mea_dtype_t dtype, int32_t causal,
                           const float* alibi_slopes, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * mea_fwd_workspace_size -- bytes of workspace mea_fwd (chunk_keys == 0) or
 * mea_fwd_splitkv (chunk_keys > 0) needs for these sizes.  Pure host function;
 * returns 0 for arguments mea_fwd would reject.
 *   max_seqlen_q == 1 (decode): num_seqs * (ceil(max_seqlen_k / W) + 1) * Hq *
 *     (D + 1) * 4, W = the piece length (chunk_keys, or the library's choice
 *     mea_default_chunk_keys(total_k, Hq, Hkv)) -- float32 partial outputs
 *     and log-sum-exps; 0 when total_k or max_seqlen_k is 0;
 *   max_seqlen_q > 1 (prefill): with S = (total_k / 64 + num_seqs) * Hkv,
 *     round256(S * D * 128) + round256(S * 4) + 256 -- one transposed 16-bit
 *     copy of every 64-key tile of V, one int32 flag per copy, and the work
 *     counters of the prefill workgroups (round256 rounds up to a multiple of
 *     256; 0 when total_k == 0).
 */
MEA_EXPORT size_t mea_fwd_workspace_size(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q,
                                         int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                                         int32_t chunk_keys);

/*
 * mea_fwd_fp8 -- mea_fwd with q, k and v in 8-bit floating point (OCP FP8
 * E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 = NaN) and one scale per tensor.  Section 3 of
 * "大模型推理加速终极指南：xformers如何让Transformer性能飙升300%"
 * (zizhi168.cn) names FP8 among the supported formats of the attention's
 * mixed-precision pipeline and asks for the key steps in high precision.
 * Computes exactly what mea_fwd computes on the values
 *   q = q_scale * q8,  k = k_scale * k8,  v = v_scale * v8
 * (same masks, ALiBi, GQA and lse; scale multiplies q k^T as usual).
 * Precision: q8 k8^T runs on the fp8 matrix cores (each product exact, fp32
 * accumulation), scaled by scale * q_scale * k_scale in fp32; the softmax is
 * fp32; the weights enter P V as IEEE halves with v8 widened to halves
 * (exact), fp32 accumulation; v_scale and the 1/rowsum are applied in fp32
 * before the output is rounded to out_dtype (MEA_F16 or MEA_BF16).
 *   q, k, v        device, bytes, layouts as for mea_fwd ([T, H, D], one byte
 *                  per element), 16-byte aligned.
 *   q/k/v_scale    host floats, finite and > 0.
 *   out            device [total_q, Hq, D] of out_dtype.
 *   D              128 only (MEA_ERR_UNSUPPORTED otherwise).
 *   workspace      mea_fwd_fp8_workspace_size(num_seqs, total_k, max_seqlen_q,
 *                  max_seqlen_k, Hq, Hkv, D) bytes, 256-byte aligned.
 * Path choice as in mea_fwd: max_seqlen_q == 1 runs the split-KV decode
 * kernels (float32 partials in the workspace), anything else the prefill
 * kernel (half-precision V^T tile images in the workspace).  The decode pieces
 * are those of mea_default_chunk_keys(total_k, Hq, Hkv), except that with
 * Hkv a multiple of 8, workgroups take 8 key/value heads (whole 1 KiB token
 * rows) instead of 4 whenever the pieces for that grouping are still at least
 * 2048 keys long; mea_fwd_fp8_workspace_size follows the same choice.  K and V in a paged cache: mea_fwd_paged_fp8.
 * Same ownership and errors as mea_fwd, plus MEA_ERR_UNSUPPORTED for a
 * non-finite or non-positive scale.
 */
MEA_EXPORT mea_status_t mea_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                                    float v_scale, void* out, float* lse, const int32_t* seqstart_q,
                                    const int32_t* seqstart_k, int32_t num_seqs, int32_t total_q, int32_t total_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                                    mea_dtype_t out_dtype, int32_t causal, const float* alibi_slopes, float scale,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * mea_fwd_paged_fp8 -- mea_fwd_fp8 with K and V in a paged cache, as
 * mea_fwd_paged does for 16-bit K and V: a serving engine's fp8 KV cache.
 * Computes exactly what mea_fwd_fp8 computes on the sequences' keys gathered
 * into the packed layout.
 *   k_cache, v_cache  [num_pages, page_size, Hkv, D] OCP e4m3 codes (one byte
 *                     per element), 16-byte aligned
 *   block_table, page_size, num_pages, max_blocks, seqstart_k
 *                     as for mea_fwd_paged
 *   q, q/k/v_scale, out, out_dtype, D
 *                     as for mea_fwd_fp8
 * Decode-shaped calls (max_seqlen_q == 1) read 64-key blocks, each within
 * one page.  Workspace: mea_fwd_fp8_workspace_size with the same sizes.
 * Same ownership and errors as mea_fwd_fp8 and mea_fwd_paged together.
 */
MEA_EXPORT mea_status_t mea_fwd_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float q_scale,
                                          float k_scale, float v_scale, void* out, float* lse,
                                          const int32_t* seqstart_q, const int32_t* seqstart_k,
                                          const int32_t* block_table, int32_t num_seqs, int32_t total_q,
                                          int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                          int32_t page_size, int32_t num_pages, int32_t max_blocks, int32_t Hq,
                                          int32_t Hkv, int32_t D, mea_dtype_t out_dtype, int32_t causal,
                                          const float* alibi_slopes, float scale, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Workspace bytes of mea_fwd_fp8: mea_fwd_workspace_size(num_seqs, total_k,
 * max_seqlen_q, max_seqlen_k, Hq, Hkv, D, 0) for D == 128, else 0.  Pure host
 * function. */
MEA_EXPORT size_t mea_fwd_fp8_workspace_size(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q,
                                             int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D);

/*
 * mea_bwd -- gradients of the attention of mea_fwd: given dout = dL/dout for
 * some scalar L, writes dq = dL/dq, dk = dL/dk and dv = dL/dv.  The
 * yifor-blog page's performance comparison (xFormers vs standard attention)
 * times the backward pass of this attention beside the forward, and the
 * tutorial trains a GPT-style model with it; the pages give no formulas, so
 * this is the chain rule applied to the
 * definition above, per sequence b and query head h (g = g(h), P the softmax
 * weights, zero in rows with no allowed key):
 *   dv[g] += P^T dout[h]
 *   dP     = dout[h] v[g]^T
 *   dS     = P * (dP - rowsum(dout[h] * out[h]))     (rowsum(P * dP))
 *   dq[h]  = scale * dS k[g]
 *   dk[g] += scale * dS^T q[h]
 * summed over the query heads of g's group.  ALiBi slopes and masks are
 * constants; lse receives no gradient.
 *
 *   q, k, v, seqstart_q/k, sizes, Hq, Hkv, D, dtype, causal, alibi_slopes,
 *                  scale: exactly as passed to the mea_fwd call that produced
 *                  out and lse (same preconditions).
 *   out            device [total_q, Hq, D], the forward's output.
 *   lse            device [Hq, total_q] float32, the forward's log-sum-exp
 *                  (required: it is how P is recomputed without the score
 *                  matrix).
 *   dout           device [total_q, Hq, D], the upstream gradient.
 *   dq             device output [total_q, Hq, D]; every row is written.
 *   dk, dv         device outputs [total_k, Hkv, D]; every row is written
 *                  (zero for keys no query row sees).
 *   workspace      device scratch of at least mea_bwd_workspace_size(...)
 *                  bytes, 256-byte aligned; clobbered.
 * dtype applies to q, k, v, out, dout, dq, dk and dv; all 16-byte aligned.
 * Ownership and execution as for mea_fwd (outputs must not alias inputs).
 * Returns MEA_ERR_INVALID for a NULL pointer among seqstart_q/k, among q,
 * out, lse, dout, dq with total_q > 0, or among k, v, dk, dv with total_k > 0;
 * negative sizes; bad heads; causal not 0/1;
 * total_q > 0 with max_seqlen_q == 0 or total_k > 0 with max_seqlen_k == 0;
 * a workspace smaller than required.  MEA_ERR_UNSUPPORTED for D not 64/128,
 * an unknown dtype, a non-finite or non-positive scale, misalignment,
 * num_seqs > 65535, or max_seqlen * heads * D * 2 >= 2^31 for q or k.
 * num_seqs == 0, or total_q == total_k == 0, is a no-op returning MEA_OK.
 *
 * Numerics: S = q k^T and dP = dout v^T run on the matrix cores in the input
 * dtype with float32 accumulation; P and dS are float32 and are rounded to the
 * input dtype as operands of the second products (dv, dk, dq), which
 * accumulate in float32; rowsum(dout * out) is float32; outputs are rounded
 * to nearest even.
 */
MEA_EXPORT mea_status_t mea_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, const int32_t* seqstart_q,
                                const int32_t* seqstart_k, int32_t num_seqs, int32_t total_q, int32_t total_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                                mea_dtype_t dtype, int32_t causal, const float* alibi_slopes, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * mea_bwd_workspace_size -- bytes of workspace mea_bwd needs (0 for arguments
 * it would reject).  Pure host function: 2 x Hq * total_q * 4, each half
 * rounded up to a multiple of 256 bytes (float32 per-row terms: the
 * log-sum-exp in log2 units and rowsum(dout * out)); 0 when total_q == 0.
 */
MEA_EXPORT size_t mea_bwd_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t Hq,
                                         int32_t Hkv, int32_t D);

/*
 * mea_swiglu_ffn -- the SwiGLU feed-forward layer of the transformer block the
 * tutorials build around this attention: section 4 of the yifor-blog page's
 * optimisations replaces the ReLU/GELU feed-forward with a SwiGLU one (the
 * 7minutos.es title names it too).  The pages give no formula; this is the
 * gated form with the SiLU (swish) gate:
 *   hidden = SiLU(x w_gate^T) * (x w_up^T)       SiLU(z) = z / (1 + exp(-z))
 *   out    = hidden w_down^T
 *   x       [tokens, d_model]      w_gate, w_up [d_ff, d_model]
 *   hidden  [tokens, d_ff]         w_down       [d_model, d_ff]
 *   out     [tokens, d_model]
 * (weights in the out_features x in_features layout of a linear layer).  All
 * arrays are device memory of `dtype` (MEA_F16 or MEA_BF16), row-major and
 * 16-byte aligned; hidden is written (rounded to dtype) and is the input of
 * the second product.  Products run on the matrix cores in dtype with float32
 * accumulation; SiLU and the gate product are float32.
 * Returns MEA_ERR_INVALID for a NULL pointer, tokens < 0, d_model or d_ff <= 0;
 * MEA_ERR_UNSUPPORTED for another dtype, misalignment, d_model not a multiple
 * of 256 or d_ff not a multiple of 128 (or either above 65536).  tokens == 0
 * is a no-op.  Ownership and execution as for mea_fwd.
 */
MEA_EXPORT mea_status_t mea_swiglu_ffn(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                                       void* hidden, void* out, int32_t tokens, int32_t d_model, int32_t d_ff,
                                       mea_dtype_t dtype, void* stream);

/* Piece length of the key axis that mea_fwd picks for a decode call with
 * these sizes (a multiple of 32, at least 128).  Pure host function. */
MEA_EXPORT int32_t mea_default_chunk_keys(int32_t total_k, int32_t Hq, int32_t Hkv);

/* Static text for a status code. */
MEA_EXPORT const char* mea_status_string(mea_status_t status);

/* Thread-local detail for the calling thread's last non-OK status ("" if none). */
MEA_EXPORT const char* mea_last_error(void);

/* MEA_ABI_VERSION of the built library. */
MEA_EXPORT int32_t mea_abi_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* MEA_H_ */
