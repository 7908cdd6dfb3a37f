/*
 * mla_fp8.h -- C ABI of libmla_fp8.so: FP8 MLA context prefill for gfx950 (MI355X).
 *
 * The operations follow the vLLM pull request "[ROCm][MLA] Add guarded gfx942
 * FP8 context prefill" (#51551): a one-kernel static per-head FP8 quantizer
 * (Summary; "What this PR does"), a packed variable-length attention kernel for
 * 12 heads with D192 Q/K and D128 V that keeps the model's attention boundary
 * (Background; "What this PR does"), and context processed in segments with Q
 * quantized once and its per-head scale reused ("What this PR does"), whose
 * partial results are combined by a log-sum-exp merge.
 *
 * Conventions for every entry point
 *   - Plain C: no C++ types and no exceptions cross this boundary.
 *   - Device pointers are borrowed for the duration of the asynchronous call.
 *     The library allocates nothing, keeps no pointer, creates no stream and
 *     never synchronizes; work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream).
 *   - Every scalar argument and pointer is checked on the host before any HIP
 *     call; a failed check returns a status and launches nothing. There is no
 *     silent fallback: unsupported shapes return MLA_ERR_UNSUPPORTED so that the
 *     caller can take its own BF16 path (the pull request keeps BF16 for
 *     unsupported shapes). A launch failure returns MLA_ERR_HIP.
 *   - mla_last_error() gives a thread-local text for the last failure.
 *   - Empty work (zero tokens, zero sequences) returns MLA_OK and launches nothing.
 *   - Values the host cannot see without a device-to-host copy (cu_seqlens
 *     contents, descale values in device memory) are the caller's contract.
 *     Kernels clamp every sequence range to [0, total), so malformed cu_seqlens
 *     give wrong numbers, never an out-of-bounds access.
 *   - FP8 is OCP E4M3FN (finite maximum 448, no infinities); bf16 is the
 *     upper half of IEEE binary32.
 */
#ifndef MLA_FP8_H
#define MLA_FP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_FP8_ABI_VERSION 1

enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad descale, ... */
  MLA_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement  */
  MLA_ERR_HIP = 3               /* the HIP runtime reported an error              */
};

/* Library ABI version (MLA_FP8_ABI_VERSION at build time). */
int mla_abi_version(void);

/* Static text for a status code; never NULL. */
const char* mla_status_string(int status);

/* Thread-local text describing the last failure in this thread ("" if none). */
const char* mla_last_error(void);

/* ------------------------------------------------------------------------ */
/* Static per-head quantizer                                                 */
/* ------------------------------------------------------------------------ */

/*
 * One tensor for mla_fp8_quant_static.
 *   x        device, bf16, logical [n_tokens, n_heads, head_dim]; element
 *            (t, h, d) at x + t*stride_token + h*stride_head + d (strides in
 *            elements; the last dimension is contiguous). Token and head
 *            strides let non-contiguous views be quantized in place.
 *   descale  device, fp32 [n_heads]; must be finite, positive, in
 *            [2^-126, 2^126] (check with mla_check_descales_host).
 *   y        device, E4M3 codes, contiguous [n_tokens, n_heads, head_dim].
 *   head_dim 192 (Q, K) or 128 (V), else MLA_ERR_UNSUPPORTED.
 */
typedef struct mla_quant_job {
  const void* x;
  int64_t stride_token;
  int64_t stride_head;
  int64_t n_tokens;
  int32_t head_dim;
  const float* descale;
  void* y;
} mla_quant_job;

/*
 * Quantize 1..3 tensors (Q, K, V or K, V) in ONE kernel launch:
 *   y[t,h,d] = E4M3(x[t,h,d] / descale[h])
 * E4M3 is the correctly rounded value of the exact quotient: round to nearest,
 * ties to even; |quotient| > 448 (and +-Inf) saturates to +-448; NaN gives
 * 0x7F with the input's sign; the sign of zero and of underflow is kept.
 * Follows "[ROCm][MLA] Add guarded gfx942 FP8 context prefill", Summary and
 * "What this PR does" (one-kernel static quantizer, no runtime amax).
 * Fast path: x 16-byte aligned and both strides multiples of 8 elements;
 * other strides take a slower element-wise path. y must be 16-byte aligned.
 */
int mla_fp8_quant_static(const mla_quant_job* jobs, int32_t n_jobs, int32_t n_heads,
                         void* stream);

/*
 * Dynamic per-head quantization: the per-head amax reduction that the static
 * path removes ("[ROCm][MLA] Add guarded gfx942 FP8 context prefill", Summary),
 * kept as the baseline to compare with. For each job j and head h:
 *   amax = max |x[t,h,d]| over the job's tokens and dims,
 *   descale = RN_fp32(amax / 448) floored at 2^-126 (so 1/descale stays finite),
 *             or 1 when the head is all zeros (any positive descale gives the same codes),
 *   y[t,h,d] = E4M3(x[t,h,d] / descale), exactly as mla_fp8_quant_static.
 *   jobs         as for mla_fp8_quant_static; jobs[j].descale is not read.
 *   descale_out  device fp32 [n_jobs * n_heads], caller-owned: receives descale of
 *                (j, h) at j * n_heads + h (usable as the descales of the prefill).
 *                It holds the amax during the call.
 * Inputs must be finite: a NaN or Inf element makes its head's descale non-finite and
 * its codes unspecified (no error is raised; the device does not report back).
 * Four launches on stream (zero, amax reduction, quantize, descale); HBM traffic
 * 5 bytes per element (2 read twice, 1 written) against 3 for the static path.
 * Errors as for mla_fp8_quant_static, and MLA_ERR_INVALID_ARGUMENT for a NULL descale_out.
 */
int mla_fp8_quant_dynamic(const mla_quant_job* jobs, int32_t n_jobs, int32_t n_heads,
                          float* descale_out, void* stream);

/*
 * Calibration: amax[h] = max |x[t,h,d]| over all tokens and dims (device fp32
 * [n_heads], overwritten). Bit-exact (max does not depend on order). The
 * pull request collects per-head maxima in a calibration pass ("What this PR
 * does"); this is that reduction for one tensor. Same x layout and
 * alignment rules as mla_quant_job. n_tokens == 0 writes zeros.
 */
int mla_fp8_amax_per_head(const void* x, int64_t stride_token, int64_t stride_head,
                          int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                          float* amax, void* stream);

/*
 * Un-absorbed MLA K/V producer fused with the static quantizer. vLLM #60110,
 * Purpose: prefill keeps the un-absorbed form, in which keys and values are
 * expanded from the latent cache per head (latent rank 512; the 192-wide key head
 * ends in the 64-dim rope part; 12 heads per rank). The codes follow
 * mla_fp8_quant_static's contract.
 *
 *   c_kv          device bf16 latent rows, row t at c_kv + t * c_kv_stride (elements);
 *                 the first 512 elements of a row are used
 *   k_pe          device bf16 rope keys (already rotated), row t at k_pe + t * k_pe_stride;
 *                 the first 64 elements are used, shared by every head
 *   w_kv_b        device bf16 [n_heads * 256, 512], row-major: rows 256h .. 256h+127 are
 *                 W_UK[h] (the no-rope key part), rows 256h+128 .. 256h+255 are W_UV[h]
 *   descale_k/v   device fp32 [n_heads], finite and positive
 *   k8, v8        device E4M3 codes, contiguous [n_tokens, n_heads, 192] and [.., 128]
 *   k_bf16/v_bf16 NULL, or device bf16 [n_tokens, n_heads, 192] / [.., 128] that receive
 *                 the same K and V before quantization (for a BF16 attention path)
 *
 *   k_nope[t,h,i] = RN_bf16(sum_j W_UK[h][i][j] * c_kv[t][j]), v[t,h,i] likewise with
 *   W_UV[h], K[t,h] = [k_nope[t,h] | k_pe[t]], k8 = E4M3(K / descale_k[h]),
 *   v8 = E4M3(v / descale_v[h]) (exact quotient, nearest even, saturating). The sums
 *   accumulate in fp32 on the matrix cores, so a bf16 value can differ by one ulp from
 *   the rounding of the exact sum where that sum lies within the accumulation error of
 *   a bf16 rounding boundary; the codes are exact for the bf16 values produced.
 *   kv_lora_rank != 512 or rope_dim != 64 -> MLA_ERR_UNSUPPORTED. NULL pointers,
 *   pointers not 16-byte aligned, strides below the row length, not multiples of 8 or
 *   >= 2^24 -> MLA_ERR_INVALID_ARGUMENT. n_tokens == 0 succeeds without a launch.
 */
int mla_fp8_kv_produce(const void* c_kv, int64_t c_kv_stride, const void* k_pe,
                       int64_t k_pe_stride, const void* w_kv_b, int64_t n_tokens,
                       int32_t n_heads, int32_t kv_lora_rank, int32_t rope_dim,
                       const float* descale_k, const float* descale_v, void* k8, void* v8,
                       void* k_bf16, void* v_bf16, void* stream);

/* ------------------------------------------------------------------------ */
/* Varlen context-prefill attention                                          */
/* ------------------------------------------------------------------------ */

/*
 * FP8 attention over packed variable-length sequences, returning out and LSE.
 * Follows "[ROCm][MLA] Add guarded gfx942 FP8 context prefill", Background
 * (packed variable-length D192/V128 kernel) and "What this PR does" (12 heads,
 * D192 Q/K, D128 V, FP8 Q/K/V with per-head scales).
 *
 *   q, k, v       device E4M3 codes, contiguous [total_q, n_heads, 192],
 *                 [total_k, n_heads, 192], [total_k, n_heads, 128]; 16-byte aligned
 *   cu_seqlens_q  device int32 [batch + 1], sequence b has query tokens
 *   cu_seqlens_k  [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key tokens
 *                 [cu_seqlens_k[b], cu_seqlens_k[b+1]); non-decreasing, last = total
 *   max_seqlen_q  >= every query length (sets the grid; longer rows are not computed)
 *   descale_q/k/v device fp32 [n_heads]: dequantized value = code value * descale
 *   softmax_scale finite, > 0; logits are softmax_scale * <q_i, k_j> (dequantized)
 *   causal        0: every key visible; 1: key j visible to query i iff
 *                 j <= i + (Lk - Lq) (bottom-right aligned; the plain lower
 *                 triangle when Lq == Lk)
 *   out           device bf16 [total_q, n_heads, 128], caller-allocated, 16-byte aligned:
 *                 out_i = sum_j softmax_ij * v_j (dequantized)
 *   lse           device fp32, NULL or [n_heads, lse_stride] (lse_stride >= total_q):
 *                 lse[h*lse_stride + i] = ln sum_j exp(logit_ij)
 *   A query row with no visible key gets out = 0 and lse = -inf.
 *   head_dim_qk/head_dim_v other than 192/128 -> MLA_ERR_UNSUPPORTED.
 *   Any n_heads >= 1 is accepted (heads are independent; the workloads use 12).
 *   Grids of at most one 256-row workgroup per two CUs (ceil(max_seqlen_q / 256) * batch
 *   * n_heads <= half the device's CU count), causal grids of at most one per CU whose
 *   first query tile sees at most half the keys of the last, and packed batches whose
 *   grid is more than a quarter padding (sequences of unequal lengths) run on 128-row
 *   workgroups; results are bitwise the same. The environment variable
 *   MLA_FP8_PREFILL_SMALL_GRID, read at each call: 0 keeps every call on 256-row
 *   workgroups, 1 also runs every grid of at most one 256-row workgroup per CU on
 *   128-row ones.
 */
int mla_fp8_prefill_varlen(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int64_t total_q, int64_t total_k, int32_t n_heads,
                           int32_t head_dim_qk, int32_t head_dim_v,
                           const float* descale_q, const float* descale_k,
                           const float* descale_v, float softmax_scale, int32_t causal,
                           void* out, float* lse, int64_t lse_stride, void* stream);

/*
 * BF16 comparator: the same attention on bf16 Q/K/V, with no quantization and no
 * scales. The close comment of the pull request measures the FP8 kernel against
 * the BF16 attention that already covers D192/V128 (faster on the non-causal
 * chunk shape, slower on both causal shapes); this is that comparison's other side,
 * on the same MFMA blocking as mla_fp8_prefill_varlen.
 *
 *   q, k, v       device bf16, contiguous [total_q, n_heads, 192], [total_k, n_heads, 192],
 *                 [total_k, n_heads, 128]; 16-byte aligned; finite values
 *   cu_seqlens_q/k, batch, max_seqlen_q/k, total_q/k, n_heads, head dims, softmax_scale,
 *   causal, out, lse, lse_stride, stream: as for mla_fp8_prefill_varlen (logits are
 *                 softmax_scale * <q_i, k_j> of the bf16 values).
 *   Errors as for mla_fp8_prefill_varlen.
 */
int mla_bf16_prefill_varlen(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int64_t total_q, int64_t total_k, int32_t n_heads,
                            int32_t head_dim_qk, int32_t head_dim_v, float softmax_scale,
                            int32_t causal, void* out, float* lse, int64_t lse_stride,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* LSE merge across context segments                                         */
/* ------------------------------------------------------------------------ */

/*
 * Combine n_segments partial results over disjoint key sets:
 *   L = ln sum_s exp(L_s),   out = sum_s exp(L_s - L) * out_s
 * (segments with L_s = -inf get weight 0; all -inf gives out = 0, L = -inf).
 * The pull request reuses one quantized Q across context segments and keeps a
 * per-chunk output buffer ("What this PR does"); the merge rule is the
 * log-sum-exp identity for softmax over a union of key sets.
 *
 *   outs        host array of n_segments device pointers, bf16 [total_q, n_heads, 128],
 *               16-byte aligned
 *   lses        host array of n_segments device pointers, fp32 [n_heads, lse_in_stride]
 *   out         device bf16 [total_q, n_heads, 128]; may be exactly one of outs[s]
 *   lse_out     device fp32 [n_heads, lse_out_stride] or NULL; may be exactly one of
 *               lses[s] when lse_out_stride == lse_in_stride
 *   1 <= n_segments <= 64; head_dim_v must be 128.
 */
int mla_merge_lse(int32_t n_segments, const void* const* outs, const float* const* lses,
                  int64_t lse_in_stride, int64_t total_q, int32_t n_heads,
                  int32_t head_dim_v, void* out, float* lse_out, int64_t lse_out_stride,
                  void* stream);

/* ------------------------------------------------------------------------ */
/* Chunked-context prefill (one sequence)                                    */
/* ------------------------------------------------------------------------ */

/*
 * Attention of Lq queries that are the last Lq of Lk tokens (bottom-right
 * causal alignment; causal = 0: every key visible), computed over context
 * segments of seg_len keys with ONE quantized Q, partials merged by the
 * log-sum-exp rule of mla_merge_lse. Follows "[ROCm][MLA] Add guarded gfx942 FP8
 * context prefill", "What this PR does" (Q quantized once per context pass, its
 * per-head scale reused across context segments). The segmentation (not given on
 * the pages): queries in chunks of seg_len rows; cached keys [0, Lk - Lq) in
 * segments of seg_len, seen in full by every query; for query chunk [r0, r1) the
 * own keys [Lk-Lq, Lk-Lq+r0) in segments of seg_len seen in full, then the diagonal
 * [Lk-Lq+r0, Lk-Lq+r1) as a causal call. Each query chunk is ONE kernel launch over
 * all its segments, which also merges them: the last workgroup of every (256-row
 * query tile, head) to finish combines the segments' partials. Adjacent non-causal
 * segments of a query chunk are attended as one range when the launch keeps at least
 * four workgroups per CU that way (the merge is associative). Partials stay in fp32
 * (workspace) and the merged output is rounded to bf16 once. The result equals
 * mla_fp8_prefill_varlen on the whole sequence up to rounding. With causal = 0 and
 * seg_len >= Lq this is split-KV attention: one launch that spreads every (query
 * tile, head) over the key segments.
 *
 *   q, k, v     device E4M3, contiguous [Lq, H, 192], [Lk, H, 192], [Lk, H, 128]
 *   out, lse    as mla_fp8_prefill_varlen (lse may be NULL; lse_stride >= Lq)
 *   workspace   device scratch of mla_fp8_chunked_workspace_size() bytes, 16-byte
 *               aligned (may be NULL when that size is 0); contents are overwritten;
 *               calls that share a workspace must not overlap in time
 *   causal = 1 requires Lk >= Lq. At most 64 segments per query chunk
 *   (MLA_ERR_UNSUPPORTED beyond). Enqueues one launch per query chunk on `stream`,
 *   after one small launch that clears the merge counters in the workspace.
 */
int mla_fp8_prefill_chunked(const void* q, const void* k, const void* v, int64_t lq, int64_t lk,
                            int32_t n_heads, const float* descale_q, const float* descale_k,
                            const float* descale_v, float softmax_scale, int32_t seg_len,
                            int32_t causal, void* out, float* lse, int64_t lse_stride,
                            void* workspace, uint64_t workspace_bytes, void* stream);

/* Workspace bytes that mla_fp8_prefill_chunked needs for these sizes (host only). */
int mla_fp8_chunked_workspace_size(int64_t lq, int64_t lk, int32_t n_heads, int32_t seg_len,
                                   int32_t causal, uint64_t* bytes);

/* Device scratch held by the library for mla_fp8_prefill_chunked_noalloc, per GPU. */
#define MLA_FP8_NOALLOC_SCRATCH_BYTES (64ll * 1024 * 1024)

/*
 * mla_fp8_prefill_chunked for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, the same plan and arithmetic. Its fp32 partials,
 * partial LSEs and merge counters live in a library-owned device array of
 * MLA_FP8_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds until
 * the process ends; the call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine). The scratch of the current device (hipGetDevice, which must be the
 * device of `stream`) is looked up on the first call on that device.
 *   When a query chunk's partials do not fit the scratch, its rows are processed in
 *   several launches of a multiple of 256 rows each (every row's result is computed the
 *   same way; only the grouping of adjacent context segments may differ). A plan whose
 *   partials for 256 rows do not fit (64 MiB < parts * 256 * n_heads * 516 bytes, e.g.
 *   more than 42 parts at 12 heads) returns MLA_ERR_UNSUPPORTED.
 *   The merge counters are cleared at the start of every call. All calls on one GPU
 *   share its scratch: calls that overlap in time on one GPU (several streams or host
 *   threads) race and give wrong results.
 *   Errors as for mla_fp8_prefill_chunked; MLA_ERR_HIP if the scratch cannot be found.
 */
int mla_fp8_prefill_chunked_noalloc(const void* q, const void* k, const void* v, int64_t lq,
                                    int64_t lk, int32_t n_heads, const float* descale_q,
                                    const float* descale_k, const float* descale_v,
                                    float softmax_scale, int32_t seg_len, int32_t causal,
                                    void* out, float* lse, int64_t lse_stride, void* stream);

/* ------------------------------------------------------------------------ */
/* Host-only helpers (no device access; usable without a GPU)                */
/* ------------------------------------------------------------------------ */

/* MLA_OK if all n descales are finite, positive and in [2^-126, 2^126], else
 * MLA_ERR_INVALID_ARGUMENT (the pull request validates finite positive descales
 * before use: "What this PR does"). */
int mla_check_descales_host(const float* descale, int32_t n);

/* descale_out[i] = amax[i] / 448 in IEEE fp32 (correctly rounded); every amax
 * must be finite and > 0, else MLA_ERR_INVALID_ARGUMENT and nothing is written. */
int mla_descale_from_amax_host(const float* amax, int32_t n, float* descale_out);

#ifdef __cplusplus
}
#endif

#endif /* MLA_FP8_H */
