/*
 * va.h -- C ABI of the MI355X (gfx950) paged GQA target-verify attention library.
 *
 * The operation.  This is attention for speculative-decoding target
 * verification.  Each sequence has a short query block of 1..4 draft tokens
 * (bf16).  A group of G = Hq/Hkv query heads shares one kv head.  The query
 * attends causally over a paged KV cache of 16-token pages (FP8 e4m3fn or
 * bf16), with per-tensor k/v descale.  This is the call the sglang PR #36330
 * summary page shows ("Key source snippets": the aiter_backend.py shape gate
 * and the unified_attention_3d_mtp_func call, plus the test
 * _check_matches_aiter).
 *
 *   for sequence b with queries q[cu[b] .. cu[b+1]) and Lk = seqused_k[b] keys:
 *     query token t (0-based) sees keys j = 0 .. Lk - Lq + t   (bottom-right causal)
 *     s_j   = softmax_scale * k_descale * < q[t][h], K[j][h/G] >
 *     out[t][h] = v_descale * sum_j softmax(s)_j * V[j][h/G]
 *
 * The key range is split into segments whose partial softmax results are
 * merged by log-sum-exp.  That split is the PR #36330 page's, "Implementation
 * breakdown" item 1: a segmented main kernel plus a reduce-segments kernel.
 * Packing the G heads of a group over one load of each KV tile comes from the
 * same item and from the sglang PR #34517 summary page ("Motivation").
 *
 * Execution model.  va_plan() runs on the host once per problem shape.  It
 * checks the domain (the analogue of the page's shape gate and of can_handle on
 * the PR #34517 page), chooses kernels and launch shape, and sizes the
 * workspace.  va_run() only enqueues work on a HIP stream.  It reads every
 * length from device memory, and never synchronises or allocates, so it may be
 * captured in a HIP graph (the PR #30105 summary page, "Key source snippets",
 * notes that the seq_lens + draft addition must stay inside the captured graph).
 *
 * Ownership.  The caller owns every device buffer: q, pools, metadata, out,
 * workspace.  The library owns only the host-side plan object.  A plan is
 * immutable after creation.  va_run may run concurrently on different streams
 * if each call has its own workspace.
 *
 * Errors.  Functions return va_status.  Host-checkable mistakes (null
 * pointers, unsupported shapes, a short workspace) return an error and enqueue
 * nothing.  Device data (the lengths and the block table) is not validated in
 * va_run.  Invalid device data yields an undefined result, but the kernels
 * never access memory outside their buffers:
 *   - a sequence whose query rows leave [0, total_q) or number more than
 *     max_seqlen_q is treated as empty;
 *   - key lengths are clamped to the block-table row;
 *   - page ids are clamped to [0, num_blocks).
 * va_validate checks the device data explicitly (the VA_BAD_* rules below).
 *
 * Validate mode.  With the environment variable VA_DEBUG set (and not "0")
 * when va_plan runs, va_plan prints the plan to stderr, and every va_run of
 * that plan first runs va_validate on the call's metadata, waits for it, and
 * returns VA_ERR_DEVICE_DATA (with a line on stderr) instead of running the
 * attention if any rule fails.  That wait makes validate mode unusable under
 * HIP graph capture; it is a debugging aid.
 */
#ifndef VA_H
#define VA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VA_OK = 0,
    VA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent sizes */
    VA_ERR_UNSUPPORTED = 2,   /* outside the supported domain (see va_plan) */
    VA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than va_plan_workspace_bytes */
    VA_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
    VA_ERR_DEVICE_DATA = 5    /* validate mode (VA_DEBUG) found invalid device metadata */
} va_status;

typedef enum {
    VA_DT_BF16 = 1,           /* bfloat16 */
    VA_DT_FP8_E4M3FN = 2      /* OCP fp8 e4m3fn: bias 7, max 448, NaN = 0x7F/0xFF, no inf */
} va_dtype;

/*
 * Where the keys live.
 *   VA_LAYOUT_PAGED          16-token pages [num_blocks, 16, Hkv, 256] addressed by a
 *                            block table; the verify tokens' K/V are already in
 *                            the cache (va_run, va_run_ex).
 *   VA_LAYOUT_PREFIX_EXTEND  the layout of the sglang PR #34517 summary page's
 *                            shared-KV verify kernel ("Key source snippets"):
 *                            the prefix K/V are token rows of a buffer
 *                            [num_blocks * page_size, Hkv, 256] addressed by
 *                            per-token slots (kv_indptr / kv_indices), the
 *                            draft tokens' K/V sit in separate buffers with one
 *                            row per query token (va_run_prefix_extend).
 *                            max_blocks_per_seq is ignored.
 */
typedef enum { VA_LAYOUT_PAGED = 0, VA_LAYOUT_PREFIX_EXTEND = 1 } va_layout;

/* Shape of one verify-attention call.  All fields are host values. */
typedef struct {
    int32_t num_seqs;            /* B >= 1 */
    int32_t num_q_heads;         /* Hq */
    int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0 */
    int32_t head_dim;            /* D; must be 256 */
    int32_t page_size;           /* must be 16 */
    int32_t max_seqlen_q;        /* upper bound of any q_len; 1..4 */
    int32_t max_seqlen_k;        /* upper bound of any seqused_k (may be loose) */
    int32_t max_blocks_per_seq;  /* row stride of block_table (int32 elements) */
    int64_t num_blocks;          /* pages in each of the k and v pools */
    int64_t total_q;             /* rows of q / out; <= num_seqs * max_seqlen_q */
    int32_t q_dtype;             /* va_dtype; must be VA_DT_BF16 (out is bf16 too) */
    int32_t kv_dtype;            /* va_dtype of both pools */
    int32_t num_cus;             /* compute units to plan for; 0 = query the current device */
    int32_t force_grid;          /* 0 = automatic; 1 .. 65536 = number of split-KV
                                    workgroups (a testing hook: every value gives the same
                                    result up to floating-point merge order; larger values
                                    are VA_ERR_INVALID_ARG) */
    int32_t window_left;         /* sliding window: -1 = none; >= 0: the query at absolute
                                    position i also needs key j >= i - window_left (the
                                    window_size = (sliding_window - 1, 0) of the PR #30105
                                    page's verify call) */
    float softcap;               /* logit softcap: 0 = none; > 0: every scaled logit s is
                                    replaced by softcap * tanh(s / softcap) */
    int32_t layout;              /* va_layout of the KV cache (VA_LAYOUT_PAGED = 0) */
    int32_t v_head_dim;          /* value / output width; 0 = head_dim.  head_dim 576 with
                                    v_head_dim 512 is absorbed MLA (see below) */
    int32_t kernel;              /* split-KV kernel of a paged FP8 GQA call: 0 = automatic,
                                    1 = one wave per SIMD holding every row (best with many
                                    pages per workgroup), 2 = two row groups per key group
                                    (best with few).  Automatic picks 1 when the pages a
                                    workgroup can get, from max_seqlen_k (and the window),
                                    are at least 112.  Every choice gives the same result up
                                    to floating-point summation order.  Other layouts and
                                    dtypes take 0 only; other values are VA_ERR_INVALID_ARG. */
} va_problem;

typedef struct va_plan_s *va_plan_t;

/*
 * Check the problem and build a plan.
 * Supported domain (VA_ERR_UNSUPPORTED otherwise):
 *   - D = 256 and page 16; or absorbed MLA (below);
 *   - Q and out bf16; KV fp8 e4m3fn or bf16;
 *   - G = Hq/Hkv in {4, 8, 16}; 1 <= max_seqlen_q <= 4;
 *   - num_seqs * num_kv_heads <= 65536;
 *   - causal only, with an optional sliding window, logit softcap and attention
 *     sinks (window_left >= -1, softcap >= 0; else VA_ERR_INVALID_ARG).
 *   - With num_cus == 0, the current HIP device must be gfx950.
 * The domain is the PR #36330 page's gate (gfx950, q len 2..4, G = 16, D = 256,
 * page 16, bf16 Q, fp8 KV), widened:
 *   - q_len 1 and G = 4/8 are the local shapes of the PR #34517 page's tests;
 *   - bf16 KV is that page's other cache type;
 *   - any KV length is allowed (short ones just get one segment).
 * On success *out holds a new plan; release it with va_plan_destroy.
 */
va_status va_plan(const va_problem *problem, va_plan_t *out);

/*
 * Absorbed MLA: the PE_DIM split of the sglang PR #34517 summary page's
 * shared-KV verify kernel ("Key source snippets": q_nope.k_nope plus q_pe.k_pe,
 * with the latent width as NOPE_DIM in its absorbed-MLA layout).
 * head_dim = 576, v_head_dim = 512, num_kv_heads = 1, paged layout, no window
 * or softcap.  A cache row [num_blocks, 16, 1, 576] is [latent (512) | RoPE
 * part (64)]; q rows [total_q, Hq, 576] are [q_nope | q_pe]; the logit is the
 * dot product over the whole row times softmax_scale * k_descale; the value
 * of a key is its latent, so out is [total_q, Hq, 512] and va_run_ex must get
 * v_pool == k_pool (VA_ERR_INVALID_ARG otherwise) and no sinks.
 */

/* Bytes of device workspace va_run needs for this plan. */
va_status va_plan_workspace_bytes(va_plan_t plan, size_t *bytes);

/*
 * The split-KV kernel the plan runs for a paged FP8 GQA call, as in
 * va_problem.kernel: 1 = one wave per SIMD, 2 = two row groups; 0 for every
 * other call (bf16, prefix + extend, MLA).  VA_ERR_INVALID_ARG for null
 * pointers.
 */
va_status va_plan_kernel(va_plan_t plan, int32_t *kernel);

/* Number of split-KV workgroups the plan launches (after force_grid). */
va_status va_plan_grid(va_plan_t plan, int32_t *grid);

/*
 * Enqueue the verify attention on `stream` (a hipStream_t; NULL = the null stream).
 *
 *   q            [total_q, Hq, 256] bf16, contiguous
 *   k_pool       [num_blocks, 16, Hkv, 256] kv_dtype, contiguous
 *   v_pool       [num_blocks, 16, Hkv, 256] kv_dtype, contiguous
 *   block_table  [num_seqs, max_blocks_per_seq] int32; entry p = pool page of
 *                the sequence's logical page p (only the first ceil(seqused_k/16)
 *                entries of a row are read)
 *   cu_seqlens_q [num_seqs + 1] int32 prefix sums of the query lengths
 *   seqused_k    [num_seqs] int32 KV length of each sequence, verify tokens included
 *   softmax_scale  host float (head_dim**-0.5 for the standard scale)
 *   k_descale, v_descale  device pointers to one float each, or NULL for 1.0
 *   out          [total_q, Hq, 256] bf16, written for every query row
 *   workspace    device buffer of >= va_plan_workspace_bytes bytes, 256-byte
 *                aligned; its contents need not be initialised.  Calls that
 *                overlap in time must use different workspaces.
 * All device pointers must be 16-byte aligned.  Returns VA_OK once both kernels
 * (split-KV main kernel, segment reduce) are enqueued.
 */
va_status va_run(va_plan_t plan, const void *q, const void *k_pool, const void *v_pool,
                 const int32_t *block_table, const int32_t *cu_seqlens_q,
                 const int32_t *seqused_k, float softmax_scale,
                 const float *k_descale, const float *v_descale, void *out,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * va_run with its optional arguments, and one kernel at a time.
 *   sinks        device pointer to Hq floats, one sink logit per query head, or
 *                NULL for none.  A sink is a logit in the units of the scaled
 *                logits (softmax_scale * k_descale * q.k, natural log); it joins
 *                the softmax denominator and carries no value:
 *                out = v_descale * sum_j e^s_j V_j / (sum_j e^s_j + e^sink).
 *                Not softcapped.  (The PR #30105 page's verify call passes sinks
 *                to the attention kernel; the pages do not define them, this is
 *                the reading.)
 *   stage VA_STAGE_ALL:      both kernels, as va_run.
 *   stage VA_STAGE_SPLIT_KV: the split-KV main kernel.  It writes the per-segment
 *                            partials to the workspace, and writes rows whose
 *                            sequence fits one segment straight to out.
 *   stage VA_STAGE_MERGE:    the segment-reduce kernel; it reads the partials and
 *                            writes the remaining rows of out.
 * VA_STAGE_MERGE must follow VA_STAGE_SPLIT_KV of the same call on the same
 * stream (with the same workspace).  The single stages exist so a caller can
 * time or profile each kernel on its own.  Other arguments and errors as va_run;
 * an unknown stage is VA_ERR_INVALID_ARG.
 */
enum { VA_STAGE_ALL = 0, VA_STAGE_SPLIT_KV = 1, VA_STAGE_MERGE = 2 };
va_status va_run_ex(va_plan_t plan, int32_t stage, const void *q, const void *k_pool,
                    const void *v_pool, const int32_t *block_table,
                    const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                    float softmax_scale, const float *k_descale,
                    const float *v_descale, const float *sinks, void *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * va_run_ex (stage VA_STAGE_ALL) for a caller that measures the split-KV main
 * kernel inside whole calls: main_start and main_stop are hipEvent_t handles
 * (created by the caller with timing enabled) that the main kernel's dispatch
 * records itself (hipExtLaunchKernelGGL), so hipEventElapsedTime(main_start,
 * main_stop) is that kernel's execution time, with no separate event commands
 * between the two kernels of the call.  Paged-layout plans only (a prefix +
 * extend plan is VA_ERR_INVALID_ARG, as for va_run_ex).  Null events are
 * VA_ERR_INVALID_ARG.  Other arguments and errors as va_run_ex.
 */
va_status va_run_timed(va_plan_t plan, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *block_table, const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                       float softmax_scale, const float *k_descale, const float *v_descale,
                       const float *sinks, void *out, void *workspace, size_t workspace_bytes,
                       void *stream, void *main_start, void *main_stop);

/*
 * va_run_ex (stage VA_STAGE_ALL) with no workspace argument and no device
 * allocation, for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  The workspace is a fixed 80 MiB array in the library's own
 * device memory (one per device the library runs on, held until the process
 * ends), enough for every plan at the default grid (one workgroup per CU);
 * a plan whose va_plan_workspace_bytes exceeds it gets VA_ERR_WORKSPACE.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the array's device address is looked up once per device, on the
 * first call with that device current.  Every call on a device shares that
 * device's array, so calls that overlap in time on one device (other streams,
 * other threads) race on it and give undefined results; serialise them.
 * Paged-layout plans only.  Other arguments and errors as va_run_ex.
 */
va_status va_run_noalloc(va_plan_t plan, const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *block_table, const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                         float softmax_scale, const float *k_descale, const float *v_descale,
                         const float *sinks, void *out, void *stream);

/*
 * Diagnostic.  A library compiled with -DVA_STAMPS records, for every wave of
 * the FP8 paged main kernel, the GPU's constant 100 MHz clock at the phase
 * boundaries of its first piece (work located, Q landed, Q operands loaded,
 * first and second steps' pages landed, page loop done, epilogue phases) and at
 * exit, the phases of the piece's middle step (K landed, QK and softmax, V
 * landed, PV) with the shader clock counter around it, plus step, piece and
 * pass counts and the wave's XCD, into `buffer`: 32 uint64 words per wave, wave
 * kg (0..3) of workgroup w at (w * 4 + kg) * 32.
 * `buffer` is a device pointer of `bytes` bytes; runs whose grid does not fit
 * record nothing.  NULL turns recording off.  The setting is process-wide.
 * Without VA_STAMPS this returns VA_ERR_UNSUPPORTED and records nothing.
 */
va_status va_set_stamp_buffer(void *buffer, size_t bytes);

/*
 * Check one call's device metadata against the plan (the rules below), as
 * va_run would read it.  Every rule follows from the operation: query rows are
 * the prefix sums cu_seqlens_q, each sequence has at most max_seqlen_q of
 * them, its KV length bounds its causal key range, and every page it reads is
 * a page of the pools.  Bits of result[0] (sequence b, q_len = cu[b+1] - cu[b]):
 *   VA_BAD_CU_SEQLENS_Q  cu[0] != 0, or cu[b+1] < cu[b], or cu[b+1] > total_q
 *   VA_BAD_Q_LEN         cu is fine for b and q_len > max_seqlen_q
 *   VA_BAD_SEQUSED_K     seqused_k[b] < 0 or > max_seqlen_k
 *   VA_BAD_Q_GT_K        q_len > seqused_k[b] (q_len counted 0 where cu is bad):
 *                        a query token would sit before the first key
 *   VA_BAD_PAGE          an entry the sequence reads is outside [0, num_blocks).
 *                        It reads entries p with first <= p and 16 p < seqused_k,
 *                        where first = 0, or with a window
 *                        max(0, seqused_k - q_len - window_left) / 16.
 *                        Entries past those (padding) are never checked.
 * result[1] = the smallest sequence index that breaks a rule, num_seqs if none.
 *   result   device pointer to 2 int32 (4-byte aligned), written by the call
 *   others   as va_run
 * Two small kernels are enqueued on `stream`; the call does not wait.  Errors:
 * VA_ERR_INVALID_ARG (null or misaligned pointer), VA_ERR_HIP.
 */
enum {
    VA_BAD_CU_SEQLENS_Q = 1,
    VA_BAD_Q_LEN = 2,
    VA_BAD_SEQUSED_K = 4,
    VA_BAD_Q_GT_K = 8,
    VA_BAD_PAGE = 16
};
va_status va_validate(va_plan_t plan, const int32_t *block_table, const int32_t *cu_seqlens_q,
                      const int32_t *seqused_k, int32_t *result, void *stream);

/*
 * Verify attention in the prefix + extend layout (plan built with
 * layout = VA_LAYOUT_PREFIX_EXTEND), through the same kernels as va_run_ex.
 *   k_buffer, v_buffer [num_blocks * page_size, Hkv, 256] kv_dtype: token rows
 *   kv_indptr    [num_seqs + 1] int32: sequence b's prefix is kv_indices
 *                [kv_indptr[b], kv_indptr[b+1]); P_b = its length
 *   kv_indices   [num_kv_indices] int32: the buffer row of every prefix token,
 *                in key order (any rows: no page structure is assumed)
 *   k_extend, v_extend  [total_q, Hkv, 256] kv_dtype: the draft tokens' K/V,
 *                row cu_seqlens_q[b] + i = draft token i of sequence b (same
 *                dtype and descale as the buffers, as if already cached)
 *   others       as va_run_ex (stage, sinks, window, softcap included)
 * Sequence b has P_b + q_len keys: the prefix, then its draft tokens; query
 * token t sees the whole prefix and draft tokens 0..t (bottom-right causal, as
 * in va_run with seqused_k = P_b + q_len); max_seqlen_k bounds P_b + q_len.
 * Device data is not validated (validate mode covers the paged layout only);
 * a prefix range outside kv_indices counts as an empty sequence and slots are
 * clamped to the buffer rows, so no access leaves the buffers.
 * Errors: as va_run_ex; VA_ERR_INVALID_ARG also for a paged plan, a null
 * kv_indptr / k_extend / v_extend, num_kv_indices < 0 or > INT32_MAX - 16, or a
 * null kv_indices with num_kv_indices > 0.  va_run / va_run_ex reject a
 * prefix + extend plan the same way.
 */
va_status va_run_prefix_extend(va_plan_t plan, int32_t stage, const void *q, const void *k_buffer,
                               const void *v_buffer, const int32_t *kv_indptr, const int32_t *kv_indices,
                               int64_t num_kv_indices, const void *k_extend, const void *v_extend,
                               const int32_t *cu_seqlens_q, float softmax_scale, const float *k_descale,
                               const float *v_descale, const float *sinks, void *out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Release a plan (NULL is ignored). */
void va_plan_destroy(va_plan_t plan);

/* Static description of a status code. */
const char *va_status_str(va_status status);

/*
 * Draft-extend (EAGLE-style KV catch-up) metadata, converted on the device into
 * the block_table / seqused_k that va_run takes, so that call runs through the
 * same kernels as target verification.  This is the PR #30105 summary page's
 * draft_extend_v2 routing ("Key source snippets": seqused_k is the kv_indptr
 * difference; a 2D page table is built from the spec metadata).
 *   kv_indptr   [num_seqs + 1] int32, prefix sums of the KV token counts
 *   kv_indices  int32 pool slot of every KV token, sequence by sequence
 *               (slot = page * page_size + offset; pages are filled from
 *               offset 0, as a paged allocator hands them out)
 *   block_table [num_seqs, max_blocks_per_seq] int32, written: entry p = the
 *               page of token p * page_size, 0 past the sequence's last page
 *   seqused_k   [num_seqs] int32, written: kv_indptr[b + 1] - kv_indptr[b]
 * All pointers are device pointers; one kernel is enqueued on `stream`.  A
 * sequence longer than max_blocks_per_seq pages gets only the first pages
 * (invalid device data).  Errors: VA_ERR_INVALID_ARG (null pointer, sizes < 1),
 * VA_ERR_HIP.
 */
va_status va_spec_block_table(const int32_t *kv_indptr, const int32_t *kv_indices, int32_t num_seqs,
                              int32_t page_size, int32_t max_blocks_per_seq, int32_t *block_table,
                              int32_t *seqused_k, void *stream);

/*
 * Decode n fp8 e4m3fn bytes to bf16 bits on the device, with the same in-register
 * conversion the attention kernel uses on K and V.  It is a diagnostic that
 * checks the dequant step over all 256 codes.  Both pointers are device
 * pointers; the call enqueues one kernel on `stream`.
 */
va_status va_fp8_to_bf16(const uint8_t *in, uint16_t *out, int64_t n, void *stream);

/*
 * Diagnostic: the streaming ceiling of the FP8 paged kernel's copy path.
 * Copies npages 4 KiB pages, pool + 4096 * pages[i] (device int32 page
 * indices; one outside [0, pool_bytes / 4096) is clamped into it), into
 * LDS with the kernel's global_load_lds copies (nontemporal), grid
 * workgroups of four waves, each wave an equal contiguous share of the list
 * in order with depth (2, 4, 6, 8 or 10) pages in flight, and no other work.
 * sums[grid * 4] (device) receives, per wave, the sum of the first 32-bit
 * word of every page it copied (for a check).  Returns VA_ERR_INVALID_ARG for
 * null pointers, a pool not 16-byte aligned or shorter than one page, an
 * unsupported depth, or grid outside [1, 65536].  The caller owns every
 * buffer; asynchronous on stream.
 */
va_status va_stream_pages(const void *pool, int64_t pool_bytes, const int32_t *pages, int64_t npages,
                          int32_t depth, int32_t grid, uint32_t *sums, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VA_H */
