/*
 * attn.h -- C ABI of libattn.so: exact scaled-dot-product attention for one
 * AMD Instinct MI355X (gfx950), computed blockwise without materialising the
 * S x T score matrix.
 *
 *   O = softmax(scale * Q K^T + mask) V,   lse = log sum_j exp(scale * q.k_j)
 *
 * Conventions shared by every call
 *  - Sizes are element counts.  Tensors are dense, C-contiguous, in the
 *    layouts given per call.  Every pointer is owned by the caller; the
 *    library keeps none after the call returns.
 *  - Device calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *    null stream).  A kernel fault surfaces at the caller's next
 *    synchronisation.  Outputs must not alias inputs.
 *  - Arguments are validated before anything is launched; on any non-OK
 *    status nothing has been written.  attn_last_error() then returns a
 *    message for the calling thread.
 *  - Grouped-query attention: G = Hq / Hkv (Hq must be a multiple of Hkv) and
 *    query head h reads KV head floor(h / G).  (Opt-GQA: LLM-CoOpt summary,
 *    "Methodology" item 2; the head-to-group mapping itself is not on the
 *    page: contiguous groups are the reading taken.)
 *  - Causal masking is bottom-right aligned: with S queries and T keys,
 *    query i sits at absolute position i + T - S and sees key j iff
 *    j <= i + T - S (absolute position = past length + local index: ONNX
 *    Runtime PR #33328 analysis, section 1).  A query row that sees no key
 *    gets O = 0 and lse = -inf.
 *  - lse is the natural-log log-sum-exp of the scaled scores of the visible
 *    keys; it is what makes partial results mergeable (ONNX Runtime PR
 *    #28695 analysis, section 2, reduce phase).
 *  - Supported head dims: D = 64 or 128.  scale is explicit; callers
 *    usually pass 1/sqrt(D).
 *  - B == 0 or S == 0 (or R == 0) is a no-op returning ATTN_OK.
 *  - Alignment: the kernels move data in 16-byte vectors, so the q, k, v and
 *    o device pointers of the prefill calls, and the q, k_cache and v_cache
 *    pointers of the decode calls, must be 16-byte aligned; every other
 *    device pointer (fp32 outputs, scales, lse, page tables, lengths) needs
 *    its natural 4-byte alignment.  A misaligned pointer is rejected with
 *    ATTN_E_INVALID before anything is launched.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_E_INVALID = 1,     /* null required pointer, bad size, Hq % Hkv != 0, non-finite scale,
                             non-pinned host memory, workspace too small */
  ATTN_E_UNSUPPORTED = 2, /* head dim or dtype not supported by this call */
  ATTN_E_BUDGET = 3,      /* attn_stream_*: the smallest sub-task does not fit the budget */
  ATTN_E_DEVICE = 4       /* HIP launch, allocation or copy error */
} attn_status;

typedef enum attn_dtype {
  ATTN_F32 = 0,       /* IEEE binary32 */
  ATTN_BF16 = 1,      /* bfloat16 (upper half of binary32) */
  ATTN_FP8_E4M3 = 2,  /* OCP 8-bit E4M3 "fn": bias 7, no infinities, 0x7F/0xFF are NaN */
  ATTN_INT8 = 3,      /* signed 8-bit code, value = code * scale */
  ATTN_INT4 = 4       /* signed 4-bit two's-complement codes, two per byte (element 2i in the low
                         nibble of byte i, 2i+1 in the high nibble); value = code * the scale of
                         the element's 32-element group.  KV caches of attn_decode_* only. */
} attn_dtype;

/*
 * Tiled prefill: exact attention of S queries against T keys per sequence,
 * one pass over K/V tiles with an online softmax (running row max and sum),
 * the P.V product accumulated in fp32.  (Tiled computation with online
 * softmax and fused SV accumulation: ONNX Runtime PR #28695 analysis,
 * section 1; GQA: LLM-CoOpt "Methodology" item 2.)
 *
 *   dt      ATTN_F32 (fp32 inputs, fp32 arithmetic) or ATTN_BF16 (bf16
 *           inputs, bf16 matrix-core products, fp32 accumulation/softmax).
 *   q       device, [B, S, Hq, D] of dt
 *   k, v    device, [B, T, Hkv, D] of dt
 *   causal  0 or 1 (bottom-right, see above)
 *   scale   > 0 (the kernels scale each row's maximum raw score)
 *   o       device, [B, S, Hq, D] fp32 (written)
 *   lse     device, [B, Hq, S] fp32 (written), or NULL
 * Errors: ATTN_E_INVALID, ATTN_E_UNSUPPORTED (D, dt), ATTN_E_DEVICE.
 * T == 0 gives O = 0, lse = -inf.
 */
attn_status attn_prefill(attn_dtype dt, const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                         int64_t S, int64_t T, int D, int causal, float scale, float* o, float* lse, void* stream);

/*
 * Tiled prefill with OCP e4m3fn (fp8) Q, K and V and per-head scales:
 *   O = softmax(scale * (q_scale[h] q)(k_scale[hk] k)^T + mask) (v_scale[hk] v).
 * Q.K^T runs on the fp8 matrix cores; the softmax weights are rounded to bf16
 * for the P.V product (as in ATTN_BF16 prefill), with V's e4m3 values
 * converted exactly to bf16.  (FP8 operands halving the bytes per token:
 * LLM-CoOpt "Methodology" item 1; tiling and online softmax as attn_prefill.)
 *
 *   q        device, [B, S, Hq, D] e4m3fn bytes
 *   k, v     device, [B, T, Hkv, D] e4m3fn bytes
 *   q_scale  device fp32 [Hq]; k_scale, v_scale device fp32 [Hkv]; all > 0
 *   other arguments as attn_prefill (scale > 0).
 * Errors: ATTN_E_INVALID (incl. null scales), ATTN_E_UNSUPPORTED (D), ATTN_E_DEVICE.
 */
attn_status attn_prefill_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                             const float* k_scale, const float* v_scale, int B, int Hq, int Hkv, int64_t S,
                             int64_t T, int D, int causal, float scale, float* o, float* lse, void* stream);

/*
 * Workspace bytes attn_decode_splitkv needs for these sizes (num_splits as
 * passed to it; 0 = automatic).  Pure host arithmetic; no device access.
 */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_kv_len, int num_splits);

/*
 * Split-KV ("flash") decoding of one query token per sequence against a KV
 * cache: the KV sequences of all (sequence, KV head) pairs, laid end to end
 * in 16-token groups, are cut into equal runs, one per work unit; each piece
 * of a sequence yields a normalised partial output and its lse, and the
 * pieces are merged exactly by log-sum-exp.  (Flash decoding: ONNX Runtime PR #28695
 * analysis, section 2; 512-token pages: LLM-CoOpt "Methodology" item 3;
 * FP8 / INT8 / INT4 caches dequantised on the fly: LLM-CoOpt "Methodology"
 * item 1, ONNX Runtime PR #28695 analysis, introduction and section 1.)
 *
 *   kv_dt       ATTN_BF16, ATTN_INT8, ATTN_FP8_E4M3 or ATTN_INT4 (element type of the caches)
 *   q           device, [B, Hq, D] bf16
 *   k_cache,
 *   v_cache     device.  Paged (page_table != NULL): [num_pages, Hkv, page_size, D].
 *               Contiguous (page_table == NULL): [B, Hkv, page_size, D], i.e.
 *               one page of page_size >= max_kv_len tokens per sequence.
 *               int4: the last dimension is D/2 bytes.
 *   k_scale,
 *   v_scale     device fp32.  int8: per token and KV head, shaped like the
 *               cache without D ([num_pages or B, Hkv, page_size]).
 *               fp8: per KV head, [Hkv].  int4: per 32-element group,
 *               [num_pages or B, Hkv, page_size, D/32].  bf16: NULL.
 *   page_table  device int32 [B, max_pages]: physical page of logical page
 *               t / page_size of sequence b; entries past the sequence's
 *               last page are never read.  Paged mode needs page_size a power
 *               of two and a multiple of 16.  Every entry that is read must
 *               lie in [0, num_pages): an entry outside it is not
 *               dereferenced (the kernels read page 0 instead) and the output
 *               rows and lse of that sequence come back NaN.
 *   kv_lens     device int32 [B]: tokens of each sequence (0..max_kv_len).
 *   max_kv_len  host int: upper bound of kv_lens (lengths are clamped to
 *               [0, max_kv_len]).
 *   num_splits  0 = automatic (one work unit per compute unit, at most
 *               2048), else the number of work units (<= 65535) the batch's
 *               KV is divided into.  B <= 4095.
 *   workspace   device, >= attn_decode_workspace_size(...) bytes, 256-byte
 *               aligned; scratch for the partials, owned by the caller.  Its
 *               contents need no initialisation: the partial records are
 *               written before they are read, and the per-segment arrival
 *               counters of the fused merge carry a per-call tag (a word
 *               from another call, or never written, counts as zero; the
 *               call leaves them cleared).
 *   o           device [B, Hq, D] fp32 (written); lse device [B, Hq] fp32 or NULL.
 * A sequence with kv_lens[b] == 0 gets O = 0, lse = -inf.
 * Tuning: attn_decode_set_tuning below.
 * Errors: ATTN_E_INVALID, ATTN_E_UNSUPPORTED (D, kv_dt, G > 8), ATTN_E_DEVICE.
 */
attn_status attn_decode_splitkv(attn_dtype kv_dt, const void* q, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, const int32_t* page_table,
                                int max_pages, int page_size, int num_pages, const int32_t* kv_lens,
                                int max_kv_len, int B, int Hq, int Hkv, int D, float scale, int num_splits,
                                void* workspace, size_t workspace_bytes, float* o, float* lse, void* stream);

/*
 * attn_decode_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The partial records live in a static
 * device array of attn_decode_noalloc_max_scratch() bytes (8 MiB), one copy
 * per GPU, held until the process ends; the call allocates nothing.  Sizes
 * whose workspace (attn_decode_workspace_size) would exceed it are rejected
 * with ATTN_E_UNSUPPORTED.  Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) race and give wrong results.  Nothing in the array
 * needs clearing: every record is written before it is read, and the fused
 * merge's arrival counters carry a per-call tag (see workspace above).
 * Arguments and errors as attn_decode_splitkv; the first call on a device
 * looks up the array's address (ATTN_E_DEVICE if that fails).
 */
attn_status attn_decode_splitkv_noalloc(attn_dtype kv_dt, const void* q, const void* k_cache, const void* v_cache,
                                        const float* k_scale, const float* v_scale, const int32_t* page_table,
                                        int max_pages, int page_size, int num_pages, const int32_t* kv_lens,
                                        int max_kv_len, int B, int Hq, int Hkv, int D, float scale, int num_splits,
                                        float* o, float* lse, void* stream);

/* Bytes of the static scratch array of attn_decode_splitkv_noalloc. */
size_t attn_decode_noalloc_max_scratch(void);

/*
 * Process-wide tuning of attn_decode_splitkv / attn_decode_multi (results
 * stay exact; the defaults are 0, 0, -1).  Thread-safe; a call already
 * issued is not affected.
 *   path         0 = matrix-core split kernel where it exists (bf16, e4m3 and
 *                int8 caches, int4 with D = 128), 1 = vector-ALU split kernel
 *   units        work units when num_splits == 0: 0 = one per compute unit,
 *                else 1..2048
 *   piece_bytes  the matrix-core split charges each non-empty (sequence, KV
 *                head) about this many bytes of cache, the fixed cost of one
 *                more piece in a work unit; < 0 = the default, 192 KiB
 * Errors: ATTN_E_INVALID (path, units out of range).
 */
attn_status attn_decode_set_tuning(int path, int units, int64_t piece_bytes);

/*
 * Workspace bytes attn_decode_multi needs for these sizes (num_splits as
 * passed to it; 0 = automatic).  Pure host arithmetic; 0 for invalid sizes.
 */
size_t attn_decode_multi_workspace_size(int B, int n_q, int Hq, int Hkv, int D, int max_kv_len, int num_splits);

/*
 * Multi-token decode (speculative verification): the last n_q tokens of each
 * sequence query its KV cache at once.  Query token s of sequence b sits at
 * absolute position kv_lens[b] - n_q + s (past length + local index: ONNX
 * Runtime PR #33328 analysis, section 1) and sees keys j <= that position;
 * the cache already holds the n_q new tokens.  The n_q * G query rows of a
 * KV head share each K/V read of the split-KV scan (several queries per pass
 * over the keys: ONNX Runtime PR #33328 analysis, section 2), in chunks of at
 * most 8 rows; later chunks of a piece re-read its K/V from the caches.
 * Everything else -- paging, int8 / e4m3 dequantisation, the balanced split
 * and the log-sum-exp merge -- is as in attn_decode_splitkv.
 *
 *   q          device, [B, n_q, Hq, D] bf16
 *   n_q        1..64 query tokens per sequence (n_q = 1 is attn_decode_splitkv)
 *   workspace  >= attn_decode_multi_workspace_size(...) bytes, 256-byte aligned
 *   o          device [B, n_q, Hq, D] fp32; lse device [B, Hq, n_q] fp32 or NULL
 *   other arguments as attn_decode_splitkv.
 * A row that sees no key (kv_lens[b] - n_q + s < 0) gets O = 0, lse = -inf.
 * Errors: ATTN_E_INVALID, ATTN_E_UNSUPPORTED (D, kv_dt, G > 8, n_q > 64),
 * ATTN_E_DEVICE.
 */
attn_status attn_decode_multi(attn_dtype kv_dt, const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* page_table, int max_pages,
                              int page_size, int num_pages, const int32_t* kv_lens, int max_kv_len, int B, int n_q,
                              int Hq, int Hkv, int D, float scale, int num_splits, void* workspace,
                              size_t workspace_bytes, float* o, float* lse, void* stream);

/*
 * Exact log-sum-exp merge of n partial results of the same R rows:
 *   M = max_c lse_c;  w_c = exp(lse_c - M);
 *   O = sum_c w_c O_c / sum_c w_c;  lse = M + log sum_c w_c.
 * A partial with lse = -inf is empty and carries no weight; all empty gives
 * O = 0, lse = -inf.  (Reduce phase of flash decoding: ONNX Runtime PR
 * #28695 analysis, section 2; exact recombination of independent
 * sub-results: Stream-CQSA summary, "Methodology" item 2.)
 *
 *   o_parts   device [n, R, D] fp32, each normalised by its own softmax sum
 *   lse_parts device [n, R] fp32 (natural log)
 *   o         device [R, D] fp32; lse device [R] fp32 or NULL.
 * D may be any value in 1..1024.  n == 0 gives O = 0, lse = -inf.
 */
attn_status attn_merge_partials(int n, const float* o_parts, const float* lse_parts, int64_t R, int D, float* o,
                                float* lse, void* stream);

/* Counters of a budgeted streaming run (or of its plan). */
typedef struct attn_stream_report {
  int64_t tasks;             /* (query block, key block) sub-tasks */
  int64_t h2d_bytes;         /* host -> device bytes */
  int64_t d2h_bytes;         /* device -> host bytes */
  int64_t peak_device_bytes; /* device bytes the library held at once */
  int64_t block_q;           /* query positions per block */
  int64_t block_k;           /* key positions per block */
  double wall_s;             /* whole call, seconds (0 for a plan) */
  double kernel_s;           /* summed sub-task kernel time, seconds (0 for a plan) */
} attn_stream_report;

/*
 * Budgeted streaming prefill in the manner of Stream-CQSA: the (query block,
 * key block) work of exact attention is split into independent sub-tasks
 * sized so that every device byte the call holds stays within
 * device_budget_bytes; Q/K/V blocks are streamed from pinned host memory on a
 * copy stream, overlapped with compute, each sub-task's partial result is
 * merged by log-sum-exp into the resident output block, and finished output
 * blocks are copied back.  (Stream-CQSA summary: "Key contributions",
 * "Methodology" items 2-4, "Results & findings": memory grows with the block
 * size, not with the sequence length.)  Blocks are rectangular: each
 * causally visible (query block, key block) pair is one sub-task and fully
 * masked pairs are never scheduled.
 *
 *   dt            ATTN_BF16 or ATTN_F32
 *   q_host        pinned host [B, S, Hq, D]; k_host, v_host pinned host [B, T, Hkv, D]
 *   block_q,
 *   block_k       0 = chosen from the budget; otherwise forced (must fit)
 *   o_host        pinned host [B, S, Hq, D] fp32; lse_host pinned host [B, Hq, S] fp32 or NULL
 *   report        NULL or filled on success
 * Synchronous: returns after all results are in host memory and every
 * device byte it allocated is freed.  Uses the current HIP device.
 * Errors: ATTN_E_INVALID (incl. non-pinned host memory), ATTN_E_UNSUPPORTED,
 * ATTN_E_BUDGET (nothing fits), ATTN_E_DEVICE.
 */
attn_status attn_stream_budgeted(attn_dtype dt, const void* q_host, const void* k_host, const void* v_host, int B,
                                 int Hq, int Hkv, int64_t S, int64_t T, int D, int causal, float scale,
                                 size_t device_budget_bytes, int64_t block_q, int64_t block_k, float* o_host,
                                 float* lse_host, attn_stream_report* report);

/*
 * The plan attn_stream_budgeted would execute, computed on the host only (no
 * device access).  tasks (nullable) receives up to cap triples
 * (sequence b, query block index, key block index) in execution order;
 * plan (nullable) receives the counters (wall_s = kernel_s = 0).
 * Errors: ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_BUDGET.
 */
attn_status attn_stream_plan(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D, int causal,
                             size_t device_budget_bytes, int64_t block_q, int64_t block_k, int64_t* tasks,
                             int64_t cap, attn_stream_report* plan);

/* Cyclic-quorum plan facts (attn_stream_cqs / attn_stream_cqs_plan). */
#define ATTN_CQS_MAX_QUORUM 128
typedef struct attn_cqs_info {
  int64_t n_blocks;    /* N: blocks per sequence, on the query and on the key side alike */
  int64_t quorum_size; /* k: blocks per quorum */
  int64_t pairs;       /* (query block, key block) pairs computed, all sequences, empty ones included */
  int64_t base[ATTN_CQS_MAX_QUORUM]; /* base quorum D (first quorum_size entries, ascending, D[0] = 0) */
} attn_cqs_info;

/*
 * Budgeted streaming prefill decomposed by cyclic quorums (the CQS Divide:
 * Stream-CQSA summary, "Methodology" items 1-3).  Query positions and key
 * positions are each cut into N blocks (block x: queries
 * [x*block_q, (x+1)*block_q), keys [x*block_k, (x+1)*block_k)).  The base
 * quorum D is a planar difference set modulo N -- every nonzero residue is a
 * difference of exactly one ordered pair of D -- and quorum i = D + i (mod N)
 * is one sub-task per sequence: it loads the Q/K/V blocks of its k members
 * and computes the (query block x, key block y) pairs with x - y a difference
 * d_a - d_b of members (x = d_a + i); the diagonal (x, x) belongs to quorum x.
 * So every pair is computed exactly once (causally invisible pairs are
 * skipped), and the pair results are merged exactly by log-sum-exp into each
 * query block's running (O, lse), which is swapped out to o_host / lse_host
 * between sub-tasks.  The textbook cyclic-quorum construction (Singer
 * difference sets) is the reading taken where the page gives none.
 *
 *   Arguments as attn_stream_budgeted, except:
 *   n_blocks   0 = the smallest supported N whose two double-buffered
 *              sub-task slots fit device_budget_bytes; else N, one of 1, 3
 *              or p*p + p + 1 for a prime p <= 127 (quorum sizes 1, 2, p + 1)
 *   lse_host   may be NULL: the running lse then lives in a pinned host
 *              buffer the call allocates and frees
 *   info       NULL or filled with N, k, the pair count and D on success
 * report->tasks counts the quorum sub-tasks that hold at least one pair.
 * Synchronous; uses the current HIP device; every device byte it allocates is
 * freed before return.
 * Errors: ATTN_E_INVALID (incl. non-pinned host memory), ATTN_E_UNSUPPORTED
 * (dt, D, an n_blocks with no difference set), ATTN_E_BUDGET, ATTN_E_DEVICE.
 */
attn_status attn_stream_cqs(attn_dtype dt, const void* q_host, const void* k_host, const void* v_host, int B, int Hq,
                            int Hkv, int64_t S, int64_t T, int D, int causal, float scale,
                            size_t device_budget_bytes, int64_t n_blocks, float* o_host, float* lse_host,
                            attn_cqs_info* info, attn_stream_report* report);

/*
 * The plan attn_stream_cqs would execute, on the host only (no device
 * access).  pairs (nullable) receives up to cap quadruples (sequence b,
 * quorum index i, query block x, key block y) in execution order, with
 * y = -1 for the empty pair of a query block that sees no key; info and plan
 * (nullable) receive the plan facts and counters (wall_s = kernel_s = 0).
 * Errors: ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_BUDGET.
 */
attn_status attn_stream_cqs_plan(attn_dtype dt, int B, int Hq, int Hkv, int64_t S, int64_t T, int D, int causal,
                                 size_t device_budget_bytes, int64_t n_blocks, int64_t* pairs, int64_t cap,
                                 attn_cqs_info* info, attn_stream_report* plan);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
