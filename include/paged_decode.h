/*
 * paged_decode.h — C ABI of the MI355X (gfx950) paged-KV decode library.
 *
 * Operation. A few query tokens per sequence attend over a KV cache whose
 * tokens live in fixed-size pages named by a per-sequence block table, plus an
 * optional contiguous scratch area of speculative tokens ("Implementing a
 * High-Performance Custom Diffusion Attention Kernel with FlyDSL",
 * introduction, item 1). The work is split-K flash decoding: each split of a
 * sequence's context produces a partial output and log-sum-exp, and a combine
 * pass merges them (same page, introduction item 3 and "Debug Systematically";
 * the decode and split-K reduce kernels of "[ROCm] Add FlyDSL paged-attention
 * decode backend (dense + fp8) with benchmark", Kernels). Dense bf16/f16 KV and
 * e4m3fn KV with one symmetric scale per (token, kv head) are supported (same
 * pull request, Kernels and Other changes).
 *
 * For sequence b, query token t and q head h, with g = Hq / Hkv and
 * kv head hk = h / g:
 *   keys/values = tokens 0..ctx_b-1 of the paged cache (token i lives in page
 *                 block_table[b][i / bs], slot i % bs), then scratch tokens
 *                 0..S_tok-1 of sequence b; fp8 values are decode(code)*scale;
 *   s_i   = softmax_scale * dot(q[b,t,h,:], k_i)
 *   out   = sum_i exp(s_i - m) v_i / sum_i exp(s_i - m),  m = max_i s_i
 *   lse   = m + ln(sum_i exp(s_i - m))                     (natural log)
 * Sequence b has T_b = q_lens[b] query tokens and S_b = scratch_lens[b]
 * scratch tokens (Tq and S_tok when those arrays are NULL; values are clamped
 * to [0, Tq] and [0, S_tok]); query tokens t >= T_b are padding. Every query
 * token sees every context token. It sees every scratch token j < S_b
 * (scratch_mask NONE), or, with scratch_mask CAUSAL, those with
 * j <= t + (S_b - T_b): the query tokens are the last T_b of the S_b
 * speculative tokens and each sees the ones up to its own position (the
 * draft tokens the scratch storage holds, same blog page, introduction,
 * item 1; the causal order among them is this library's choice). A row that
 * sees no token at all, padding rows included, gets out = 0 and lse = -inf.
 *
 * Layouts (contiguous, row-major, element counts):
 *   q            [B, Tq, Hq, D]      q_dtype
 *   k_pages      [P, bs, Hkv, D]     kv_dtype (fp8: one byte per element)
 *   v_pages      [P, bs, Hkv, D]     kv_dtype
 *   k_scale      [P, bs, Hkv]        f32 (or f16, scale_dtype F16), fp8 only
 *   v_scale      [P, bs, Hkv]        same
 *   (kv_layout HEAD_MAJOR: pages [P, Hkv, bs, D] and scales [P, Hkv, bs])
 *   block_table  [B, >= W] int32, row stride block_table_stride elements
 *   context_lens [B] int32
 *   scratch_k/v  [B, S_tok, Hkv, D]  q_dtype (dense KV only)
 *   q_lens       [B] int32 (optional)   scratch_lens [B] int32 (optional)
 *   out          [B, Tq, Hq, D]      q_dtype
 *   lse          [B, Tq, Hq]         f32 (optional)
 *
 * Work partition (num_splits, per call). Split s of S covers the pages
 * [s*pps, min((s+1)*pps, npages)) of a sequence, with npages = ceil(ctx_b / bs)
 * and pps = ceil(npages / S); the scratch tokens belong to the last split. An
 * empty split contributes nothing. num_splits = 0 lets the library choose S
 * (paged_decode_num_splits). For S > 1 the workspace holds the partials
 *   O_part   f32 [B, Tq, Hq, S, D]  at offset 0 (each split normalised by its
 *                                    own softmax sum)
 *   LSE_part f32 [B, Tq, Hq, S]     at the next 256-byte boundary (-inf for an
 *                                    empty split, whose O_part is 0)
 * The workspace holds nothing between calls; calls that share one must not
 * overlap. out and lse do not depend on S beyond rounding.
 *
 * Memory and ownership. Every pointer in pd_args is a device pointer owned by
 * the caller; the library keeps none of them past a call and allocates no
 * device memory. Calls are asynchronous on the caller's stream, do no host
 * synchronisation and no allocation, so run + reduce can be captured in a
 * HIP graph. Page offsets are computed in 64-bit arithmetic.
 *
 * Errors. Every function returns a pd_status and never throws. Faults that
 * the host can see (null required pointers, unsupported shapes or dtypes,
 * fp8 without scales, scratch with fp8 KV, splits above the handle's maximum,
 * a workspace too small, a device that is not gfx950) are reported before any
 * launch, with a message in paged_decode_last_error(). PD_ERR_HIP reports a
 * failed launch. The kernels clamp each context_lens[b] to
 * [0, max_blocks_per_seq * block_size], so the block-table row is never read
 * past its max_blocks_per_seq entries, and with num_pages = P > 0 they clamp
 * every block-table entry they read to [0, P - 1], so no page outside the
 * pools is read. With num_pages = 0 the entries are the caller's contract:
 * block_table[b][p] in [0, P) for every p < ceil(context_lens[b] / bs).
 * Entries past that are never read, nor are page slots past the context.
 */
#ifndef PAGED_DECODE_H
#define PAGED_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pd_status {
  PD_OK = 0,
  PD_ERR_INVALID_ARG = 1,
  PD_ERR_UNSUPPORTED = 2,
  PD_ERR_WORKSPACE_TOO_SMALL = 3,
  PD_ERR_HIP = 4
} pd_status;

typedef enum pd_dtype {
  PD_DTYPE_BF16 = 0,
  PD_DTYPE_F16 = 1,
  PD_DTYPE_FP8_E4M3FN = 2
} pd_dtype;

/* Order inside a page: token-major [bs, Hkv, D] (the default) or head-major
 * [Hkv, bs, D], where each kv head's rows of a page are contiguous. */
typedef enum pd_kv_layout {
  PD_KV_LAYOUT_TOKEN_MAJOR = 0,
  PD_KV_LAYOUT_HEAD_MAJOR = 1
} pd_kv_layout;

/* Storage type of the fp8 scales. The pull request's inputs carry a
 * use_fp32_scales switch whose default is off ("[ROCm] Add FlyDSL
 * paged-attention decode backend (dense + fp8) with benchmark", review
 * thread); F16 is that narrower storage: 2 bytes per (token, kv head)
 * instead of 4, the decoded value being code * (float)scale. */
typedef enum pd_scale_dtype {
  PD_SCALE_F32 = 0,
  PD_SCALE_F16 = 1
} pd_scale_dtype;

/* Visibility of the scratch tokens to the query tokens (see above). */
typedef enum pd_scratch_mask {
  PD_SCRATCH_MASK_NONE = 0,
  PD_SCRATCH_MASK_CAUSAL = 1
} pd_scratch_mask;

/* Values fixed for the life of a handle. Fixed values such as the page size
 * and the split limit may be compile-time choices of the kernel; values that
 * change from call to call are run-time arguments ("Implementing a
 * High-Performance Custom Diffusion Attention Kernel with FlyDSL", Integration
 * Notes, Graph Capture). */
typedef struct pd_config {
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv, divides Hq */
  int32_t head_dim;           /* D: 64, 128 or 256 */
  int32_t block_size;         /* bs: tokens per page, a power of two in [1, 256] */
  int32_t q_tokens;           /* Tq: query tokens per sequence; (Hq/Hkv)*Tq <= 128
                               * (above 16 the rows form 16-row groups, each of
                               * which reads the kv head's pages) */
  int32_t scratch_tokens;     /* S_tok: 0..64 scratch tokens per sequence */
  int32_t q_dtype;            /* pd_dtype: BF16 or F16; also out and scratch dtype */
  int32_t kv_dtype;           /* pd_dtype: same as q_dtype, or FP8_E4M3FN */
  int32_t max_batch;          /* largest B a call may pass */
  int32_t max_blocks_per_seq; /* W: block-table entries a sequence may use */
  int32_t max_num_splits;     /* largest S, 1..256 */
  int32_t scratch_mask;       /* pd_scratch_mask; CAUSAL needs no scratch (a no-op then) */
  int32_t kv_layout;          /* pd_kv_layout of the page pools and scales */
  int32_t scale_dtype;        /* pd_scale_dtype of k_scale/v_scale; F16 needs FP8_E4M3FN KV */
} pd_config;

/* Values of one call. All pointers are device pointers (see the layouts). */
typedef struct pd_args {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const void* k_scale;          /* fp8 only, else NULL: f32, or f16 (scale_dtype F16) */
  const void* v_scale;          /* fp8 only, else NULL */
  const int32_t* block_table;
  int64_t block_table_stride;   /* elements between rows, >= max_blocks_per_seq */
  const int32_t* context_lens;
  const void* scratch_k;        /* required iff scratch_tokens > 0 */
  const void* scratch_v;
  void* out;
  float* lse;                   /* may be NULL */
  int32_t batch;                /* B, 0..max_batch (0 launches nothing) */
  int32_t num_splits;           /* S >= 1, or 0 to let the library choose */
  float softmax_scale;          /* multiplies q.k; custom scales are allowed */
  const int32_t* q_lens;        /* [B] query tokens per sequence, or NULL (all Tq) */
  const int32_t* scratch_lens;  /* [B] scratch tokens per sequence, or NULL (all S_tok) */
  int32_t num_pages;            /* P, pages in each pool: block-table entries are clamped
                                 * to [0, P - 1]; 0 = not checked */
} pd_args;

/* New tokens for paged_decode_write_kv. All pointers are device pointers. */
typedef struct pd_write_args {
  const void* k;                /* [N, Hkv, D] q_dtype, 16-byte aligned */
  const void* v;                /* [N, Hkv, D] q_dtype, 16-byte aligned */
  const int64_t* slot_mapping;  /* [N]: page * block_size + slot; < 0 skips the token */
  int32_t num_tokens;           /* N >= 0 (0 launches nothing) */
  void* k_pages;                /* [P, bs, Hkv, D] kv_dtype: the cache written into,
                                 * 16-byte aligned */
  void* v_pages;
  void* k_scale;                /* [P, bs, Hkv] scale_dtype, fp8 only, else NULL */
  void* v_scale;
  int64_t num_slots;            /* pool capacity P * bs: slots >= it are skipped; 0 = not checked */
} pd_write_args;

typedef struct pd_handle pd_handle;

/* Validate cfg and bind it to the current device, which must be gfx950
 * (else PD_ERR_UNSUPPORTED). Allocates host memory only. The caller owns
 * *out and releases it with paged_decode_destroy. The handle holds the values
 * that stay fixed between calls, the pd_args of each call the values that
 * change ("Implementing a High-Performance Custom Diffusion Attention Kernel
 * with FlyDSL", Integration Notes, Graph Capture). */
pd_status paged_decode_create(const pd_config* cfg, pd_handle** out);

/* Release a handle; NULL is ignored. (Library housekeeping: no passage of
 * the pages defines it.) */
void paged_decode_destroy(pd_handle* h);

/* The split count S a call with this batch and requested num_splits uses
 * (the per-call split knob whose default 0 means "choose": "[ROCm] Add FlyDSL
 * paged-attention decode backend (dense + fp8) with benchmark", review
 * thread, num_splits: int = 0):
 * the request itself, or for 0 a choice made from the batch, the kv heads, the
 * largest context the handle allows and how many decode workgroups the device
 * holds at once. A pure function of the handle, batch and request that never
 * reads device memory (so it is safe under graph capture, and run and reduce
 * always agree). A request above max_num_splits or below 0 is
 * PD_ERR_INVALID_ARG. */
pd_status paged_decode_num_splits(const pd_handle* h, int32_t batch,
                                  int32_t requested, int32_t* resolved);

/* Workspace bytes for (batch, num_splits): 0 when S resolves to 1; otherwise
 * round256(round256(N*D*4) + N*4) with N = B*Tq*Hq*S. (Library housekeeping:
 * no passage of the pages defines it; the layout is this library's.) */
pd_status paged_decode_workspace_size(const pd_handle* h, int32_t batch,
                                      int32_t num_splits, size_t* bytes);

/* Launch the decode kernel for one batch on `stream`. With S = 1 it writes out
 * and lse directly and the workspace may be NULL. Otherwise it writes partials
 * into the workspace (256-byte aligned) and paged_decode_reduce must follow on
 * the same stream with the same arguments. This is the split-K decode step
 * ("Implementing a High-Performance Custom Diffusion Attention Kernel with
 * FlyDSL", introduction item 3) of the decode kernels of "[ROCm] Add FlyDSL
 * paged-attention decode backend (dense + fp8) with benchmark", Kernels
 * (head-packed dense decode, native e4m3fn decode; the stream is threaded
 * through the launch so the call can be graph-captured). */
pd_status paged_decode_run(pd_handle* h, const pd_args* a, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Launch the split-K combine on `stream` (the split-K partial combine kernel
 * of "[ROCm] Add FlyDSL paged-attention decode backend (dense + fp8) with
 * benchmark", Kernels; "Implementing a High-Performance Custom Diffusion
 * Attention Kernel with FlyDSL", introduction item 3): for every (b, t, h),
 * M = max_s LSE_s, w_s = exp(LSE_s - M), out = sum w_s O_s / sum w_s,
 * lse = M + ln sum w_s; all splits empty gives out = 0, lse = -inf. Returns
 * PD_OK without launching when S resolves to 1. */
pd_status paged_decode_reduce(pd_handle* h, const pd_args* a, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): paged_decode_run followed by paged_decode_reduce on `stream`,
 * with the split partials in a workspace the library owns. That workspace is
 * a fixed array of 16 MiB (16777216 bytes) on each device the library runs
 * on, set up by paged_decode_create and held until the process ends; the
 * call allocates nothing. A call whose split workspace
 * (paged_decode_workspace_size) exceeds 16 MiB is rejected with
 * PD_ERR_WORKSPACE_TOO_SMALL before any launch; so is a call made while
 * another device than the handle's is current (PD_ERR_INVALID_ARG). Every
 * call on a device shares that device's array, which keeps the last call's
 * partials: calls that overlap on one device (other streams, other handles,
 * other threads) race and must be ordered by the caller. Arguments, results
 * and errors are otherwise those of the run + reduce pair. */
pd_status paged_decode_run_noalloc(pd_handle* h, const pd_args* a, hipStream_t stream);

/* Write N new tokens' K and V rows into the paged cache on `stream`: row
 * (i, hk) goes to page slot_mapping[i] / bs, slot slot_mapping[i] % bs, kv head
 * hk; a negative slot_mapping[i] skips token i. Dense caches take the rows as
 * they are. An e4m3fn cache quantises each (token, kv head) row with one
 * symmetric scale: scale = absmax / 448 and y = x / scale in single precision,
 * code = e4m3fn of clamp(y, -448, 448) rounded to nearest even, and a zero row
 * gets scale 0 and codes 0. The scale is fixed when the cache is written, not
 * per decode call ("[ROCm] Add FlyDSL paged-attention decode backend (dense +
 * fp8) with benchmark", review thread; the codes and per-token scales are what
 * its fp8 decode kernel reads, Kernels). A NaN value gives unspecified
 * codes in its row, and so does an infinite one with f32 scales (the row's
 * scale becomes infinite); with f16 scales, which saturate at 65504, an
 * infinite value quantises to +-448 like any value past the range. With
 * num_slots > 0 a slot at or past it is skipped like a negative one. Device-side contract: slots < P * bs
 * when num_slots is 0, and distinct within a call (two tokens naming one slot
 * race). Host-visible faults (null pointers, misalignment, scales missing for
 * fp8 or given for a dense cache, N < 0, num_slots < 0, N * Hkv above
 * 2^31 - 1 rows) are reported before any launch. */
pd_status paged_decode_write_kv(pd_handle* h, const pd_write_args* a, hipStream_t stream);

/* Bits of the word paged_decode_check writes to flags[0]. */
typedef enum pd_check_flag {
  PD_CHECK_CONTEXT_LENS = 1,   /* some context_lens[b] < 0 or > max_blocks_per_seq * bs */
  PD_CHECK_BLOCK_TABLE = 2,    /* some block_table[b][p] with p < ceil(ctx_b / bs) is < 0,
                                * or >= num_pages when num_pages > 0 (ctx_b clamped to
                                * [0, max_blocks_per_seq * bs] as the decode kernel does) */
  PD_CHECK_Q_LENS = 4,         /* some q_lens[b] outside [0, q_tokens] (q_lens given) */
  PD_CHECK_SCRATCH_LENS = 8    /* some scratch_lens[b] outside [0, scratch_tokens] */
} pd_check_flag;

/* Opt-in validation of the device-side contents paged_decode_run reads (the
 * contract above: context lengths, the used block-table entries, the
 * per-sequence counts). The decode kernels clamp these values, so a
 * violation gives wrong attention rather than an access outside the
 * buffers; this call tells the caller which contract broke. The opt-in
 * convention (a debug check that is off by default, costs a host wait and is
 * skipped during graph capture) is that of the slot check in "[FlyDSL]
 * feat(flydsl): add fused KDA decode kernels on gfx950" (ROCm/aiter #6026),
 * Changes, the contract table's environment-variable row.
 *
 * flags: device pointer to two uint32 words, 4-byte aligned, owned by the
 * caller; no prior clearing is needed. Asynchronously on `stream`, the call
 * sets flags[0] to the OR of the pd_check_flag bits violated (0 when every
 * contract holds) and flags[1] to the lowest sequence index with a violation
 * (0xFFFFFFFF for none). It takes the same pd_args as paged_decode_run and
 * reports the same host-visible faults before any launch; batch 0 writes the
 * no-violation result. It launches two small kernels and allocates nothing
 * (graph-capturable); the Python binding runs it before each decode when the
 * environment sets PAGED_DECODE_CHECK=1 and the stream is not capturing. */
pd_status paged_decode_check(pd_handle* h, const pd_args* a, uint32_t* flags,
                             hipStream_t stream);

/* Message of the last failing call on this thread ("" if none). (Library
 * housekeeping: no passage of the pages defines it.) */
const char* paged_decode_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_DECODE_H */
