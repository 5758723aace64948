/*
 * mla_ragged.h -- C ABI of the MI355X (gfx950) MLA ragged prefill library.
 *
 * The operation is DeepSeek-style MLA prefill attention over a ragged batch
 * (multi-head attention after the latent KV has been decompressed):
 *   query/key head dim 192 (128 NoPE + 64 RoPE), value/output head dim 128
 *   ("[DeepseekR1] How ragged prefill manage kv_cache?", sglang issue 3849,
 *   the question about chunked prefill using MHA with 192/128 dims);
 *   sequences packed back to back and indexed by qo_indptr / kv_indptr, NHD
 *   layout, num_kv_heads equal to num_qo_heads, one causal pass over the new
 *   tokens and one non-causal pass per context chunk, each returning O and
 *   the per-(token, head) log-sum-exp
 *   ("vllm.v1.attention.backends.mla.prefill.flashinfer",
 *   FlashInferPrefillBackend.finalize_attention_metadata and
 *   FlashInferPrefillImpl.run_prefill_new_tokens / run_prefill_context_chunk);
 *   the softmax scale is always passed by the caller
 *   ("[KVCache] PagedKVCache refactor, FlashInfer JIT and MLA integration",
 *   apache/tvm PR 17674, the sm_scale bullet).
 *
 * Definition computed for query row i (0-based within its sequence b) and
 * head h, with qo_len = qo_indptr[b+1]-qo_indptr[b], kv_len likewise:
 *   visible keys J = { j : j < kv_len } when not causal, and
 *   J = { j : j < kv_len - qo_len + i + 1 } when causal (bottom-right
 *   aligned; this reduces to the usual lower triangle when qo_len == kv_len);
 *   s_j = sm_scale * <q_i, k_j>;  LSE = ln sum_{j in J} exp(s_j)  (natural log
 *   of the scaled logits);  O = sum_{j in J} exp(s_j - LSE) v_j.
 *   A row with J empty gets O = 0 and LSE = -inf.
 *
 * Around that prefill the library exports, each declared below with its
 * passage: the plan-once / run-per-layer form, a paged K/V form, a form
 * planned on the device (graph-capturable), merge_state for chunked prefill,
 * the KV decompression that feeds the MHA pass, and the weight-absorbed form
 * that attends the 576-dim latent cache directly (one shared cache row per
 * key, 512-dim values; prefill, paged prefix and decode).
 *
 * Conventions for every entry point:
 *  - Tensors are dense, row-major, device pointers unless marked HOST.
 *    q [Tq, H, 192], k [Tk, H, 192], v [Tk, H, 128], out [Tq, H, 128]
 *    share one dtype (MLA_DTYPE_BF16 or MLA_DTYPE_FP32); lse [Tq, H] is fp32.
 *    Device pointers must be 16-byte aligned.
 *  - The caller owns every tensor and every indptr array; the library never
 *    frees them. HOST arrays are read only during the call.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued on it and the call returns; device faults surface at the
 *    caller's next synchronisation, as with any HIP launch.
 *  - Every call returns MLA_OK or an error status. Arguments are validated on
 *    the host before any HIP call; an invalid call touches no device state.
 *    mla_last_error() gives a message for the last failing call of the
 *    calling thread. No C++ exception crosses this boundary.
 */
#ifndef MLA_RAGGED_H
#define MLA_RAGGED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_DTYPE_BF16 0
#define MLA_DTYPE_FP32 1

#define MLA_HEAD_DIM_QK 192
#define MLA_HEAD_DIM_VO 128
#define MLA_LATENT_DIM 512
#define MLA_ROPE_DIM 64

enum mla_status {
    MLA_OK = 0,
    MLA_EINVAL = 1,       /* bad pointer, size, indptr or scale */
    MLA_EUNSUPPORTED = 2, /* a dtype or configuration this library does not build */
    MLA_EHIP = 3,         /* a HIP runtime call failed; see mla_last_error() */
    MLA_ENOMEM = 4,       /* host or device allocation failed */
    MLA_ESTATE = 5        /* the plan does not match the call (see mla_ragged_run) */
};

/* Human-readable name of a status code. Never NULL. */
const char *mla_status_string(int status);

/* Message for the last failing call on this thread ("" if none). Never NULL. */
const char *mla_last_error(void);

/* Library version, e.g. "0.1.0". */
const char *mla_version(void);

/*
 * One-shot ragged prefill: plans the work list from the HOST indptrs, uploads
 * it and launches the prefill kernel on `stream`.
 *
 *   q, k, v      device, NHD (see above), dtype `dtype`.
 *   qo_indptr    HOST int32 [batch+1]; qo_indptr[0] == 0, non-decreasing;
 *                qo_indptr[batch] == Tq.
 *   kv_indptr    HOST int32 [batch+1]; kv_indptr[0] == 0, non-decreasing.
 *                The pages' causal pass over new tokens uses kv_indptr equal
 *                to qo_indptr; a context-chunk pass uses that chunk's
 *                cumulative lengths with causal = 0.
 *   batch        >= 0 (0 is a no-op). num_heads >= 1.
 *   causal       0 or 1 (bottom-right aligned, see the definition above).
 *   sm_scale     finite and > 0; used exactly as given.
 *   out          device [Tq, H, 128], dtype `dtype`; every row is written.
 *   lse          device fp32 [Tq, H] natural log, or NULL to skip it.
 *
 * Scratch: the work list lives in a library-owned, grow-only device buffer
 * kept per (device, stream) (plus pinned host staging), so calls on different
 * streams do not share it. Calls on one stream are ordered by that stream;
 * threads that share a stream are serialised on the host from planning to
 * launch, so they may call concurrently. Growing that buffer never waits
 * for work on other streams (the outgrown buffer is kept, not freed).
 */
int mla_ragged_prefill(const void *q, const void *k, const void *v,
                       const int32_t *qo_indptr, const int32_t *kv_indptr,
                       int32_t batch, int32_t num_heads, int32_t causal, float sm_scale,
                       int32_t dtype, void *out, float *lse, void *stream);

/*
 * Paged K/V variant of mla_ragged_prefill: the keys and values come from
 * page-organised caches through a block table instead of contiguous [Tk, H, D]
 * buffers (how serving systems hold a request's prefix: the token-to-KV pool
 * of "[DeepseekR1] How ragged prefill manage kv_cache?", sglang issue 3849,
 * token_to_kv_pool; and the per-request block table of the attention
 * metadata on the vLLM page "vllm/models/deepseek_v4/sparse_mla.py",
 * DeepseekV4FlashMLAMetadata.block_table, filled by the metadata builder's
 * build()).
 *
 *   k_cache      device [num_pages, page_size, H, 192], dtype `dtype`.
 *   v_cache      device [num_pages, page_size, H, 128].
 *   block_table  DEVICE int32 [batch, max_pages]: key j of sequence b is slot
 *                j % page_size of page block_table[b * max_pages + j / page_size].
 *                Entries outside [0, num_pages) are clamped into the cache
 *                (no out-of-bounds access; the result is then meaningless).
 *   page_size    a positive multiple of 32.
 *   kv_indptr    HOST, as for mla_ragged_prefill: only the lengths
 *                kv_indptr[b+1] - kv_indptr[b] are used (each must be at most
 *                max_pages * page_size).
 * Everything else (q, out, lse, qo_indptr, causal, sm_scale, dtype, stream)
 * is as for mla_ragged_prefill; for the same keys and values the outputs are
 * identical bit for bit to the contiguous call.
 */
int mla_ragged_prefill_paged(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *qo_indptr, const int32_t *kv_indptr,
                             const int32_t *block_table, int32_t max_pages, int32_t page_size,
                             int32_t num_pages, int32_t batch, int32_t num_heads, int32_t causal,
                             float sm_scale, int32_t dtype, void *out, float *lse, void *stream);

/*
 * Plan / run split (the pages plan once per batch and run once per layer:
 * "vllm.v1.attention.backends.mla.prefill.flashinfer", plan() inside
 * finalize_attention_metadata versus run() inside run_prefill_new_tokens).
 */
typedef struct mla_plan mla_plan;

/* Create an empty plan object (host only, no HIP call). *out receives it. */
int mla_plan_create(mla_plan **out);

/* Destroy a plan and free its host and device buffers. NULL is a no-op.
 * Every run records an event on its stream; destroy first waits (on the
 * host) for the plan's most recent run to finish, then frees, so a launched
 * run never reads freed memory. Runs of one plan on several streams must be
 * ordered by the caller (the last one launched is the one waited for). */
void mla_plan_destroy(mla_plan *plan);

/*
 * Build the work list on the host: the work partitioner splits every
 * sequence into query tiles, one work item per (query tile, block of
 * consecutive heads) (see mla_plan_set_heads_per_item), ordered so the
 * heaviest groups go first and all tiles of one (sequence, head block) land
 * on the same XCD. Validates like mla_ragged_prefill.
 * Makes no HIP call, so it also runs on a machine without a GPU.
 * `dtype` selects the kernel (and so the query-tile height).
 */
int mla_ragged_plan(mla_plan *plan, const int32_t *qo_indptr, const int32_t *kv_indptr,
                    int32_t batch, int32_t num_heads, int32_t causal, int32_t dtype);

/* Copy the planned work list to the plan's device buffer (allocated or grown
 * on first use) with an asynchronous copy on `stream`, through pinned host
 * staging. Run the kernel on the same stream (or synchronise first).
 * A buffer outgrown by a larger work list is kept (not freed) until the plan
 * is destroyed, since runs launched earlier may still read it: growing makes
 * no device-wide synchronisation. The host waits only when all four pinned
 * staging slots hold copies still in flight (for the oldest of them). */
int mla_plan_upload(mla_plan *plan, void *stream);

/*
 * Launch the prefill kernel for an uploaded plan. Tensors as for
 * mla_ragged_prefill, with their sizes:
 *   q_rows     rows of q and out (tokens); must equal the planned
 *              qo_indptr[batch].
 *   kv_rows    rows of k and v; must be >= the planned kv_indptr[batch].
 *   num_heads  heads of q, k, v and out; must equal the planned num_heads.
 * `dtype` must equal the planned dtype. Any mismatch returns MLA_ESTATE
 * before a kernel is enqueued. Enqueues exactly one kernel, then records the
 * plan's completion event on `stream`.
 */
int mla_ragged_run(const mla_plan *plan, const void *q, const void *k, const void *v,
                   int64_t q_rows, int64_t kv_rows, int32_t num_heads, float sm_scale,
                   int32_t dtype, void *out, float *lse, void *stream);

/*
 * Work-list inspection (host only): item count, and a copy of the items as
 * int32 [n, 8] = {q_row0, n_rows, head0, n_heads, kv_start, kv_len, diag0, kv_hi}:
 *   q_row0   first query token of the tile (global index);
 *   n_rows   query rows in the tile (0 marks a padding item);
 *   head0    first head of the item's head block;  n_heads heads in the block
 *            (the kernel runs them one after the other);
 *   kv_start first key token of the sequence;  kv_len keys in the sequence;
 *   diag0    row r of the tile sees keys < min(kv_len, max(0, diag0 + r + 1));
 *   kv_hi    keys the last row of the tile sees (the loop bound per head).
 * `block_m` receives the query-tile height, `n_xcd` the XCD count used and
 * `heads_per_item` the head-block size (any pointer may be NULL).
 */
int mla_plan_info(const mla_plan *plan, int64_t *n_items, int32_t *block_m, int32_t *n_xcd,
                  int32_t *heads_per_item);
int mla_plan_items(const mla_plan *plan, int32_t *dst, int64_t capacity_items);

/* Work-list entries per workgroup (host only). A bf16 plan of one head per
 * item puts two query tiles of one sequence into one workgroup when
 * (a) going up from the sequence's lightest tile, two neighbours see at most
 * 512 keys together, or (b) all of its tiles see the same keys (non-causal),
 * there are at least 8 of them and at most 4096 keys: then tiles 2k and
 * 2k + 1 pair. If any pair formed, entries 2w and 2w + 1 belong to
 * workgroup w and run back to back (an entry 2w + 1 with n_rows == 0 is
 * absent) and this returns 2; otherwise, and for fp32 plans and head blocks,
 * entry w is workgroup w and it returns 1. The hardware hands workgroup w to
 * XCD w mod n_xcd. EINVAL on a NULL argument, ESTATE before a plan. */
int mla_plan_items_per_workgroup(const mla_plan *plan, int32_t *items_per_workgroup);

/* Number of XCDs the partitioner groups work for (default 8, MI355X; 1
 * turns the grouping off). Applies to later mla_ragged_plan calls. */
int mla_plan_set_xcds(mla_plan *plan, int32_t n_xcd);

/* Heads per work item (default 0: automatic, currently one head per item,
 * the fastest measured choice at the MLA shapes). A nonzero value must
 * divide num_heads, else mla_ragged_plan returns MLA_EINVAL; the kernel then
 * runs that many consecutive heads of one query tile back to back. Applies
 * to later mla_ragged_plan calls. */
int mla_plan_set_heads_per_item(mla_plan *plan, int32_t heads_per_item);

/*
 * Device-planned prefill (for HIP graph capture and host-sync-free loops;
 * the workspace plays the part of the metadata buffers that the builder of
 * "vllm/models/deepseek_v4/sparse_mla.py" pre-allocates in __init__ so their
 * addresses stay fixed under CUDA-graph replay):
 * the same operation as mla_ragged_prefill, but qo_indptr and kv_indptr are
 * DEVICE int32 [batch+1] arrays read only by the GPU, and the work list is
 * built on the GPU into a caller-provided workspace. The call enqueues three
 * kernels (sequence order, work list, prefill) on `stream`, makes no
 * synchronising call and allocates nothing, so it can be captured in a graph
 * and replayed with new indptr contents (same batch and bounds).
 *
 *   batch        0 .. 4096 (0 is a no-op).
 *   max_tq       upper bound on qo_indptr[batch]: q and out have at least
 *                max_tq rows (and lse, if given). max_tk likewise bounds
 *                kv_indptr[batch] and the rows of k and v. The grid size
 *                depends only on batch, max_tq and num_heads.
 *   workspace    device, 16-byte aligned, at least the size reported by
 *                mla_device_plan_workspace_size(batch, max_tq, num_heads,
 *                dtype); owned by the caller, reused across calls (calls on
 *                one workspace must be ordered, e.g. on one stream).
 *                Its first int32 is a flag the GPU sets nonzero when some
 *                sequence's indptrs are invalid (not non-decreasing, negative,
 *                beyond max_tq / max_tk, or indptr[0] != 0); such sequences
 *                are skipped (no reads, their output rows are not written)
 *                instead of faulting. Read it after the stream has run.
 * Host-side arguments are validated as for mla_ragged_prefill before any
 * HIP call. Outputs match mla_ragged_prefill bit for bit (every (row, head)
 * is computed by the same arithmetic; only the order of work differs).
 */
int mla_device_plan_workspace_size(int32_t batch, int64_t max_tq, int32_t num_heads,
                                   int32_t dtype, int64_t *bytes);
int mla_ragged_prefill_device_plan(const void *q, const void *k, const void *v,
                                   const int32_t *qo_indptr, const int32_t *kv_indptr,
                                   int32_t batch, int64_t max_tq, int64_t max_tk,
                                   int32_t num_heads, int32_t causal, float sm_scale,
                                   int32_t dtype, void *out, float *lse, void *workspace,
                                   int64_t workspace_bytes, void *stream);

/*
 * Allocation-free form of mla_ragged_prefill_device_plan, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same operation, arguments and
 * outputs, but the device-plan workspace is a 16 MiB array inside the
 * library (a file-scope __device__ array; each GPU the library runs on holds
 * its own copy until the process ends), so the call allocates nothing, makes
 * no synchronising call and takes no workspace argument.
 *   Limit: the batch's workspace (see mla_device_plan_workspace_size) must
 *   fit in MLA_NOALLOC_SCRATCH_BYTES, e.g. 128 heads over 262,144 query
 *   tokens in 64 sequences needs 7.9 MB; larger calls return
 *   MLA_EUNSUPPORTED before any HIP call.
 *   Sharing: every call on one GPU uses that GPU's array. Calls that can
 *   overlap on one GPU (concurrent streams, or threads without ordering)
 *   race on it and must be serialised by the caller, e.g. issued on one
 *   stream. Each call rewrites every word it reads, so no clearing is needed
 *   between calls. Sequences with invalid device indptrs are skipped as in
 *   the workspace form; this form does not report the flag word.
 * Outputs are identical bit for bit to mla_ragged_prefill_device_plan's.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (16 << 20)
int mla_ragged_prefill_device_plan_noalloc(const void *q, const void *k, const void *v,
                                           const int32_t *qo_indptr, const int32_t *kv_indptr,
                                           int32_t batch, int64_t max_tq, int64_t max_tk,
                                           int32_t num_heads, int32_t causal, float sm_scale,
                                           int32_t dtype, void *out, float *lse, void *stream);

/*
 * merge_state: combine two attention states computed over disjoint key sets
 * (the chunked-prefill combine of the causal new-token pass with the
 * non-causal context-chunk passes; the pages return each pass's (O, LSE)
 * for this: "vllm.v1.attention.backends.mla.prefill.flashinfer",
 * run_prefill_context_chunk; sglang issue 3849, forward_return_lse used
 * for chunked prefill). Per row r:
 *   lse = ln(e^lse_a[r] + e^lse_b[r]),
 *   o[r] = e^(lse_a[r]-lse) o_a[r] + e^(lse_b[r]-lse) o_b[r];
 * a side with lse = -inf has weight 0; both -inf gives o = 0, lse = -inf.
 *
 *   o_a, o_b, o  device [num_rows, head_dim] in `dtype` (rows = tokens x heads).
 *   lse_a, lse_b, lse  device fp32 [num_rows].
 *   head_dim     must be 128 (the MLA value dim).
 *   o may alias o_a or o_b and lse may alias lse_a or lse_b (in-place merge).
 */
int mla_merge_state(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b,
                    void *o, float *lse, int64_t num_rows, int32_t head_dim, int32_t dtype,
                    void *stream);

/*
 * MLA KV decompression (the question in sglang issue 3849 about
 * decompressing the 512-dim latent cache for MHA prefill): for every token
 * t and head h,
 *   K[t,h,0:128]   = c_kv[t,:] . W_UK[:, h*128:(h+1)*128]
 *   K[t,h,128:192] = k_rope[t,:]          (shared by all heads)
 *   V[t,h,0:128]   = c_kv[t,:] . W_UV[:, h*128:(h+1)*128]
 * bf16 inputs, fp32 accumulation, bf16 outputs.
 *
 *   c_kv   device bf16 [T, 512];  k_rope device bf16 [T, 64];
 *   w_uk, w_uv device bf16 [512, H*128] (column h*128+d is head h, dim d);
 *   k_out  device bf16 [T, H, 192];  v_out device bf16 [T, H, 128].
 *   num_tokens >= 0 (0 is a no-op), num_heads >= 1.
 */
int mla_decompress_kv(const void *c_kv, const void *k_rope, const void *w_uk, const void *w_uv,
                      int64_t num_tokens, int32_t num_heads, void *k_out, void *v_out,
                      void *stream);

/*
 * Ragged MLA prefill with the decompression above fused into the attention
 * kernel (the other answer to sglang issue 3849's question: decompress the
 * latent per key tile on chip instead of writing K/V to HBM). The result is
 * mla_decompress_kv followed by mla_ragged_prefill (bf16, same indptrs and
 * causal rule), up to the order of fp32 additions: K and V are rounded to
 * bf16 before the attention uses them, exactly as the two-call path stores
 * them. Every query tile of 128 rows decompresses each 32-key tile it
 * visits again, so the decompression work grows with the query length; the
 * benchmark measures this against the two-call path and the absorbed path.
 *
 *   q        device bf16 [Tq, H, 192], Tq = qo_indptr[batch].
 *   c_kv     device bf16 [Tk, 512], k_rope device bf16 [Tk, 64]
 *            (Tk = kv_indptr[batch]; key j of sequence b is row kv_indptr[b] + j).
 *   w_uk, w_uv device bf16 [512, H*128] (column h*128+d is head h, dim d).
 *   qo_indptr, kv_indptr  host int32 [batch+1], as for mla_ragged_prefill.
 *   out      device bf16 [Tq, H, 128]; lse device fp32 [Tq, H] or NULL.
 *   num_heads in [1, 65535]; causal 0 or 1 (bottom-right aligned);
 *   sm_scale finite and > 0. All device pointers 16-byte aligned.
 * Rows that see no key get O = 0 and LSE = -inf. The call keeps a device
 * work list per (device, stream), grown as needed and freed at exit.
 * Returns MLA_EINVAL for bad arguments (before any HIP call), MLA_EUNSUPPORTED
 * when Tq x H or Tk x H exceeds 2^31, MLA_ENOMEM, or MLA_EHIP.
 */
int mla_decompress_prefill(const void *q, const void *c_kv, const void *k_rope, const void *w_uk,
                           const void *w_uv, const int32_t *qo_indptr, const int32_t *kv_indptr,
                           int32_t batch, int32_t num_heads, int32_t causal, float sm_scale,
                           void *out, float *lse, void *stream);

/*
 * Weight-absorbed MLA prefill over the latent cache (sglang issue 3849,
 * "[DeepseekR1] How ragged prefill manage kv_cache?": the absorb path that
 * attends the compressed cache directly instead of decompressing it). Each
 * query token t and head h carries an absorbed query of 576 dims (latent
 * 512 | RoPE 64); each key token j one cache row kv[j] = [c_kv | k_rope],
 * shared by all heads, whose first 512 dims are also its value:
 *   s[t,h,j]  = sm_scale * q[t,h,:] . kv[j,:]
 *   O[t,h,:]  = sum_j softmax_j(s[t,h,j]) kv[j,0:512]
 *   lse[t,h]  = ln sum_j e^s[t,h,j]
 * over the keys j visible to token t of its sequence (bottom-right causal:
 * j < kv_len - qo_len + i + 1 for the sequence's i-th query; all keys when
 * non-causal). A token with no visible key gets O = 0 and lse = -inf. bf16
 * inputs and outputs, fp32 accumulation and softmax.
 *
 *   q     device bf16 [Tq, H, 576], Tq = qo_indptr[batch].
 *   kv    device bf16 [Tk, 576],    Tk = kv_indptr[batch].
 *   qo_indptr, kv_indptr  HOST int32 [batch + 1], indptr[0] = 0,
 *         non-decreasing; Tq * H < 2^31.
 *   out   device bf16 [Tq, H, 512];  lse device fp32 [Tq, H] or NULL.
 *   All device pointers 16-byte aligned. The call plans on the host (the
 *   work list is kept per (device, stream) and reused) and enqueues one
 *   kernel on `stream`; it returns before the kernel ends. Threads that
 *   share a stream are serialised on the host from planning to launch. When
 *   the row tiles alone
 *   cannot fill the GPU (e.g. a decode step, one token per sequence), the
 *   keys of each tile are split over up to 32 work items (flash-decoding
 *   style); their partial states (O in bf16, normalised; LSE in fp32) go to
 *   a library-owned, grow-only buffer per (device, stream) and a second
 *   kernel merges them (one more bf16 rounding of each partial O before the
 *   weighted sum).
 */
int mla_absorbed_prefill(const void *q, const void *kv, const int32_t *qo_indptr,
                         const int32_t *kv_indptr, int32_t batch, int32_t num_heads,
                         int32_t causal, float sm_scale, void *out, float *lse, void *stream);

/*
 * Paged variant of mla_absorbed_prefill: the latent cache rows come from a
 * page pool through a block table (the absorb path of sglang issue 3849 runs
 * over a paged prefix held in the token-to-KV pool; the block table as in
 * the attention metadata of "vllm/models/deepseek_v4/sparse_mla.py",
 * DeepseekV4FlashMLAMetadata.block_table).
 *
 *   kv_cache     device bf16 [num_pages, page_size, 576].
 *   block_table  DEVICE int32 [batch, max_pages]: key j of sequence b is slot
 *                j % page_size of page block_table[b * max_pages + j / page_size].
 *                Entries outside [0, num_pages) are clamped into the pool (no
 *                out-of-bounds access; the result is then meaningless).
 *   page_size    a positive multiple of 32.
 *   kv_indptr    HOST: only the lengths kv_indptr[b+1] - kv_indptr[b] are used
 *                (each at most max_pages * page_size).
 * Everything else is as for mla_absorbed_prefill; for the same cache rows the
 * outputs are identical bit for bit to the contiguous call.
 */
int mla_absorbed_prefill_paged(const void *q, const void *kv_cache, const int32_t *qo_indptr,
                               const int32_t *kv_indptr, const int32_t *block_table,
                               int32_t max_pages, int32_t page_size, int32_t num_pages,
                               int32_t batch, int32_t num_heads, int32_t causal, float sm_scale,
                               void *out, float *lse, void *stream);

/*
 * Plan-once / run-per-layer form of the absorbed prefill (the plan()/run()
 * split of "vllm.v1.attention.backends.mla.prefill.flashinfer": the work list
 * depends only on the indptrs, so one plan serves every layer of a step).
 *   create / destroy  the plan object (destroy waits on the host for the
 *            plan's most recent run, then frees its buffers).
 *   build    plans from HOST indptrs as mla_absorbed_prefill does (including
 *            the choice of KV splits); paged = 1 plans for run_paged.
 *   upload   copies the work list to the current device on `stream` and
 *            allocates the split buffer (a larger one after a rebuild; the
 *            outgrown buffer is kept until destroy, so no device-wide
 *            synchronisation is needed).
 *   run      one kernel (plus the split merge) on `stream`: q, kv, out, lse
 *            as for mla_absorbed_prefill, with q_rows = rows of q and out
 *            (must equal the planned qo_indptr[batch]), kv_rows = rows of kv
 *            (must be >= the planned kv_indptr[batch]) and num_heads (must
 *            equal the plan's); run_paged as for mla_absorbed_prefill_paged,
 *            with q_rows and num_heads checked the same way.
 *   info     number of work items and KV splits.
 * Runs of one plan that uses KV splits share its split buffer: they must not
 * overlap (issue them on one stream, or order them). Errors: MLA_ESTATE when
 * the plan is not built/uploaded, built for the other cache kind, or the
 * tensor sizes do not match it.
 */
typedef struct mla_absorbed_plan mla_absorbed_plan;
int mla_absorbed_plan_create(mla_absorbed_plan **out);
void mla_absorbed_plan_destroy(mla_absorbed_plan *plan);
int mla_absorbed_plan_build(mla_absorbed_plan *plan, const int32_t *qo_indptr,
                            const int32_t *kv_indptr, int32_t batch, int32_t num_heads,
                            int32_t causal, int32_t paged);
int mla_absorbed_plan_upload(mla_absorbed_plan *plan, void *stream);
int mla_absorbed_run(const mla_absorbed_plan *plan, const void *q, const void *kv,
                     int64_t q_rows, int64_t kv_rows, int32_t num_heads, float sm_scale,
                     void *out, float *lse, void *stream);
int mla_absorbed_run_paged(const mla_absorbed_plan *plan, const void *q, const void *kv_cache,
                           int64_t q_rows, int32_t num_heads, const int32_t *block_table,
                           int32_t max_pages, int32_t page_size, int32_t num_pages,
                           float sm_scale, void *out, float *lse, void *stream);
int mla_absorbed_plan_info(const mla_absorbed_plan *plan, int64_t *n_items, int32_t *splits);

/*
 * Host-only view of the absorbed prefill's work list (no HIP call): writes
 * *n_items and, if dst is non-NULL and capacity_items suffices, the items
 * as 12 int32 each: {row0, n_rows, seq_row0, kv_hi, kv_start, kv_len,
 * diag_base, kv_lo, part, 0, 0, 0}, flat row = token * H + head, the item's
 * keys [kv_lo, kv_hi); n_rows = 0 marks padding. part = -1 when the call
 * writes the output directly; when a call has too few row tiles to fill the
 * GPU (decode), each tile's keys are split over several items (part = the
 * split index) whose partial states a second kernel merges.
 */
int mla_absorbed_plan_items(const int32_t *qo_indptr, const int32_t *kv_indptr, int32_t batch,
                            int32_t num_heads, int32_t causal, int32_t *dst,
                            int64_t capacity_items, int64_t *n_items);

#ifdef __cplusplus
}
#endif

#endif /* MLA_RAGGED_H */
