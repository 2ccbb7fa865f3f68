/*
 * pkv.h -- C ABI of libpkv: paged-KV append and decode attention on MI355X.
 *
 * The operation is the decode step of a speech-token LM served from a paged
 * KV cache, as the vox-serve "Adding a Model" page describes it: each layer
 * writes this step's keys and values into the paged cache
 * (set_kv_cache(kv_cache, k, v)) and then attends one query row per request
 * over that request's pages (run(q, kv_cache)); section 1 "The model code"
 * fixes the cache layout, and "How a program runs" fixes the per-step KV page
 * tables and the padding entries that point at scratch KV page 0.
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers unless a parameter says "host".  The caller
 *    owns every buffer; the library keeps no pointer after a call returns.
 *  - Calls only validate host-side arguments and enqueue kernels on `stream`.
 *    They never synchronise, never read device memory from the host and never
 *    allocate, so they may be captured into a HIP graph.
 *  - Invalid host arguments return a negative pkv_status_t before anything is
 *    enqueued.  A failed launch returns PKV_ERR_HIP.  No C++ exception crosses
 *    this boundary.  batch == 0 is a no-op that returns PKV_OK.
 *  - Device-side preconditions are the caller's (checked on host copies by
 *    pkv_validate_page_table, never on the fast path): every entry lists at
 *    least one page, 1 <= last_page_len <= page_size, page ids lie in
 *    [0, num_pages), and no entry lists more than max_pages_per_req pages.
 *  - bf16 means IEEE bfloat16 stored as 16-bit words; every bf16 array and the
 *    cache must be 16-byte aligned, a workspace 256-byte aligned.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_NULL_PTR = -1,    /* a required pointer is NULL                  */
    PKV_ERR_BAD_SHAPE = -2,   /* a size, index or scale is out of range      */
    PKV_ERR_UNSUPPORTED = -3, /* valid but not built: head_dim, group, ...   */
    PKV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required  */
    PKV_ERR_HIP = -5,         /* the HIP runtime refused a launch            */
    PKV_ERR_ALIGNMENT = -6,   /* an array is not aligned as required         */
    PKV_ERR_BAD_TABLE = -7    /* pkv_validate_page_table found a bad entry   */
} pkv_status_t;

/*
 * Shape of the paged cache, passed by value.  The cache is one contiguous
 * bf16 array [num_layers, num_pages, 2, page_size, num_kv_heads, head_dim]
 * ("Adding a Model", section 1); index 0 of the third axis holds keys and
 * index 1 values.  Token t of a request lives in page
 * page_indices[page_indptr[b] + t / page_size], slot t % page_size.
 * Page 0 is the scratch page that padding entries point at.
 * Supported: page_size a power of two in [1, 256]; head_dim 64 or 128 for
 * pkv_decode, any multiple of 8 for pkv_append.
 */
typedef struct {
    int32_t num_layers;
    int32_t num_pages;
    int32_t page_size;
    int32_t num_kv_heads;
    int32_t head_dim;
} pkv_cache_desc_t;

/*
 * pkv_append -- write this step's K and V rows into the cache
 * ("Adding a Model", section 1: set_kv_cache).
 *
 * For each entry b in [0, batch): page p = page_indices[page_indptr[b+1]-1]
 * (its last listed page), slot s = last_page_len[b] - 1, and
 *   cache[layer, p, 0, s, :, :] = k_new[b, :, :]
 *   cache[layer, p, 1, s, :, :] = v_new[b, :, :]
 * as a bit copy.  The page table therefore already counts the new row.
 *  kv_cache       bf16 cache described by `desc`, modified in place.
 *  k_new, v_new   bf16 [batch, num_kv_heads, head_dim], contiguous.
 *  page_indptr    int32 [batch + 1], page_indptr[0] == 0, non-decreasing.
 *  page_indices   int32 [page_indptr[batch]].
 *  last_page_len  int32 [batch], rows used in the last page after the append.
 * Padding entries list page 0 with last_page_len 1 and write only its slot 0;
 * when several do, their writes race and that slot ends up holding, element
 * by element, the value of one or another of their rows.  Two real entries
 * must not share a last page slot.
 */
int pkv_append(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
               const void *k_new, const void *v_new,
               const int32_t *page_indptr, const int32_t *page_indices,
               const int32_t *last_page_len, int32_t batch, hipStream_t stream);

/*
 * pkv_prefill -- paged prefill and mixed prefill + decode steps: several new
 * rows per entry, appended and attended causally ("Adding a Model", "How a
 * program runs": prefill runs several rows per request over the paged cache;
 * "Supported Models", Qwen3-Omni / Qwen3-TTS notes: new prompts ride a decode
 * step as one mixed step).
 *
 * Entry b brings n_b = qo_indptr[b+1] - qo_indptr[b] >= 0 rows (n_b = 1 is a
 * decode row); the page table already counts them, so the entry holds
 * L = (pages - 1) * page_size + last_page_len[b] tokens ending with them.
 * Row j (global row r = qo_indptr[b] + j) sits at position p = L - n_b + j:
 *   with k_new / v_new:  cache[layer, page(p), 0/1, slot(p), :, :] = k_new[r] / v_new[r]
 *   out[r, hq, :] = sum_{t <= p} softmax_t(sm_scale * q[r, hq, :] . K_t) V_t
 *   lse[r, hq]    = ln sum_{t <= p} exp(sm_scale * q[r, hq, :] . K_t)
 * with KV head hq / (Hq / Hkv), as in pkv_decode.  Rows see each other's keys
 * (the attention reads the new rows from k_new / v_new and writes them into
 * the cache in the same launch).
 *  q, out        bf16 [total rows, num_qo_heads, head_dim]; total rows =
 *                qo_indptr[batch].
 *  qo_indptr     int32 [batch + 1], non-decreasing, qo_indptr[0] == 0.
 *  k_new, v_new  bf16 [total rows, num_kv_heads, head_dim], or both NULL when
 *                the rows are already in the cache.
 *  lse           fp32 [total rows, num_qo_heads], natural log, or NULL.
 *  max_q_rows    host upper bound on any n_b (>= 1); it sizes the grid.
 * Preconditions as for pkv_decode, plus n_b <= L and n_b <= max_q_rows; rows
 * past max_q_rows are neither appended nor computed.  head_dim 64 or 128
 * (else PKV_ERR_UNSUPPORTED); batch <= 65535.  Uses matrix-core (MFMA)
 * products.
 */
int pkv_prefill(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
                int32_t num_qo_heads, const int32_t *qo_indptr, const void *k_new,
                const void *v_new, const int32_t *page_indptr, const int32_t *page_indices,
                const int32_t *last_page_len, int32_t batch, int32_t max_q_rows,
                float sm_scale, void *out, float *lse, hipStream_t stream);

/*
 * pkv_qk_norm_rope_append -- the fused step that feeds decode on Qwen3-style
 * attention: per-head RMSNorm of q and k, rotary embedding at each entry's
 * position, and the KV write ("Supported Models", M* docs, Qwen3-Omni and
 * Qwen3-TTS notes: q/k norm, RoPE and KV write as one kernel, in fp32
 * throughout and rounded once; the RoPE theta comes with the positions).
 *
 * For each entry b and head row x (D values) at position p = positions[b]:
 *   y = x / sqrt(mean(x^2) + eps) * w            (w: q_norm_weight for q
 *                                                 heads, k_norm_weight for k)
 *   z_i       = y_i cos a_i - y_{i+D/2} sin a_i,  a_i = p * rope_theta^(-2i/D)
 *   z_{i+D/2} = y_{i+D/2} cos a_i + y_i sin a_i   (rotate-half pairing, i < D/2)
 * computed in fp32 (the angle in fp64) and rounded once to bf16.  The q rows
 * go to q_out; the k rows to cache[layer, p_b, 0, s_b, h, :] and v_new's rows,
 * bit for bit, to cache[layer, p_b, 1, s_b, h, :], with page p_b and slot s_b
 * chosen as pkv_append chooses them (entries whose table row is malformed
 * get no KV write, as in pkv_append).  It replaces pkv_append in a layer
 * whose decode then runs with pkv_run(k_new = v_new = NULL) on q_out.
 *  kv_cache       bf16 cache described by `desc`, modified in place.
 *  q              bf16 [batch, num_qo_heads, head_dim], contiguous.
 *  k_new, v_new   bf16 [batch, num_kv_heads, head_dim], contiguous.
 *  q_norm_weight, k_norm_weight   bf16 [head_dim].
 *  eps            >= 0, finite (Qwen3: 1e-6).
 *  rope_theta     > 0, finite (Qwen3: 1e6).
 *  positions      int32 [batch]: the position of the entry's new token.
 *  page_indptr, page_indices, last_page_len   as for pkv_append.
 *  q_out          bf16 [batch, num_qo_heads, head_dim]; may be q itself.
 * head_dim 64 or 128 (else PKV_ERR_UNSUPPORTED).  Padding entries write page 0
 * slot 0 as in pkv_append; their q_out rows are computed all the same.
 */
int pkv_qk_norm_rope_append(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                            const void *q, int32_t num_qo_heads, const void *k_new,
                            const void *v_new, const void *q_norm_weight,
                            const void *k_norm_weight, float eps, float rope_theta,
                            const int32_t *positions, const int32_t *page_indptr,
                            const int32_t *page_indices, const int32_t *last_page_len,
                            int32_t batch, void *q_out, hipStream_t stream);

/*
 * pkv_qk_norm_mrope_append -- pkv_qk_norm_rope_append with multimodal RoPE,
 * the Qwen3-Omni Thinker's variant ("Supported Models", M* docs, Qwen3-Omni
 * notes: q/k RMSNorm and multimodal RoPE with the KV write in one kernel,
 * fp32 throughout, rounded once).  Each entry has a (t, h, w) position and
 * each rotary pair i (elements i and i + D/2) follows one component:
 *   a_i = positions[b, pair_axis[i]] * rope_theta^(-2i/D)
 * everything else as in pkv_qk_norm_rope_append.  With t = h = w it gives
 * exactly pkv_qk_norm_rope_append's result.
 *  positions   int32 [batch, 3], device, row-major (t, h, w).
 *  pair_axis   uint8 [head_dim / 2], HOST, each 0, 1 or 2 (else
 *              PKV_ERR_BAD_SHAPE): contiguous sections (t for the first
 *              pairs, then h, then w) and interleaved layouts are both a
 *              choice of this map.  Read during the call only.
 */
int pkv_qk_norm_mrope_append(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                             const void *q, int32_t num_qo_heads, const void *k_new,
                             const void *v_new, const void *q_norm_weight,
                             const void *k_norm_weight, float eps, float rope_theta,
                             const int32_t *positions, const uint8_t *pair_axis,
                             const int32_t *page_indptr, const int32_t *page_indices,
                             const int32_t *last_page_len, int32_t batch, void *q_out,
                             hipStream_t stream);

/*
 * pkv_decode_workspace_size -- bytes of device workspace that pkv_plan,
 * pkv_run, pkv_decode and pkv_append_decode need for these arguments.  Host
 * function; no device work.  Returns 0 for arguments the calls would reject.
 * The size grows with batch * max_pages_per_req (16 bytes per 8-token tile
 * of that many pages, for the step's plan, plus a few records per entry and
 * per workgroup) plus partial rows for split entries (fp16 outputs and an
 * fp32 {lse, scale} pair per query head).
 */
size_t pkv_decode_workspace_size(pkv_cache_desc_t desc, int32_t num_qo_heads,
                                 int32_t batch, int32_t max_pages_per_req,
                                 int32_t kv_chunk_pages);

/*
 * pkv_plan -- walk a step's page table once and write the decode schedule
 * into `workspace`, for any number of pkv_run calls (one per layer: the
 * table is the same for every layer, because the layer is the outermost axis
 * of the cache).  This is the page-table walk and work split of a decode
 * step ("How a program runs": the KV page tables are written once per step).
 *
 * Work is split into runs of tokens whose partial (output, lse) pairs are
 * merged by log-sum-exp, the way partial attentions are merged on the
 * "Supported Models" page (LTX-2.5 notes):
 *   kv_chunk_pages == 0  balanced: the work of the whole batch (its tokens,
 *                        plus a fixed cost per entry) is shared evenly among
 *                        the workgroups the GPU holds at once.  Fastest; the
 *                        split, so the last bits of a row, can change with
 *                        the rest of the batch.
 *   kv_chunk_pages  > 0  fixed: each entry is cut into runs of
 *                        kv_chunk_pages pages; a row is bit-identical
 *                        whatever else is in the batch.  At most 65536.
 * Batches above 4096 entries use fixed runs of 16 pages.
 *  page_indptr/page_indices/last_page_len   as for pkv_append.
 *  max_pages_per_req  host upper bound on any entry's page count; it sizes
 *                     the schedule.  An entry listing more pages gets NaN
 *                     rows from pkv_run instead of a truncated result.
 *  workspace          device memory, 256-byte aligned, of workspace_bytes >=
 *                     pkv_decode_workspace_size(...).  Its contents need no
 *                     initialisation; the plan overwrites what it uses.
 * Errors as for pkv_decode.  Asynchronous like every call: the page table
 * is read on the device when the plan runs, in stream order.
 */
int pkv_plan(pkv_cache_desc_t desc, int32_t num_qo_heads,
             const int32_t *page_indptr, const int32_t *page_indices,
             const int32_t *last_page_len, int32_t batch, int32_t max_pages_per_req,
             int32_t kv_chunk_pages, void *workspace, size_t workspace_bytes,
             hipStream_t stream);

/*
 * pkv_run -- the decode of one layer on a plan that pkv_plan wrote into
 * `workspace`; with k_new and v_new also the append, in the same pass (see
 * pkv_append_decode).  Computes exactly what pkv_decode computes.
 *  kv_cache      bf16 cache described by `desc`; written only when k_new and
 *                v_new are given (both or neither).
 *  q, out, lse, sm_scale   as for pkv_decode.
 *  batch, max_pages_per_req, kv_chunk_pages, desc.page_size,
 *  desc.num_kv_heads, num_qo_heads   must equal those of the pkv_plan call
 *                that wrote the workspace; the page table must be unchanged
 *                since, and the plan must precede this call in stream order.
 * Between the plan and its pkv_run calls the workspace may serve nothing
 * else; pkv_run calls on one workspace must not overlap (each leaves the
 * plan intact for the next).
 */
int pkv_run(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
            const void *k_new, const void *v_new, const void *q,
            int32_t num_qo_heads, int32_t batch, float sm_scale, void *out,
            float *lse, int32_t max_pages_per_req, int32_t kv_chunk_pages,
            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_plan_mixed -- pkv_plan for a mixed step (new prompts riding a decode
 * step, as pkv_prefill takes them): the entries with exactly one new row are
 * decode rows and are planned like pkv_plan's entries, but under their row
 * index r = qo_indptr[b] (a batch of total_rows rows); the rows of entries
 * with several new rows get no decode work.  With pkv_mixed_run, a long
 * decode row is split over workgroups and merged exactly as in pkv_run,
 * while the prompts go through the prefill ("Supported Models", Qwen3-Omni /
 * Qwen3-TTS notes: prompts and decode rows in one step; "How a program
 * runs": the page tables are written once per step).
 *  qo_indptr     int32 [batch + 1] as for pkv_prefill; total_rows =
 *                qo_indptr[batch] (host value), at most 8192.
 *  workspace     sized by pkv_decode_workspace_size(desc, num_qo_heads,
 *                total_rows, max_pages_per_req, kv_chunk_pages).
 * Other arguments and errors as for pkv_plan; batch <= 65535.
 */
int pkv_plan_mixed(pkv_cache_desc_t desc, int32_t num_qo_heads, const int32_t *qo_indptr,
                   const int32_t *page_indptr, const int32_t *page_indices,
                   const int32_t *last_page_len, int32_t batch, int32_t total_rows,
                   int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_mixed_run -- one layer of a mixed step in one call, on a plan of
 * pkv_plan_mixed: the decode rows through the decode run (with their append
 * when k_new / v_new are given), then every entry with several new rows
 * through the prefill (its append and causal attention).  Computes what
 * pkv_prefill computes for the same arguments, the decode rows up to the
 * rounding of the decode's split and merge; the cache writes are identical.
 *  q, out, lse, k_new, v_new, qo_indptr, max_q_rows, sm_scale   as for
 *                pkv_prefill ([total_rows, ...] arrays).
 *  batch, total_rows, max_pages_per_req, kv_chunk_pages   as for the
 *                pkv_plan_mixed call that wrote the workspace (whose rules
 *                for pkv_run hold here too).
 * Errors as for pkv_prefill and pkv_run; two launches in stream order.
 */
int pkv_mixed_run(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
                  int32_t num_qo_heads, const int32_t *qo_indptr, const void *k_new,
                  const void *v_new, const int32_t *page_indptr, const int32_t *page_indices,
                  const int32_t *last_page_len, int32_t batch, int32_t total_rows,
                  int32_t max_q_rows, float sm_scale, void *out, float *lse,
                  int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_run_qk_norm_rope -- pkv_run with the append (k_new, v_new required) and
 * the q/k RMSNorm and rotary embedding of pkv_qk_norm_rope_append folded into
 * the same pass: one launch per layer instead of two for Qwen3-style
 * attention ("Supported Models", M* docs, Qwen3-Omni and Qwen3-TTS notes: q/k
 * norm, RoPE and KV write fused).  q is the raw projection; every workgroup
 * that computes a run of an entry normalizes and rotates that entry's q rows
 * itself, and the workgroup whose run holds the new token does the same to
 * its k row before it uses and stores it.  The q rows are transformed with
 * the same formulas as pkv_qk_norm_rope_append (fp32, angle reduced in fp64,
 * rounded once to bf16) but are not written out; the cache receives the
 * transformed k row and v_new's row, bit for bit, in the append's slot.
 * Results match pkv_qk_norm_rope_append followed by pkv_run within rounding
 * (the sum of squares adds in another order, so a q or k element can differ
 * by one bf16 step).
 *  q_norm_weight, k_norm_weight, eps, rope_theta, positions
 *                 as for pkv_qk_norm_rope_append (16-byte aligned weights).
 *  every other argument as for pkv_run.
 * Supported: head_dim 128 with num_qo_heads / num_kv_heads in 1..4 (else
 * PKV_ERR_UNSUPPORTED).  Padding entries write page 0 slot 0 as in pkv_append.
 */
int pkv_run_qk_norm_rope(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                         const void *k_new, const void *v_new, const void *q,
                         int32_t num_qo_heads, int32_t batch,
                         const void *q_norm_weight, const void *k_norm_weight,
                         float eps, float rope_theta, const int32_t *positions,
                         float sm_scale, void *out, float *lse,
                         int32_t max_pages_per_req, int32_t kv_chunk_pages,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * pkv_run_qk_norm_mrope -- pkv_run_qk_norm_rope with multimodal RoPE, the
 * Qwen3-Omni Thinker's variant ("Supported Models", Qwen3-Omni notes: q/k
 * RMSNorm and multimodal RoPE with the KV write in one kernel): entry b has
 * a (t, h, w) position and rotary pair i (elements i and i + D/2) turns by
 *   a_i = positions[b, pair_axis[i]] * rope_theta^(-2i/D)
 * as in pkv_qk_norm_mrope_append, but folded into the decode launch like
 * pkv_run_qk_norm_rope.  With t = h = w it gives exactly
 * pkv_run_qk_norm_rope's result.
 *  positions   int32 [batch, 3], device, row-major (t, h, w).
 *  pair_axis   uint8 [head_dim / 2], HOST, each 0, 1 or 2 (else
 *              PKV_ERR_BAD_SHAPE; NULL: PKV_ERR_NULL_PTR).  Read during the
 *              call only.
 *  every other argument, and what is supported, as for pkv_run_qk_norm_rope.
 */
int pkv_run_qk_norm_mrope(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                          const void *k_new, const void *v_new, const void *q,
                          int32_t num_qo_heads, int32_t batch, const void *q_norm_weight,
                          const void *k_norm_weight, float eps, float rope_theta,
                          const int32_t *positions, const uint8_t *pair_axis, float sm_scale,
                          void *out, float *lse, int32_t max_pages_per_req,
                          int32_t kv_chunk_pages, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * pkv_decode -- grouped-query attention of one query row per entry over its
 * pages ("Adding a Model", section 1: run(q, kv_cache); "How a program
 * runs": lm_decode is one row per request).
 *
 * For entry b with n = page_indptr[b+1] - page_indptr[b] pages and
 * L = (n - 1) * page_size + last_page_len[b] tokens, and for query head hq
 * reading KV head h = hq / (num_qo_heads / num_kv_heads):
 *   s_t = sm_scale * dot(q[b, hq, :], K_t[h, :])          t = 0 .. L-1
 *   lse[b, hq] = ln(sum_t exp(s_t))                         natural log
 *   out[b, hq, :] = sum_t exp(s_t - lse[b, hq]) * V_t[h, :]
 * Accumulation is fp32; out is rounded once to bf16 (nearest even).
 * The call is pkv_plan followed by pkv_run on the same workspace (two
 * launches); a step that decodes several layers on one page table plans once
 * and runs per layer instead.
 *  kv_cache           bf16 cache described by `desc` (read only).
 *  q                  bf16 [batch, num_qo_heads, head_dim], RoPE applied.
 *  page_indptr/page_indices/last_page_len   as for pkv_append.
 *  sm_scale           finite softmax scale, e.g. 1/sqrt(head_dim).
 *  out                bf16 [batch, num_qo_heads, head_dim], written.
 *  lse                fp32 [batch, num_qo_heads], written; may be NULL.
 *  max_pages_per_req, kv_chunk_pages, workspace   as for pkv_plan.
 * Supported: head_dim 64 or 128, num_kv_heads <= 16, num_qo_heads /
 * num_kv_heads in 1..8.  Rows of padding entries are computed over scratch
 * page 0 and are garbage by design; they never fault and never touch other
 * entries' rows.  The balanced split is sized for the current HIP device.
 */
int pkv_decode(const void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
               const void *q, int32_t num_qo_heads,
               const int32_t *page_indptr, const int32_t *page_indices,
               const int32_t *last_page_len, int32_t batch, float sm_scale,
               void *out, float *lse, int32_t max_pages_per_req,
               int32_t kv_chunk_pages, void *workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * pkv_append_decode -- pkv_append followed by pkv_decode for one layer, in
 * one pass: the same two calls the "Adding a Model" page makes per layer
 * (set_kv_cache, then run).  The workgroup that attends over an entry's new
 * token takes that row from k_new / v_new and writes it into the cache slot
 * pkv_append would write, so the cache afterwards is bit-identical to
 * pkv_append's and out / lse equal pkv_decode's on that cache (the two
 * calls' bounds, arguments and errors combined; k_new and v_new are
 * required).  Several padding entries writing scratch page 0 race exactly as
 * in pkv_append.
 */
int pkv_append_decode(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                      const void *k_new, const void *v_new, const void *q,
                      int32_t num_qo_heads, const int32_t *page_indptr,
                      const int32_t *page_indices, const int32_t *last_page_len,
                      int32_t batch, float sm_scale, void *out, float *lse,
                      int32_t max_pages_per_req, int32_t kv_chunk_pages,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_decode_static -- pkv_decode with no workspace argument and no
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Computes exactly what pkv_decode computes (same plan and kernels, so the
 * same bits), with the plan and partial rows in a 16 MiB (16 << 20 bytes)
 * device array inside the library instead of a caller's workspace.  Each GPU
 * the library runs on holds its own array from the first call on that device
 * until the process ends; the first call on a device looks its address up
 * (no allocation, then or later).  Every call on a GPU shares that GPU's
 * array and leaves its plan there: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller, as they
 * would be on one shared workspace.
 *  Arguments as for pkv_decode, without workspace / workspace_bytes.
 * Returns PKV_ERR_WORKSPACE, before touching the device, when the call needs
 * more than 16 MiB (pkv_decode_workspace_size gives the need); other errors
 * as for pkv_decode.
 */
int pkv_decode_static(const void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                      const void *q, int32_t num_qo_heads,
                      const int32_t *page_indptr, const int32_t *page_indices,
                      const int32_t *last_page_len, int32_t batch, float sm_scale,
                      void *out, float *lse, int32_t max_pages_per_req,
                      int32_t kv_chunk_pages, hipStream_t stream);

/*
 * pkv_validate_page_table -- debug check of HOST copies of a page table
 * against the device-side preconditions above.  Returns PKV_OK or
 * PKV_ERR_BAD_TABLE (with *bad_entry set to the first offending entry, or -1
 * for a problem with page_indptr[0]); PKV_ERR_NULL_PTR / PKV_ERR_BAD_SHAPE
 * for bad arguments.  Checks: indptr starts at 0 and never decreases; every
 * entry has 1..max_pages_per_req pages (max_pages_per_req <= 0 disables that
 * bound); 1 <= last_page_len <= page_size; ids in [0, num_pages); an entry
 * that lists page 0 is a padding entry (one page, last_page_len 1); no two
 * entries append into the same real page slot.
 */
int pkv_validate_page_table(const int32_t *page_indptr, const int32_t *page_indices,
                            const int32_t *last_page_len, int32_t batch,
                            int32_t num_pages, int32_t page_size,
                            int32_t max_pages_per_req, int32_t *bad_entry);

/*
 * pkv_last_hip_error -- the hipError_t code behind the most recent
 * PKV_ERR_HIP returned on the calling thread (0 if there was none).  Host
 * function; diagnostics only.
 */
int pkv_last_hip_error(void);

/* Static, human-readable name of a pkv_status_t value. */
const char *pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
