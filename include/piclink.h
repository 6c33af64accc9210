/*
 * piclink — the link step of position-independent KV caching on AMD MI355X
 * (gfx950), as a C ABI.
 *
 * The operation. Position-independent caching splits prompt processing into
 * a per-chunk compile step and a per-request link step: every immutable chunk
 * is prefilled on its own (positions from 0) and its KV stored; at request
 * time the stored chunks are concatenated and only a few rows are recomputed,
 * the first k tokens of each chunk (LegoLink-k, k <= 32 in the paper) plus
 * the request's new suffix (EPIC, atlas.scime.ai summary, "Approach"; EPIC
 * abstract on shd-paper.top). MEPIC's paged layout stores chunk KV page
 * aligned and without positional encoding, applies RoPE inside attention,
 * recomputes a whole first page per chunk in its block-level variant, and
 * shares every other page across requests and batches (MEPIC,
 * searcharxiv.org abstract).
 *
 * This library implements:
 *   pic_store_*   a paged chunk-KV store over caller-owned device pools:
 *                 page-aligned, refcounted, shareable pages;
 *   pic_link_plan the host link planner: absolute positions, selected rows,
 *                 per-request block tables, private/copy-on-write pages and
 *                 the attention work list;
 *   pic_link_attend the device link step: scatter of the recomputed rows'
 *                 K/V into private pages, then causal attention of the
 *                 selected rows over the linked cache with RoPE applied at
 *                 each token's linked absolute position.
 *
 * Conventions shared by every call.
 *   - Layouts are row-major. Device K/V pools are [num_pages][Hkv][page][d];
 *     per-row tensors are [rows][heads][d]; element type is the store's dtype
 *     (bfloat16 or float32).
 *   - RoPE pairs dimension i with i + d/2 ("rotate half") at angle
 *     pos * theta^(-2i/d), no frequency scaling.
 *   - Attention: query head h reads KV head h / (Hq/Hkv); softmax scale
 *     1/sqrt(d); a row at position p sees every linked token at position
 *     <= p.
 *   - All device memory belongs to the caller. The library allocates none:
 *     no hipMalloc, no device-side buffers. It owns host metadata and one
 *     pinned host buffer per store (hipHostMalloc) that plan tables are
 *     uploaded from, grown as needed and freed by pic_store_destroy.
 *   - Device work is enqueued on the caller's stream and returns
 *     asynchronously; execution faults surface at the caller's next
 *     synchronisation. One thread at a time per store.
 *   - Every call returns a pic_status. On a non-OK status, pic_last_error()
 *     gives a message (thread-local, valid until the next call on the
 *     thread). No C++ exception crosses the ABI.
 */
#ifndef PICLINK_H
#define PICLINK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pic_status;
#define PIC_OK 0
#define PIC_ERR_INVALID (-1)    /* bad argument, shape or option */
#define PIC_ERR_OOM (-2)        /* page pool exhausted */
#define PIC_ERR_NOT_FOUND (-3)  /* unknown chunk id */
#define PIC_ERR_EXISTS (-4)     /* chunk id already stored */
#define PIC_ERR_DEVICE (-5)     /* HIP runtime error or kernel launch failure */
#define PIC_ERR_WORKSPACE (-6)  /* workspace too small, misaligned, or not holding the plan */
#define PIC_ERR_STATE (-7)      /* call out of order (e.g. attend before upload) */

#define PIC_DTYPE_BF16 0
#define PIC_DTYPE_F32 1

/* How stored keys carry position (pic_store_config.key_layout). */
#define PIC_KEYS_POSITION_FREE 0   /* pre-RoPE keys (MEPIC abstract: positional encodings removed) */
#define PIC_KEYS_SEGMENT_ROPE 1    /* keys rotated at their position inside their own segment, as a
                                      chunk compiled from position 0 leaves them (EPIC summary,
                                      "Approach") */

typedef struct pic_store pic_store;
typedef struct pic_plan pic_plan;

/* Shape of the attention layer and of the page pool.
 *   head_dim      64 or 128
 *   page_size     tokens per page: 16, 32 or 64
 *   num_q_heads   a multiple of num_kv_heads, with Hq/Hkv in {1, 2, 4, 8}
 *   max_position  every linked position must be < max_position (RoPE table rows);
 *                 at most 4,194,304
 *   key_layout    PIC_KEYS_POSITION_FREE: stored keys are pre-RoPE and each key is rotated at
 *                 its absolute linked position t. PIC_KEYS_SEGMENT_ROPE: a key stored at
 *                 position s of its segment holds R(s)k, and is re-rotated by the segment's
 *                 linked start a (R(a)R(s)k = R(a + s)k, the RoPE composition rule). Both give
 *                 the same attention up to rounding. Other values: PIC_ERR_INVALID.
 *   compile_offset  PIC_KEYS_SEGMENT_ROPE stores: the position of a chunk's first token when it
 *                 was compiled, c in [0, 4096]. A compile step that puts c leading tokens first and
 *                 drops their KV (LegoLink-0 prepends four dummy tokens: EPIC summary, "Measured
 *                 effects" table) leaves token j's key rotated at c + j; the link step then
 *                 re-rotates a segment's keys by its start a minus c, a negative angle when
 *                 a < c, and writes new keys rotated at c + their position in the segment.
 *                 Every segment's c + length must stay below max_position. No effect in a
 *                 PIC_KEYS_POSITION_FREE store (its keys carry no position).
 *   num_layers    decoder layers the store holds K/V for, in [0, 1024] (0 means 1). Each pool is
 *                 [num_layers][num_pages][Hkv][page][d]: every layer holds a chunk's tokens on the
 *                 same page ids, so one plan serves every layer. */
typedef struct {
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_pages;
    int32_t dtype;
    double rope_theta;
    int32_t max_position;
    int32_t key_layout;
    int32_t compile_offset;
    int32_t num_layers;
} pic_store_config;

/* One prompt to link: [prefix] chunk_ids[0..n_chunks) [suffix of suffix_len new tokens].
 * The prefix is a stored chunk placed first and never recomputed (unless
 * recompute_all). chunk_ids point to host memory read during pic_link_plan only. */
typedef struct {
    int32_t has_prefix;
    uint64_t prefix_id;
    const uint64_t *chunk_ids;
    int32_t n_chunks;
    int32_t suffix_len;
} pic_request;

/* k            recomputed leading rows per chunk (LegoLink-k); 0 = link half of LegoLink-0
 * block_level  recompute the whole first page of every chunk instead (MEPIC)
 * pos_offset   absolute position of the first token of every request (>= 0)
 * recompute_all  select every row of every segment (full-recompute comparator)
 * split_pages  KV pages per attention work item: 0 = automatic, > 0 = at most
 *              that many, < 0 = split a (row tile, KV head) only where its key
 *              range exceeds the kernel's limit of 2,048 pages per work item
 * rope_keys    where the keys get their RoPE rotation (MEPIC abstract: inside
 *              attention): 1 = in the attention kernel, for every key tile a work
 *              item reads; 2 = once per link call, every logical page's keys into
 *              the workspace, before attention (bfloat16 stores only; the results
 *              are bit-identical to 1); 0 = automatic: 2 for bfloat16 stores when
 *              the work list reads each key page at least 5 times on average,
 *              else 1. Other values: PIC_ERR_INVALID.
 * decode       T > 0: also prepare T steps of pic_link_decode (bfloat16 stores; any
 *              rope_keys: decode reads the keys rotated ahead when the link call rotates them
 *              ahead, else rotates the pool's keys itself). Every request gets T
 *              decode slots after its last token, positions end .. end + T - 1: the tail of
 *              its suffix's last page and further private pages (a private segment of their
 *              own when the request has no suffix). They count toward max_position and the
 *              page pool, and show in pic_plan_export as valid slots. 0: link only */
typedef struct {
    int32_t k;
    int32_t block_level;
    int32_t pos_offset;
    int32_t recompute_all;
    int32_t split_pages;
    int32_t rope_keys;
    int32_t decode;
} pic_link_options;

/* Sizes of a plan. rows = selected rows R over all requests (the first dim of
 * q_new/k_new/v_new/out); pages = logical pages over all requests;
 * rotated_pages = logical pages whose keys pic_link_attend rotates into the
 * workspace before attention (0: keys are rotated inside attention);
 * decode_items = split-KV work items of pic_link_decode (0: plan not made for decode);
 * workspace_bytes = table_bytes (the uploaded tables) + the larger of the link call's scratch,
 * partial_bytes (float32 partial results of split key ranges) + rotated_key_bytes (the keys of
 * every logical page rotated ahead of attention: a per-request copy of shared pages, 0 when keys
 * are rotated inside attention), and decode's, decode_partial_bytes (float32 partial results of
 * decode's page ranges), + alignment. Both scratch regions start at the same offset when the keys
 * are rotated inside attention (decode runs after the link call and needs none of its scratch);
 * with rotated_pages, decode reads the rotated keys and its partials follow them. */
typedef struct {
    int64_t rows;
    int64_t pages;
    int64_t private_pages;
    int64_t cow_pages;
    int64_t work_items;
    int64_t split_items;
    int64_t workspace_bytes;
    int64_t requests;
    int64_t rotated_pages;
    int64_t decode_items;
    int64_t table_bytes;
    int64_t partial_bytes;
    int64_t rotated_key_bytes;
    int64_t decode_partial_bytes;
} pic_plan_sizes;

/* Device bytes the caller must provide: each K and V pool
 * (num_pages * Hkv * page_size * head_dim * element size) and the RoPE table
 * (max_position * head_dim * 4: per position, d/2 cosines then d/2 sines,
 * float32). */
pic_status pic_store_sizes(const pic_store_config *cfg, int64_t *pool_bytes, int64_t *rope_table_bytes);

/* Create a store over caller-owned device pools (MEPIC abstract: paged,
 * page-aligned chunk KV). k_pool/v_pool/rope_table may all be NULL for a
 * metadata-only store (host planning and tests; pic_link_attend then fails
 * with PIC_ERR_STATE). With a rope_table, the cos/sin table is computed on the
 * host in double precision, rounded once to float32, and copied in (blocking
 * copy on `stream`). The caller keeps the pools alive until pic_store_destroy. */
pic_status pic_store_create(const pic_store_config *cfg, void *k_pool, void *v_pool, void *rope_table,
                            hipStream_t stream, pic_store **out);

/* Destroy a store. Outstanding plans must be freed first (PIC_ERR_STATE otherwise). */
pic_status pic_store_destroy(pic_store *store);

/* Compile-step product in: store the K and V of one chunk (EPIC summary,
 * "Approach": each chunk compiled independently from position 0; MEPIC
 * abstract: KV kept without positional encoding, page aligned).
 * k, v: device [num_layers][n_tokens][Hkv][d] of the store dtype (every layer's K/V
 * of the chunk; [n_tokens][Hkv][d] for a single-layer store). K is pre-RoPE in a
 * PIC_KEYS_POSITION_FREE store; in a PIC_KEYS_SEGMENT_ROPE store token j's key
 * is already rotated at position j (rotate-half pairs (i, i + d/2), angle
 * j * theta^(-2i/d)), as compiling the chunk from position 0 produces it.
 * Takes ceil(n_tokens / page_size) pages, lowest free ids first; the last
 * page's padding slots are zero-filled. NULL k and v reserve the pages
 * without writing (metadata-only use). Errors: PIC_ERR_EXISTS,
 * PIC_ERR_OOM, PIC_ERR_INVALID (n_tokens <= 0). Asynchronous on `stream`. */
pic_status pic_store_chunk(pic_store *store, uint64_t id, const void *k, const void *v, int32_t n_tokens,
                           hipStream_t stream);

/* Page ids (in order) and token count of a stored chunk. pages may be NULL to
 * query the count; otherwise cap must be >= the page count. */
pic_status pic_store_chunk_pages(const pic_store *store, uint64_t id, int32_t *pages, int32_t cap,
                                 int32_t *n_pages, int32_t *n_tokens);

/* Drop a chunk from the table. Its pages return to the pool once no live
 * plan references them. */
pic_status pic_store_release(pic_store *store, uint64_t id);

/* Store lifecycle: evict least recently used chunks until at least target_free_pages pages
 * of the pool are free (EPIC digest, 关键设计 / key design: the cache replacement policy, LRU for
 * example, and the cache size are key parameters). A chunk's use is its ingest and every
 * pic_link_plan that links it (as a prefix or a chunk). Only chunks whose pages no live plan
 * holds are candidates, since releasing the others frees nothing until those plans are freed.
 * *evicted (may be NULL) receives the number of chunks released. Errors: PIC_ERR_INVALID
 * (target outside [0, num_pages]), PIC_ERR_OOM (the target cannot be reached; nothing is
 * evicted then). */
pic_status pic_store_evict(pic_store *store, int32_t target_free_pages, int32_t *evicted);

/* Footprint of a store's pool: every page is free, held by a stored chunk (shared by every plan
 * that links it), or held only by live plans (their private pages, and pages of chunks released
 * while plans still use them). */
typedef struct {
    int64_t pages_total;
    int64_t pages_free;
    int64_t pages_chunks;
    int64_t pages_plans_only;
    int64_t chunks;
    int64_t plans;
    int64_t evictions;   /* chunks released by pic_store_evict since the store was created */
} pic_store_usage_info;

pic_status pic_store_usage(const pic_store *store, pic_store_usage_info *usage);

/* Free pages in the pool, stored chunks, live plans. Any pointer may be NULL. */
pic_status pic_store_stats(const pic_store *store, int32_t *free_pages, int32_t *chunks, int32_t *plans);

/* Link planner (host only, no device work). For every request it walks the
 * segments, accumulates absolute starts from pos_offset, selects rows (first
 * min(k, L) of each chunk, or min(page_size, L) in block mode, plus the whole
 * suffix; EPIC summary, "Approach"; MEPIC abstract), lays every segment on
 * fresh pages, keeps pages without selected rows shared with the store, and
 * takes private pages (lowest free ids) for the rest; a private chunk page
 * that keeps cached rows is copy-on-write from its stored page. It then
 * builds the attention work list. The plan references every page it uses, so
 * releasing a chunk while a plan is alive is safe. Errors: PIC_ERR_NOT_FOUND,
 * PIC_ERR_OOM (private pages), PIC_ERR_INVALID (positions >= max_position,
 * negative k or offset). */
pic_status pic_link_plan(pic_store *store, const pic_request *reqs, int32_t n_reqs,
                         const pic_link_options *opts, pic_plan **out);

pic_status pic_plan_info(const pic_plan *plan, pic_plan_sizes *sizes);

/* Host copies of the plan tables, for checks. Any pointer may be NULL.
 *   row_pos   [rows]         absolute position of each selected row (request order, then position)
 *   row_dst   [rows]         physical slot written: page * page_size + slot
 *   block_table [pages]      physical page of each logical page (requests concatenated)
 *   pos_map   [pages*page_size] absolute position per logical slot, -1 = padding
 *   cu_rows   [requests+1]   row offsets per request
 *   cu_pages  [requests+1]   logical page offsets per request
 *   cow_src, cow_dst [cow_pages]  stored page copied into each copy-on-write private page */
pic_status pic_plan_export(const pic_plan *plan, int32_t *row_pos, int32_t *row_dst, int32_t *block_table,
                           int32_t *pos_map, int32_t *cu_rows, int32_t *cu_pages, int32_t *cow_src,
                           int32_t *cow_dst);

/* Copy the plan's device tables into the caller's workspace (device memory
 * of at least sizes.workspace_bytes, 256-byte aligned). Stream-ordered: the
 * tables are staged into the store's pinned host buffer and the copy is
 * enqueued on `stream`; the call waits only for the previous upload's copy
 * out of that buffer. Work already enqueued on `stream` that reads the same
 * workspace (an earlier link call) runs before the copy.
 * Workspace ownership: the region [workspace, workspace + sizes.workspace_bytes)
 * now holds this plan, and no longer holds any other plan whose region it
 * overlaps; a plan holds one region at a time. pic_link_attend uploads the
 * plan itself when the workspace does not hold it, so this call is needed
 * only to copy the tables ahead of time (for example while the previous link
 * call runs). Errors: PIC_ERR_WORKSPACE (too small, misaligned). */
pic_status pic_plan_upload(pic_store *store, pic_plan *plan, void *workspace, int64_t workspace_bytes,
                           hipStream_t stream);

/* The link step on the device (EPIC summary, "Approach"; MEPIC abstract).
 *   q_new  [rows][Hq][d]   queries of the selected rows, pre-RoPE
 *   k_new, v_new [rows][Hkv][d]  their recomputed keys (pre-RoPE) and values
 *   out    [rows][Hq][d]   attention output, store dtype
 *   lse    [rows][Hq]      optional float32 natural-log softmax denominators
 * 1. scatter: every private page gets the new rows it holds, the cached rows
 *    copied from its stored page (copy-on-write) and zeroed padding; in a
 *    PIC_KEYS_SEGMENT_ROPE store a new row's key is written rotated at its
 *    position inside its segment, the store's key form;
 * 2. key rotation, when the plan has rotated_pages: the keys of every logical
 *    page rotated to their absolute positions into the workspace (by the
 *    key's position, or by its segment's start in a PIC_KEYS_SEGMENT_ROPE
 *    store);
 * 3. attention: every selected row attends causally over its request's linked
 *    pages with every key rotated to its absolute position;
 * 4. merge of split KV ranges (log-sum-exp weighted), when the plan split.
 * workspace: device memory of at least sizes.workspace_bytes, 256-byte aligned.
 * When it does not hold this plan's tables (pic_plan_upload), they are copied in
 * first, on `stream`, as pic_plan_upload does. Errors: PIC_ERR_WORKSPACE (too
 * small, misaligned), PIC_ERR_INVALID (null row tensor with rows > 0),
 * PIC_ERR_STATE (metadata-only store), PIC_ERR_DEVICE (launch failure).
 * Asynchronous; no kernel is launched when an error is returned before the
 * first launch. The workspace also holds the split partials and the attention
 * launch's work counters (zero between calls): link calls on one workspace
 * whose device work overlaps (other streams) race. */
pic_status pic_link_attend(pic_store *store, const pic_plan *plan, const void *q_new, const void *k_new,
                           const void *v_new, void *out, float *lse, void *workspace, int64_t workspace_bytes,
                           hipStream_t stream);

/* pic_link_attend on one layer of a multi-layer store: the same steps over that layer's K/V
 * pools (the plan's pages, private pages and rotated keys are those of the layer).
 * pic_link_attend is layer 0. Errors: PIC_ERR_INVALID (layer outside [0, num_layers)) and
 * those of pic_link_attend. */
pic_status pic_link_attend_layer(pic_store *store, const pic_plan *plan, int32_t layer, const void *q_new,
                                 const void *k_new, const void *v_new, void *out, float *lse, void *workspace,
                                 int64_t workspace_bytes, hipStream_t stream);

/* ---- Decoder layers around the link step (synthetic weights; EPIC summary, "Key results"
 * and "Limitations": the recomputed rows run through a 7-9B Llama-class model).
 * The selected rows' hidden states go through every layer of the store:
 *   h = RMSNorm(x) * attn_norm;  q, k, v = h W_qkv^T (split by heads);
 *   a = link attention of the layer (scatter of k, v; causal RoPE attention of q over the layer's
 *       linked cache);  x = x + a W_o^T;
 *   h = RMSNorm(x) * mlp_norm;  x = x + (SiLU(h W_gate^T) * (h W_up^T)) W_down^T.
 * RMSNorm(x) = x / sqrt(mean(x^2) + norm_eps). Every tensor is bfloat16 in device memory,
 * row-major; products accumulate in float32 and are rounded to bfloat16 once per output. */
typedef struct {
    int32_t d_model;   /* hidden size: num_q_heads * head_dim, a multiple of 128 */
    int32_t d_ff;      /* MLP width, a multiple of 64 */
    float norm_eps;
} pic_model_config;

/* One layer's weights, device bfloat16, each [out features][in features]. */
typedef struct {
    const void *attn_norm;   /* [d_model] */
    const void *w_qkv;       /* [(Hq + 2 Hkv) d][d_model]: query heads, then key heads, then value heads */
    const void *w_o;         /* [d_model][Hq d] */
    const void *mlp_norm;    /* [d_model] */
    const void *w_gate_up;   /* [2 d_ff][d_model]: rows alternate 32 gate rows and 32 up rows */
    const void *w_down;      /* [d_model][d_ff] */
} pic_layer_weights;

/* Device bytes pic_link_forward needs: the plan's workspace, then the activations of the
 * selected rows (normed input, q, k, v, attention output, MLP hidden). */
pic_status pic_forward_workspace(const pic_store *store, const pic_plan *plan, const pic_model_config *model,
                                 int64_t *bytes);

/* Every layer of a bfloat16 store over the plan's selected rows, in order. x [rows][d_model]
 * holds the rows' hidden states entering layer 0 and is overwritten with those leaving the last
 * layer. layers: num_layers entries (host array of device pointers). workspace: at least
 * pic_forward_workspace bytes, 256-byte aligned; its first bytes serve as the plan's workspace
 * (the tables are copied in when it does not hold them). Errors, before any launch:
 * PIC_ERR_INVALID (shapes the kernels do not take, null weights, float32 store),
 * PIC_ERR_WORKSPACE, PIC_ERR_STATE (metadata-only store). Asynchronous on `stream`. */
pic_status pic_link_forward(pic_store *store, const pic_plan *plan, const pic_model_config *model,
                            const pic_layer_weights *layers, void *x, void *workspace, int64_t workspace_bytes,
                            hipStream_t stream);

/* The layers' building blocks, on their own (bfloat16, device, row-major, asynchronous):
 * out [m][n] = a [m][k] w^T (w [n][k]) with epilogue 0: nothing, 1: + residual [m][n] (may be
 * out), 2: w's rows alternate 32 gate and 32 up rows and out [m][n/2] = SiLU(gate) * up;
 * n a multiple of 128, k of 64. PIC_ERR_INVALID otherwise. */
pic_status pic_linear(const void *a, const void *w, void *out, int32_t m, int32_t n, int32_t k, int32_t epilogue,
                      const void *residual, hipStream_t stream);
/* y [rows][dm] = x / sqrt(mean(x^2) + eps) * w; dm a multiple of 8, at most 8,192. */
pic_status pic_rmsnorm(const void *x, const void *w, void *y, int32_t rows, int32_t dm, float eps,
                       hipStream_t stream);

/* Bytes of the library's static device scratch: the largest plan workspace that
 * pic_link_attend_static takes. */
#define PIC_STATIC_SCRATCH_BYTES (64ll << 20)

/* pic_link_attend without a caller workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The library keeps one static device array of PIC_STATIC_SCRATCH_BYTES (64 MiB) per GPU,
 * held until the process ends; the plan's tables are copied into it from the plan's host
 * arrays (plain hipMemcpyAsync, no staging buffer) and the link step's kernels use it as
 * their workspace (tables, split partials, rotated keys). The caller still passes the row
 * tensors and the outputs, as for pic_link_attend, whose results it reproduces bit for bit.
 * The call allocates nothing: no hipMalloc, hipFree, hipHostMalloc or other allocating
 * routine. Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls whose device work overlaps on one GPU (other streams, other threads) race
 * and must be ordered by the caller. After it, the plan's tables are in the scratch, not in
 * its earlier workspace: a later pic_link_attend copies them in again, and pic_link_decode
 * needs a pic_link_attend first. Errors, before any copy or launch: PIC_ERR_WORKSPACE (the
 * plan's sizes.workspace_bytes exceeds PIC_STATIC_SCRATCH_BYTES), and those of
 * pic_link_attend. */
pic_status pic_link_attend_static(pic_store *store, const pic_plan *plan, const void *q_new, const void *k_new,
                                  const void *v_new, void *out, float *lse, hipStream_t stream);

/* Decode after link: one generation step per request (EPIC digest, abstract: chunks are
 * compiled, then linked, then the request generates; MEPIC abstract: the paged, shared cache
 * serves the request). For a plan made with opts.decode = T, after pic_link_attend ran on the
 * same workspace, call i (i = 0 .. T-1) is decode step i: every request's token at position
 * p = end + i (end = the position after its last linked token) attends over the request's
 * linked cache (positions < end, with the recomputed rows' K/V that pic_link_attend
 * scattered), over the tokens of steps 0 .. i-1 and over itself; the step then writes the
 * token's key and value into its decode slot, for the later steps (the key in the store's
 * key form: rotated at its position inside its segment in a PIC_KEYS_SEGMENT_ROPE store).
 *   q      [n_req][Hq][d]   the tokens' queries, pre-RoPE
 *   k, v   [n_req][Hkv][d]  their keys (pre-RoPE) and values
 *   out    [n_req][Hq][d]   attention output, store dtype
 *   lse    [n_req][Hq]      optional float32 natural-log softmax denominators
 * The cache's keys: when the plan has rotated_pages (the link call rotated every page's keys
 * into the workspace), decode reads that copy, and each step adds its token's rotated key to it;
 * else decode reads the pools as stored and rotates the keys itself (by their position, or by
 * their segment's start in a PIC_KEYS_SEGMENT_ROPE store), and the plan keeps no rotated copy:
 * the choice between speed and workspace is the link call's rope_keys. Split-KV: every
 * (request, KV head) is cut into page ranges whose partial results are merged with the token's
 * own score. pic_link_attend zeroes the decode slots and restarts at step 0. Decode must run after
 * that pic_link_attend in stream order (it reads the rows the link call scattered, and its partial
 * results may reuse the link call's workspace scratch). The workspace must still hold this plan
 * (no other plan uploaded over it since pic_link_attend), because the decode tables (and rotated
 * keys) live there. Errors, each returned before any launch:
 * PIC_ERR_WORKSPACE (too small, or the workspace does not hold this plan's tables),
 * PIC_ERR_STATE (plan not made for decode, pic_link_attend not run on this workspace since
 * its last upload, or all T steps used), PIC_ERR_INVALID (null tensor). Asynchronous on
 * `stream`. */
pic_status pic_link_decode(pic_store *store, const pic_plan *plan, const void *q, const void *k, const void *v,
                           void *out, float *lse, void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* Free a plan and drop its page references (its private pages return to the
 * pool, where a later plan may take them). Device work that uses the plan must
 * have completed, or every later device call on the store must use the same
 * stream as that work: stream order then keeps the freed pages from being
 * rewritten before that work has read them. */
pic_status pic_plan_free(pic_store *store, pic_plan *plan);

/* Per-kernel timing of pic_link_attend with HIP events on the call's stream.
 * While enabled, every call records events around the scatter, key rotation,
 * attention and merge launches. pic_profile_read synchronises on the recorded
 * events and returns the summed milliseconds of each stage in ms[0..3]
 * (scatter, attention, merge, key rotation; ms needs room for 4) and the number
 * of calls since enabling; enabling again resets the sums. */
pic_status pic_profile_enable(pic_store *store, int32_t on);
pic_status pic_profile_read(pic_store *store, double *ms, int32_t *calls);

const char *pic_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PICLINK_H */
