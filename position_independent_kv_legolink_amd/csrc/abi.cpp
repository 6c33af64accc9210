// The C ABI (include/piclink.h): paged chunk store, planner entry points and the link call.
// Every export converts C++ exceptions into a pic_status and a thread-local message.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>

#include "runtime.h"

static_assert(piclink::kStaticScratchBytes == PIC_STATIC_SCRATCH_BYTES, "scratch size differs from the header");

namespace piclink {

thread_local std::string g_last_error;

void fail(pic_status status, const std::string &message) { throw Error{status, message}; }

void check_hip(hipError_t e, const char *what) {
    if (e != hipSuccess) fail(PIC_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

namespace {

int64_t elem_bytes(int32_t dtype) { return dtype == PIC_DTYPE_BF16 ? 2 : 4; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace

void store_check_config(const pic_store_config &c) {
    if (c.num_kv_heads <= 0 || c.num_q_heads <= 0 || c.num_q_heads % c.num_kv_heads != 0)
        fail(PIC_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
    const int g = c.num_q_heads / c.num_kv_heads;
    if (!pow2(g) || g > 8) fail(PIC_ERR_INVALID, "num_q_heads / num_kv_heads must be 1, 2, 4 or 8");
    if (c.head_dim != 64 && c.head_dim != 128) fail(PIC_ERR_INVALID, "head_dim must be 64 or 128");
    if (c.page_size != 16 && c.page_size != 32 && c.page_size != 64)
        fail(PIC_ERR_INVALID, "page_size must be 16, 32 or 64");
    if (c.num_pages <= 0) fail(PIC_ERR_INVALID, "num_pages must be positive");
    if (c.dtype != PIC_DTYPE_BF16 && c.dtype != PIC_DTYPE_F32) fail(PIC_ERR_INVALID, "dtype must be bf16 or f32");
    if (!(c.rope_theta > 0.0)) fail(PIC_ERR_INVALID, "rope_theta must be positive");
    if (c.max_position <= 0 || c.max_position > kMaxPosition)
        fail(PIC_ERR_INVALID, "max_position must be in [1, " + std::to_string(kMaxPosition) + "]");
    if (c.key_layout != PIC_KEYS_POSITION_FREE && c.key_layout != PIC_KEYS_SEGMENT_ROPE)
        fail(PIC_ERR_INVALID, "key_layout must be PIC_KEYS_POSITION_FREE or PIC_KEYS_SEGMENT_ROPE");
    if (c.num_layers < 0 || c.num_layers > kMaxLayers)
        fail(PIC_ERR_INVALID, "num_layers must be in [0, " + std::to_string(kMaxLayers) + "] (0 means 1)");
    if (c.compile_offset < 0 || c.compile_offset > kMaxCompileOffset || c.compile_offset >= c.max_position)
        fail(PIC_ERR_INVALID, "compile_offset must be in [0, " + std::to_string(kMaxCompileOffset) +
                                  "] and below max_position");
}

int32_t store_alloc_page(pic_store *s) {
    if (s->free_pages.empty()) fail(PIC_ERR_OOM, "page pool exhausted");
    const int32_t p = *s->free_pages.begin();
    s->free_pages.erase(s->free_pages.begin());
    s->refs[p] = 1;
    return p;
}

void store_ref(pic_store *s, int32_t page) { s->refs[page] += 1; }

void store_unref(pic_store *s, int32_t page) {
    if (--s->refs[page] == 0) s->free_pages.insert(page);
}

const Chunk &store_find(const pic_store *s, uint64_t id) {
    auto it = s->chunks.find(id);
    if (it == s->chunks.end()) fail(PIC_ERR_NOT_FOUND, "chunk " + std::to_string(id) + " is not stored");
    return it->second;
}


// The plan's device tables, laid out as the workspace holds them (offsets from the planner).
void pack_tables(const pic_plan &plan, uint8_t *blob) {
    memset(blob, 0, (size_t)plan.table_bytes);
    auto put = [&](int64_t off, const void *src, size_t bytes) {
        if (bytes) memcpy(blob + off, src, bytes);
    };
    put(plan.off_pages, plan.pages.data(), plan.pages.size() * sizeof(PageDesc));
    put(plan.off_page_scatter, plan.page_scatter.data(), plan.page_scatter.size() * sizeof(int32_t));
    put(plan.off_row_pos, plan.row_pos.data(), plan.row_pos.size() * sizeof(int32_t));
    put(plan.off_scatter, plan.scatter.data(), plan.scatter.size() * sizeof(ScatterDesc));
    put(plan.off_work, plan.work.data(), plan.work.size() * sizeof(WorkDesc));
    put(plan.off_merge, plan.merge.data(), plan.merge.size() * sizeof(MergeDesc));
    put(plan.off_dec_work, plan.dec_work.data(), plan.dec_work.size() * sizeof(DecodeDesc));
    put(plan.off_dec_merge, plan.dec_merge.data(), plan.dec_merge.size() * sizeof(DecodeMergeDesc));
}

// Stage a plan's tables in the store's pinned buffer and enqueue their copy into the workspace on
// `stream`; the workspace region then holds this plan (the ledger), and the plan has not yet been
// attended there.
void upload_tables(pic_store *s, pic_plan *plan, void *workspace, int64_t workspace_bytes, hipStream_t stream) {
    if (!workspace || workspace_bytes < plan->workspace_bytes)
        fail(PIC_ERR_WORKSPACE, "workspace needs " + std::to_string(plan->workspace_bytes) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) fail(PIC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    // the previous upload's copy out of the staging buffer must have finished before it is rewritten
    if (plan->table_bytes > 0) {
        if (s->staging_done) check_hip(hipEventSynchronize(s->staging_done), "staging buffer wait");
        if (s->staging_bytes < plan->table_bytes) {
            const int64_t cap = std::max<int64_t>({plan->table_bytes, 2 * s->staging_bytes, 1 << 16});
            if (s->staging) check_hip(hipHostFree(s->staging), "hipHostFree");
            s->staging = nullptr;
            s->staging_bytes = 0;
            check_hip(hipHostMalloc(&s->staging, (size_t)cap, hipHostMallocDefault), "hipHostMalloc");
            s->staging_bytes = cap;
        }
        if (!s->staging_done)
            check_hip(hipEventCreateWithFlags(&s->staging_done, hipEventDisableTiming), "hipEventCreate");
        pack_tables(*plan, static_cast<uint8_t *>(s->staging));
        check_hip(hipMemcpyAsync(workspace, s->staging, (size_t)plan->table_bytes, hipMemcpyHostToDevice, stream),
                  "plan upload");
        check_hip(hipEventRecord(s->staging_done, stream), "hipEventRecord");
    }
    s->ledger.claim(plan, workspace, plan->workspace_bytes);
    plan->attended_ws = nullptr;
    plan->dec_next = 0;
}


// Argument checks shared by the link calls; every failure is raised before any launch.
void check_link_call(pic_store *s, const pic_plan *plan, const void *q_new, const void *k_new, const void *v_new,
                     const void *out) {
    if (!s || !plan) fail(PIC_ERR_INVALID, "null argument");
    if (plan->owner != s) fail(PIC_ERR_INVALID, "plan belongs to another store");
    if (!s->k_pool) fail(PIC_ERR_STATE, "metadata-only store has no device");
    if (!plan->row_pos.empty() && (!q_new || !k_new || !v_new || !out)) fail(PIC_ERR_INVALID, "null row tensor");
}

// The device link step over a workspace that holds the plan's tables: scatter, key rotation (when
// the plan rotates ahead), attention and the merge of split ranges, with per-kernel events when
// `prof`.
void launch_link(pic_store *s, const pic_plan *plan, int layer, const void *q_new, const void *k_new,
                 const void *v_new, void *out, float *lse, uint8_t *ws, bool prof, hipStream_t stream) {
    // the layer's pools: every layer holds the same pages at the same ids
    const int64_t layer_bytes = s->shape.page_elems * s->cfg.num_pages * elem_bytes(s->cfg.dtype);
    void *k_pool = static_cast<uint8_t *>(s->k_pool) + layer * layer_bytes;
    void *v_pool = static_cast<uint8_t *>(s->v_pool) + layer * layer_bytes;
    AttnTables t;
    t.pages = reinterpret_cast<const PageDesc *>(ws + plan->off_pages);
    t.row_pos = reinterpret_cast<const int32_t *>(ws + plan->off_row_pos);
    t.work = reinterpret_cast<const WorkDesc *>(ws + plan->off_work);
    t.n_work = (int)plan->work.size();
    t.ticket = reinterpret_cast<uint32_t *>(ws + plan->off_ticket);
    t.n_queues = plan->work_queues;
    t.n_groups = std::min<int>(t.n_work, s->num_cus);
    t.merge = reinterpret_cast<const MergeDesc *>(ws + plan->off_merge);
    t.n_merge = (int)plan->merge.size();
    t.part_o = reinterpret_cast<float *>(ws + plan->off_part_o);
    t.part_lse = reinterpret_cast<float *>(ws + plan->off_part_lse);
    if (plan->rotate_keys) t.k_rot = ws + plan->off_k_rot;

    ProfileMarks marks{};
    if (prof) {
        for (int i = 0; i < 5; ++i) {
            if (!s->spare_events.empty()) {
                marks.ev[i] = s->spare_events.back();
                s->spare_events.pop_back();
            } else {
                check_hip(hipEventCreate(&marks.ev[i]), "hipEventCreate");
            }
        }
        check_hip(hipEventRecord(marks.ev[0], stream), "hipEventRecord");
    }
    const auto *table = reinterpret_cast<const ScatterDesc *>(ws + plan->off_scatter);
    if (plan->rotate_keys) {
        // the scatter runs inside the key rotation's launch: the profile's scatter interval is
        // empty and its rotation interval holds both
        if (prof) check_hip(hipEventRecord(marks.ev[1], stream), "hipEventRecord");
        check_hip(launch_prepare(s->shape, k_pool, v_pool, k_new, v_new, s->rope, t.pages,
                                 reinterpret_cast<const int32_t *>(ws + plan->off_page_scatter),
                                 (int)plan->pages.size(), table, (int)plan->scatter.size(),
                                 const_cast<void *>(t.k_rot), stream),
                  "scatter and key rotation launch");
    } else {
        check_hip(launch_scatter(s->shape, k_pool, v_pool, k_new, v_new, s->rope, table, (int)plan->scatter.size(),
                                 stream),
                  "scatter launch");
        if (prof) check_hip(hipEventRecord(marks.ev[1], stream), "hipEventRecord");
    }
    if (prof) check_hip(hipEventRecord(marks.ev[2], stream), "hipEventRecord");
    check_hip(launch_attention(s->shape, q_new, k_pool, v_pool, s->rope, t, out, lse, stream),
              "attention launch");
    if (prof) check_hip(hipEventRecord(marks.ev[3], stream), "hipEventRecord");
    check_hip(launch_merge(s->shape, t, out, lse, stream), "merge launch");
    pic_plan *mp = const_cast<pic_plan *>(plan);
    mp->attended_ws = ws;
    mp->dec_next = 0;   // the scatter zeroed the decode slots
    if (prof) {
        check_hip(hipEventRecord(marks.ev[4], stream), "hipEventRecord");
        s->pending.push_back(marks);
    }
}

}  // namespace piclink

using namespace piclink;

extern "C" {

const char *pic_last_error(void) { return g_last_error.c_str(); }

pic_status pic_store_sizes(const pic_store_config *cfg, int64_t *pool_bytes, int64_t *rope_table_bytes) {
    return guarded([&] {
        if (!cfg) fail(PIC_ERR_INVALID, "null config");
        store_check_config(*cfg);
        if (pool_bytes)
            *pool_bytes = (int64_t)std::max(1, cfg->num_layers) * cfg->num_pages * cfg->num_kv_heads *
                          cfg->page_size * cfg->head_dim * elem_bytes(cfg->dtype);
        if (rope_table_bytes) *rope_table_bytes = (int64_t)cfg->max_position * cfg->head_dim * 4;
    });
}

pic_status pic_store_create(const pic_store_config *cfg, void *k_pool, void *v_pool, void *rope_table,
                            hipStream_t stream, pic_store **out) {
    return guarded([&] {
        if (!cfg || !out) fail(PIC_ERR_INVALID, "null argument");
        *out = nullptr;
        store_check_config(*cfg);
        const bool any = k_pool || v_pool || rope_table;
        if (any && !(k_pool && v_pool && rope_table))
            fail(PIC_ERR_INVALID, "k_pool, v_pool and rope_table must all be given or all be NULL");
        pic_store *s = new pic_store();
        s->cfg = *cfg;
        s->cfg.num_layers = std::max(1, cfg->num_layers);
        s->shape = {cfg->num_q_heads, cfg->num_kv_heads, cfg->head_dim, cfg->page_size, cfg->dtype,
                    (int64_t)cfg->num_kv_heads * cfg->page_size * cfg->head_dim, cfg->key_layout};
        s->k_pool = k_pool;
        s->v_pool = v_pool;
        s->rope = static_cast<float *>(rope_table);
        s->refs.assign(cfg->num_pages, 0);
        for (int32_t p = 0; p < cfg->num_pages; ++p) s->free_pages.insert(s->free_pages.end(), p);
        if (rope_table) {
            try {
                int dev = 0;
                hipDeviceProp_t prop;
                check_hip(hipGetDevice(&dev), "hipGetDevice");
                check_hip(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
                s->num_cus = prop.multiProcessorCount;
                // cos/sin of pos * theta^(-2i/d) in double precision, rounded once to float
                const int d = cfg->head_dim, half = d / 2;
                std::vector<double> inv(half);
                for (int i = 0; i < half; ++i) inv[i] = pow(cfg->rope_theta, -2.0 * i / d);
                std::vector<float> table((size_t)cfg->max_position * d);
                for (int64_t pos = 0; pos < cfg->max_position; ++pos)
                    for (int i = 0; i < half; ++i) {
                        const double a = (double)pos * inv[i];
                        table[pos * d + i] = (float)cos(a);
                        table[pos * d + half + i] = (float)sin(a);
                    }
                check_hip(hipMemcpyAsync(rope_table, table.data(), table.size() * sizeof(float),
                                         hipMemcpyHostToDevice, stream),
                          "RoPE table upload");
                check_hip(hipStreamSynchronize(stream), "RoPE table upload");
            } catch (...) {
                delete s;
                throw;
            }
        }
        *out = s;
    });
}

pic_status pic_store_destroy(pic_store *s) {
    return guarded([&] {
        if (!s) return;
        if (s->live_plans > 0) fail(PIC_ERR_STATE, "free every plan before destroying the store");
        for (auto &m : s->pending)
            for (hipEvent_t e : m.ev) (void)hipEventDestroy(e);
        for (hipEvent_t e : s->spare_events) (void)hipEventDestroy(e);
        if (s->staging_done) {
            (void)hipEventSynchronize(s->staging_done);
            (void)hipEventDestroy(s->staging_done);
        }
        if (s->staging) (void)hipHostFree(s->staging);
        delete s;
    });
}

pic_status pic_store_chunk(pic_store *s, uint64_t id, const void *k, const void *v, int32_t n_tokens,
                           hipStream_t stream) {
    return guarded([&] {
        if (!s) fail(PIC_ERR_INVALID, "null store");
        if (n_tokens <= 0) fail(PIC_ERR_INVALID, "n_tokens must be positive");
        if ((k == nullptr) != (v == nullptr)) fail(PIC_ERR_INVALID, "k and v must both be given or both be NULL");
        if (k && !s->k_pool) fail(PIC_ERR_STATE, "metadata-only store cannot hold chunk data");
        if (s->chunks.count(id)) fail(PIC_ERR_EXISTS, "chunk " + std::to_string(id) + " is already stored");
        const int B = s->cfg.page_size;
        const int32_t n_pages = (n_tokens + B - 1) / B;
        if (n_pages > (int64_t)s->free_pages.size())
            fail(PIC_ERR_OOM, "chunk needs " + std::to_string(n_pages) + " pages, " +
                                  std::to_string(s->free_pages.size()) + " free");
        Chunk c;
        c.n_tokens = n_tokens;
        c.last_use = ++s->use_clock;
        for (int i = 0; i < n_pages; ++i) c.pages.push_back(store_alloc_page(s));
        if (k) {
            // k, v hold every layer: [num_layers][n_tokens][Hkv][d]
            const int64_t elem = elem_bytes(s->cfg.dtype);
            const int64_t layer_bytes = s->shape.page_elems * s->cfg.num_pages * elem;
            const int64_t src_bytes = (int64_t)n_tokens * s->cfg.num_kv_heads * s->cfg.head_dim * elem;
            for (int l = 0; l < s->cfg.num_layers; ++l) {
                for (int32_t first = 0; first < n_pages; first += kMaxFillPages) {
                    FillPages fp;
                    fp.count = std::min<int32_t>(kMaxFillPages, n_pages - first);
                    fp.first_token = first * B;
                    fp.n_tokens = n_tokens;
                    for (int i = 0; i < fp.count; ++i) fp.ids[i] = c.pages[first + i];
                    const hipError_t e = launch_store_fill(
                        s->shape, static_cast<uint8_t *>(s->k_pool) + l * layer_bytes,
                        static_cast<uint8_t *>(s->v_pool) + l * layer_bytes,
                        static_cast<const uint8_t *>(k) + l * src_bytes, static_cast<const uint8_t *>(v) + l * src_bytes,
                        fp, stream);
                    if (e != hipSuccess) {
                        for (int32_t p : c.pages) store_unref(s, p);
                        check_hip(e, "store_fill launch");
                    }
                }
            }
        }
        s->chunks.emplace(id, std::move(c));
    });
}

pic_status pic_store_chunk_pages(const pic_store *s, uint64_t id, int32_t *pages, int32_t cap, int32_t *n_pages,
                                 int32_t *n_tokens) {
    return guarded([&] {
        if (!s) fail(PIC_ERR_INVALID, "null store");
        const Chunk &c = store_find(s, id);
        if (n_pages) *n_pages = (int32_t)c.pages.size();
        if (n_tokens) *n_tokens = c.n_tokens;
        if (pages) {
            if (cap < (int32_t)c.pages.size()) fail(PIC_ERR_INVALID, "page buffer too small");
            std::copy(c.pages.begin(), c.pages.end(), pages);
        }
    });
}

pic_status pic_store_release(pic_store *s, uint64_t id) {
    return guarded([&] {
        if (!s) fail(PIC_ERR_INVALID, "null store");
        auto it = s->chunks.find(id);
        if (it == s->chunks.end()) fail(PIC_ERR_NOT_FOUND, "chunk " + std::to_string(id) + " is not stored");
        for (int32_t p : it->second.pages) store_unref(s, p);
        s->chunks.erase(it);
    });
}

pic_status pic_store_evict(pic_store *s, int32_t target_free_pages, int32_t *evicted) {
    return guarded([&] {
        if (!s) fail(PIC_ERR_INVALID, "null store");
        if (evicted) *evicted = 0;
        if (target_free_pages < 0 || target_free_pages > s->cfg.num_pages)
            fail(PIC_ERR_INVALID, "target_free_pages must be in [0, num_pages]");
        // candidates: chunks whose pages only the chunk table holds, least recently used first
        std::vector<std::pair<uint64_t, uint64_t>> order;   // (last use, id)
        int64_t reclaimable = 0;
        for (const auto &kv : s->chunks) {
            bool only_table = true;
            for (int32_t p : kv.second.pages) only_table = only_table && s->refs[p] == 1;
            if (only_table) {
                order.push_back({kv.second.last_use, kv.first});
                reclaimable += (int64_t)kv.second.pages.size();
            }
        }
        const int64_t free_now = (int64_t)s->free_pages.size();
        if (free_now >= target_free_pages) return;
        if (free_now + reclaimable < target_free_pages)
            fail(PIC_ERR_OOM, "only " + std::to_string(free_now + reclaimable) + " pages can be freed (" +
                                  std::to_string(target_free_pages) + " asked): the rest are held by live plans");
        std::sort(order.begin(), order.end());
        int32_t n = 0;
        for (const auto &c : order) {
            if ((int64_t)s->free_pages.size() >= target_free_pages) break;
            auto it = s->chunks.find(c.second);
            for (int32_t p : it->second.pages) store_unref(s, p);
            s->chunks.erase(it);
            ++n;
        }
        s->evictions += n;
        if (evicted) *evicted = n;
    });
}

pic_status pic_store_usage(const pic_store *s, pic_store_usage_info *u) {
    return guarded([&] {
        if (!s || !u) fail(PIC_ERR_INVALID, "null argument");
        int64_t chunk_pages = 0;
        for (const auto &kv : s->chunks) chunk_pages += (int64_t)kv.second.pages.size();
        u->pages_total = s->cfg.num_pages;
        u->pages_free = (int64_t)s->free_pages.size();
        u->pages_chunks = chunk_pages;
        u->pages_plans_only = u->pages_total - u->pages_free - chunk_pages;
        u->chunks = (int64_t)s->chunks.size();
        u->plans = s->live_plans;
        u->evictions = s->evictions;
    });
}

pic_status pic_store_stats(const pic_store *s, int32_t *free_pages, int32_t *chunks, int32_t *plans) {
    return guarded([&] {
        if (!s) fail(PIC_ERR_INVALID, "null store");
        if (free_pages) *free_pages = (int32_t)s->free_pages.size();
        if (chunks) *chunks = (int32_t)s->chunks.size();
        if (plans) *plans = s->live_plans;
    });
}

pic_status pic_link_plan(pic_store *s, const pic_request *reqs, int32_t n_reqs, const pic_link_options *opts,
                         pic_plan **out) {
    return guarded([&] {
        if (!s || !opts || !out) fail(PIC_ERR_INVALID, "null argument");
        *out = nullptr;
        *out = build_plan(s, reqs, n_reqs, *opts);
    });
}

pic_status pic_plan_info(const pic_plan *plan, pic_plan_sizes *sz) {
    return guarded([&] {
        if (!plan || !sz) fail(PIC_ERR_INVALID, "null argument");
        sz->rows = (int64_t)plan->row_pos.size();
        sz->pages = (int64_t)plan->pages.size();
        sz->private_pages = (int64_t)plan->scatter.size();
        sz->cow_pages = (int64_t)plan->cow_src.size();
        sz->work_items = (int64_t)plan->work.size();
        sz->split_items = plan->n_split_items;
        sz->workspace_bytes = plan->workspace_bytes;
        sz->requests = plan->n_requests;
        sz->rotated_pages = plan->rotate_keys ? (int64_t)plan->pages.size() : 0;
        sz->decode_items = plan->n_dec_slots;
        sz->table_bytes = plan->table_bytes;
        sz->partial_bytes = plan->off_k_rot - plan->off_part_o;
        sz->rotated_key_bytes = plan->off_link_end - plan->off_k_rot;
        sz->decode_partial_bytes = plan->off_dec_end - plan->off_dec_o;
    });
}

pic_status pic_plan_export(const pic_plan *plan, int32_t *row_pos, int32_t *row_dst, int32_t *block_table,
                           int32_t *pos_map, int32_t *cu_rows, int32_t *cu_pages, int32_t *cow_src,
                           int32_t *cow_dst) {
    return guarded([&] {
        if (!plan) fail(PIC_ERR_INVALID, "null plan");
        const int B = plan->owner->cfg.page_size;
        if (row_pos) std::copy(plan->row_pos.begin(), plan->row_pos.end(), row_pos);
        if (row_dst) std::copy(plan->row_dst.begin(), plan->row_dst.end(), row_dst);
        for (size_t i = 0; i < plan->pages.size(); ++i) {
            const PageDesc &pd = plan->pages[i];
            if (block_table) block_table[i] = pd.phys;
            if (pos_map)
                for (int sl = 0; sl < B; ++sl) pos_map[i * B + sl] = sl < pd.valid ? pd.pos0 + sl : -1;
        }
        if (cu_rows) std::copy(plan->cu_rows.begin(), plan->cu_rows.end(), cu_rows);
        if (cu_pages) std::copy(plan->cu_pages.begin(), plan->cu_pages.end(), cu_pages);
        if (cow_src) std::copy(plan->cow_src.begin(), plan->cow_src.end(), cow_src);
        if (cow_dst) std::copy(plan->cow_dst.begin(), plan->cow_dst.end(), cow_dst);
    });
}

pic_status pic_plan_upload(pic_store *s, pic_plan *plan, void *workspace, int64_t workspace_bytes,
                           hipStream_t stream) {
    return guarded([&] {
        if (!s || !plan) fail(PIC_ERR_INVALID, "null argument");
        if (plan->owner != s) fail(PIC_ERR_INVALID, "plan belongs to another store");
        if (!s->k_pool) fail(PIC_ERR_STATE, "metadata-only store has no device");
        upload_tables(s, plan, workspace, workspace_bytes, stream);
    });
}

pic_status pic_link_attend(pic_store *s, const pic_plan *plan, const void *q_new, const void *k_new,
                           const void *v_new, void *out, float *lse, void *workspace, int64_t workspace_bytes,
                           hipStream_t stream) {
    return guarded([&] {
        check_link_call(s, plan, q_new, k_new, v_new, out);
        if (workspace_bytes < plan->workspace_bytes) fail(PIC_ERR_WORKSPACE, "workspace too small");
        // the plan's tables are copied in first unless this workspace region still holds them
        if (!s->ledger.holds(plan, workspace))
            upload_tables(s, const_cast<pic_plan *>(plan), workspace, workspace_bytes, stream);
        launch_link(s, plan, 0, q_new, k_new, v_new, out, lse, static_cast<uint8_t *>(workspace), s->profiling, stream);
    });
}

pic_status pic_link_attend_layer(pic_store *s, const pic_plan *plan, int32_t layer, const void *q_new,
                                 const void *k_new, const void *v_new, void *out, float *lse, void *workspace,
                                 int64_t workspace_bytes, hipStream_t stream) {
    return guarded([&] {
        check_link_call(s, plan, q_new, k_new, v_new, out);
        if (layer < 0 || layer >= s->cfg.num_layers)
            fail(PIC_ERR_INVALID, "layer must be in [0, " + std::to_string(s->cfg.num_layers) + ")");
        if (workspace_bytes < plan->workspace_bytes) fail(PIC_ERR_WORKSPACE, "workspace too small");
        if (!s->ledger.holds(plan, workspace))
            upload_tables(s, const_cast<pic_plan *>(plan), workspace, workspace_bytes, stream);
        launch_link(s, plan, layer, q_new, k_new, v_new, out, lse, static_cast<uint8_t *>(workspace), s->profiling,
                    stream);
    });
}

pic_status pic_link_attend_static(pic_store *s, const pic_plan *plan, const void *q_new, const void *k_new,
                                  const void *v_new, void *out, float *lse, hipStream_t stream) {
    return guarded([&] {
        check_link_call(s, plan, q_new, k_new, v_new, out);
        if (plan->workspace_bytes > kStaticScratchBytes)
            fail(PIC_ERR_WORKSPACE, "the plan needs " + std::to_string(plan->workspace_bytes) +
                                        " bytes of workspace; the static scratch holds " +
                                        std::to_string(kStaticScratchBytes));
        void *scratch = nullptr;
        check_hip(static_scratch(&scratch), "static scratch address");
        // the tables go straight from the plan's host arrays (pageable memory: each copy has read
        // its source when it returns), so no staging buffer is needed
        uint8_t *ws = static_cast<uint8_t *>(scratch);
        auto put = [&](int64_t off, const void *src, size_t bytes) {
            if (bytes)
                check_hip(hipMemcpyAsync(ws + off, src, bytes, hipMemcpyHostToDevice, stream), "plan table copy");
        };
        put(plan->off_pages, plan->pages.data(), plan->pages.size() * sizeof(PageDesc));
        put(plan->off_page_scatter, plan->page_scatter.data(), plan->page_scatter.size() * sizeof(int32_t));
        put(plan->off_row_pos, plan->row_pos.data(), plan->row_pos.size() * sizeof(int32_t));
        put(plan->off_scatter, plan->scatter.data(), plan->scatter.size() * sizeof(ScatterDesc));
        put(plan->off_work, plan->work.data(), plan->work.size() * sizeof(WorkDesc));
        put(plan->off_merge, plan->merge.data(), plan->merge.size() * sizeof(MergeDesc));
        static const uint32_t zero_tickets[kMaxWorkQueues + 1] = {};
        put(plan->off_ticket, zero_tickets, sizeof(zero_tickets));
        put(plan->off_dec_work, plan->dec_work.data(), plan->dec_work.size() * sizeof(DecodeDesc));
        put(plan->off_dec_merge, plan->dec_merge.data(), plan->dec_merge.size() * sizeof(DecodeMergeDesc));
        pic_plan *mp = const_cast<pic_plan *>(plan);
        s->ledger.claim(mp, scratch, plan->workspace_bytes);   // its caller workspace no longer holds it
        launch_link(s, plan, 0, q_new, k_new, v_new, out, lse, ws, false, stream);
    });
}

pic_status pic_link_decode(pic_store *s, const pic_plan *plan, const void *q, const void *k, const void *v,
                           void *out, float *lse, void *workspace, int64_t workspace_bytes, hipStream_t stream) {
    return guarded([&] {
        if (!s || !plan) fail(PIC_ERR_INVALID, "null argument");
        if (plan->owner != s) fail(PIC_ERR_INVALID, "plan belongs to another store");
        if (!s->k_pool) fail(PIC_ERR_STATE, "metadata-only store has no device");
        if (!plan->decode) fail(PIC_ERR_STATE, "plan was not made for decode (opts.decode)");
        if (s->cfg.num_layers != 1) fail(PIC_ERR_STATE, "decode after link runs on single-layer stores");
        if (workspace_bytes < plan->workspace_bytes) fail(PIC_ERR_WORKSPACE, "workspace too small");
        if (!s->ledger.holds(plan, workspace))
            fail(PIC_ERR_WORKSPACE, "the workspace does not hold this plan's tables (never uploaded there, or "
                                    "another plan was uploaded over them)");
        if (plan->attended_ws != workspace)
            fail(PIC_ERR_STATE, "run pic_link_attend on this workspace first (it writes the recomputed rows and "
                                "clears the decode slots that decode reads)");
        if (plan->dec_next >= plan->dec_steps)
            fail(PIC_ERR_STATE, "all " + std::to_string(plan->dec_steps) + " reserved decode steps are used");
        if (plan->n_requests == 0) return;
        if (!q || !k || !v || !out) fail(PIC_ERR_INVALID, "null tensor");
        uint8_t *ws = static_cast<uint8_t *>(workspace);
        DecodeTables t;
        t.pages = reinterpret_cast<const PageDesc *>(ws + plan->off_pages);
        t.step = plan->dec_next;
        t.work = reinterpret_cast<const DecodeDesc *>(ws + plan->off_dec_work);
        t.n_work = (int)plan->dec_work.size();
        t.merge = reinterpret_cast<const DecodeMergeDesc *>(ws + plan->off_dec_merge);
        t.n_merge = (int)plan->dec_merge.size();
        t.part_o = reinterpret_cast<float *>(ws + plan->off_dec_o);
        t.part_lse = reinterpret_cast<float *>(ws + plan->off_dec_lse);
        t.max_pos = s->cfg.max_position;
        t.k_rot = plan->rotate_keys ? ws + plan->off_k_rot : nullptr;
        check_hip(launch_decode(s->shape, q, k, v, s->k_pool, s->v_pool, s->rope, t, out, lse, stream),
                  "decode launch");
        const_cast<pic_plan *>(plan)->dec_next += 1;
    });
}

pic_status pic_plan_free(pic_store *s, pic_plan *plan) {
    return guarded([&] {
        if (!s || !plan) fail(PIC_ERR_INVALID, "null argument");
        if (plan->owner != s) fail(PIC_ERR_INVALID, "plan belongs to another store");
        s->ledger.drop(plan);
        release_plan(s, plan);
    });
}

pic_status pic_profile_enable(pic_store *s, int32_t on) {
    return guarded([&] {
        if (!s) fail(PIC_ERR_INVALID, "null store");
        for (auto &m : s->pending)
            for (hipEvent_t e : m.ev) s->spare_events.push_back(e);
        s->pending.clear();
        s->profiling = on != 0;
        s->profiled_calls = 0;
        for (double &m : s->profiled_ms) m = 0.0;
    });
}

pic_status pic_profile_read(pic_store *s, double *ms, int32_t *calls) {
    return guarded([&] {
        if (!s) fail(PIC_ERR_INVALID, "null store");
        for (auto &m : s->pending) {
            check_hip(hipEventSynchronize(m.ev[4]), "hipEventSynchronize");
            // event intervals: scatter, key rotation, attention, merge
            static const int kStage[4] = {0, 3, 1, 2};
            for (int i = 0; i < 4; ++i) {
                float t = 0.0f;
                check_hip(hipEventElapsedTime(&t, m.ev[i], m.ev[i + 1]), "hipEventElapsedTime");
                s->profiled_ms[kStage[i]] += t;
            }
            s->profiled_calls += 1;
            for (hipEvent_t e : m.ev) s->spare_events.push_back(e);
        }
        s->pending.clear();
        if (ms)
            for (int i = 0; i < 4; ++i) ms[i] = s->profiled_ms[i];
        if (calls) *calls = s->profiled_calls;
    });
}

}  // extern "C"
