// Link planner: turns requests into the device tables of one link call.
//
// Rules (EPIC, atlas.scime.ai summary, "Approach"; MEPIC, searcharxiv.org abstract):
//   - segments are [prefix] chunk* [suffix]; chunk tokens were compiled from position 0 and
//     are placed at the running offset of the prompt, starting at pos_offset;
//   - recomputed rows: the first min(k, L) tokens of every chunk, or min(page, L) in the
//     block-level variant, and every suffix token; a prefix is cached and not recomputed;
//   - every segment starts on a fresh page; pages that hold no recomputed row stay shared
//     with the store; the others are private to the request and, when they also keep cached
//     rows, are filled copy-on-write from their stored page;
//   - every page carries its segment's start, the rotation of keys stored as a chunk compiled
//     from position 0 leaves them, and every private page its first slot's position inside the
//     segment, where the scatter rotates new keys to in such a store.
// The attention work list then cuts each request's rows into tiles of tile_qrows / G rows,
// one work item per (tile, KV head), splits key ranges longer than a compute unit's average
// load (or the kernel's page-table limit) and orders the items longest first, grouped so that
// one KV head's items land on one XCD.
#include <algorithm>
#include <numeric>

#include "runtime.h"

namespace piclink {
namespace {

struct Seg {
    const Chunk *chunk;    // nullptr for the suffix
    int32_t length;
    int64_t start;
    int32_t recompute;
    bool suffix;
};

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

pic_plan *build_plan(pic_store *s, const pic_request *reqs, int32_t n_reqs, const pic_link_options &o) {
    const pic_store_config &cfg = s->cfg;
    const int B = cfg.page_size;
    if (n_reqs < 0 || (n_reqs > 0 && !reqs)) fail(PIC_ERR_INVALID, "bad request array");
    if (o.k < 0) fail(PIC_ERR_INVALID, "k must be >= 0");
    if (o.pos_offset < 0) fail(PIC_ERR_INVALID, "pos_offset must be >= 0");
    if (o.rope_keys < 0 || o.rope_keys > 2) fail(PIC_ERR_INVALID, "rope_keys must be 0, 1 or 2");
    if (o.rope_keys == 2 && cfg.dtype != PIC_DTYPE_BF16)
        fail(PIC_ERR_INVALID, "keys are rotated ahead of attention for bfloat16 stores only");
    if (o.decode < 0 || o.decode > kMaxPosition) fail(PIC_ERR_INVALID, "decode must be in [0, max_position]");
    if (o.decode && cfg.dtype != PIC_DTYPE_BF16) fail(PIC_ERR_INVALID, "decode after link needs a bfloat16 store");

    // keys rotated inside their segment carry the compile offset on top of their position there
    const int32_t c_off = cfg.key_layout == PIC_KEYS_SEGMENT_ROPE ? cfg.compile_offset : 0;

    // ---- pass 1: segments, validation and private-page count
    std::vector<std::vector<Seg>> all(n_reqs);
    std::vector<int32_t> ends(n_reqs);   // position after each request's last token
    int64_t private_needed = 0;
    for (int r = 0; r < n_reqs; ++r) {
        const pic_request &q = reqs[r];
        if (q.n_chunks < 0 || q.suffix_len < 0 || (q.n_chunks > 0 && !q.chunk_ids))
            fail(PIC_ERR_INVALID, "request " + std::to_string(r) + ": bad chunk list or suffix");
        std::vector<Seg> &segs = all[r];
        int64_t pos = o.pos_offset;
        if (q.has_prefix) {
            const Chunk &c = store_find(s, q.prefix_id);
            segs.push_back({&c, c.n_tokens, pos, o.recompute_all ? c.n_tokens : 0, false});
            pos += c.n_tokens;
        }
        for (int i = 0; i < q.n_chunks; ++i) {
            const Chunk &c = store_find(s, q.chunk_ids[i]);
            int32_t rc;
            if (o.recompute_all) rc = c.n_tokens;
            else if (o.block_level) rc = std::min<int32_t>(B, c.n_tokens);
            else rc = std::min<int32_t>(o.k, c.n_tokens);
            segs.push_back({&c, c.n_tokens, pos, rc, false});
            pos += c.n_tokens;
        }
        if (q.suffix_len > 0) {
            segs.push_back({nullptr, q.suffix_len, pos, q.suffix_len, true});
            pos += q.suffix_len;
        }
        ends[r] = (int32_t)std::min<int64_t>(pos, INT32_MAX);
        if (o.decode > 0) {
            // decode slots after the last token: the suffix's tail and pages, or a private segment
            if (!segs.empty() && segs.back().suffix) segs.back().length += o.decode;
            else segs.push_back({nullptr, o.decode, pos, 0, true});
            pos += o.decode;
        }
        if (pos > cfg.max_position)
            fail(PIC_ERR_INVALID, "request " + std::to_string(r) + " reaches position " + std::to_string(pos - 1) +
                                      " but the store's RoPE table ends at " + std::to_string(cfg.max_position - 1));
        for (const Seg &g : segs)
            if ((int64_t)c_off + g.length > cfg.max_position)
                fail(PIC_ERR_INVALID, "request " + std::to_string(r) + ": a segment of " + std::to_string(g.length) +
                                          " tokens after the compile offset " + std::to_string(c_off) +
                                          " passes the store's RoPE table");

        for (const Seg &g : segs) {
            if (g.suffix) private_needed += (g.length + B - 1) / B;
            else private_needed += (g.recompute + B - 1) / B;
        }
    }
    if (private_needed > (int64_t)s->free_pages.size())
        fail(PIC_ERR_OOM, "link needs " + std::to_string(private_needed) + " private pages, " +
                              std::to_string(s->free_pages.size()) + " free");

    // ---- pass 2: pages, rows, scatter list
    pic_plan *plan = new pic_plan();
    plan->owner = s;
    plan->n_requests = n_reqs;
    plan->cu_rows.push_back(0);
    plan->cu_pages.push_back(0);
    std::vector<int32_t> row_page;   // request-relative logical page of every row
    for (int r = 0; r < n_reqs; ++r) {
        const int32_t page_base = (int32_t)plan->pages.size();
        for (const Seg &g : all[r]) {
            const int32_t n_pages = (g.length + B - 1) / B;
            const int32_t seg_page0 = (int32_t)plan->pages.size() - page_base;
            const int32_t seg_row0 = (int32_t)plan->row_pos.size();
            std::vector<int32_t> phys(n_pages);
            for (int q = 0; q < n_pages; ++q) {
                const int32_t valid = std::min(B, g.length - q * B);
                const int32_t n_new = std::max(0, std::min(g.recompute - q * B, valid));
                if (g.suffix || n_new > 0) {
                    const int32_t dst = store_alloc_page(s);
                    const bool cow = !g.suffix && n_new < valid;
                    const int32_t src = cow ? g.chunk->pages[q] : -1;
                    if (cow) {
                        plan->cow_src.push_back(src);
                        plan->cow_dst.push_back(dst);
                        store_ref(s, src);
                        plan->page_refs.push_back(src);
                    }
                    // slots past the new rows are copied from the stored page, or zeroed
                    plan->page_scatter.push_back((int32_t)plan->scatter.size());
                    plan->scatter.push_back(
                        {dst, src, n_new, seg_row0 + q * B, src >= 0 ? valid : n_new, q * B + c_off, 0, 0});
                    phys[q] = dst;
                } else {
                    plan->page_scatter.push_back(-1);
                    phys[q] = g.chunk->pages[q];
                    store_ref(s, phys[q]);
                }
                plan->page_refs.push_back(phys[q]);
                plan->pages.push_back({phys[q], (int32_t)(g.start + (int64_t)q * B), valid, (int32_t)(g.start - c_off)});
            }
            for (int j = 0; j < g.recompute; ++j) {
                plan->row_pos.push_back((int32_t)(g.start + j));
                plan->row_dst.push_back(phys[j / B] * B + j % B);
                row_page.push_back(seg_page0 + j / B);
            }
        }
        plan->cu_rows.push_back((int32_t)plan->row_pos.size());
        plan->cu_pages.push_back((int32_t)plan->pages.size());
    }
    s->live_plans += 1;
    // the chunks this plan links are the store's most recently used ones now
    const uint64_t now = ++s->use_clock;
    auto touch = [&](uint64_t id) {
        auto it = s->chunks.find(id);
        if (it != s->chunks.end()) it->second.last_use = now;
    };
    for (int r = 0; r < n_reqs; ++r) {
        if (reqs[r].has_prefix) touch(reqs[r].prefix_id);
        for (int i = 0; i < reqs[r].n_chunks; ++i) touch(reqs[r].chunk_ids[i]);
    }

    // ---- attention work list
    const int G = cfg.num_q_heads / cfg.num_kv_heads;
    const int tile_rows = tile_qrows(cfg.dtype) / G;
    const int ppt = kKeysPerTile / B;
    struct Item {
        WorkDesc w;
        int32_t len;
    };
    std::vector<Item> items;
    int64_t total = 0;
    for (int r = 0; r < n_reqs; ++r) {
        for (int32_t t0 = plan->cu_rows[r]; t0 < plan->cu_rows[r + 1]; t0 += tile_rows) {
            const int32_t n = std::min(tile_rows, plan->cu_rows[r + 1] - t0);
            const int32_t need = row_page[t0 + n - 1] + 1;
            for (int h = 0; h < cfg.num_kv_heads; ++h) {
                items.push_back({{plan->cu_pages[r], 0, need, t0, n, h, -1, 0}, need});
                total += need;
            }
        }
    }
    // where the keys are rotated: a key page is read once per (row tile, KV head) item that
    // covers it, and rotating it once ahead of attention pays when that happens often
    const int64_t page_heads = (int64_t)plan->pages.size() * cfg.num_kv_heads;
    if (!items.empty()) {
        if (o.rope_keys == 2) plan->rotate_keys = true;
        else if (o.rope_keys == 0)
            plan->rotate_keys = cfg.dtype == PIC_DTYPE_BF16 && total >= (int64_t)kRotateReuse * page_heads;
    }
    int64_t max_pages;
    if (o.split_pages > 0) {
        max_pages = align_up(o.split_pages, ppt);
    } else if (o.split_pages < 0) {
        max_pages = INT32_MAX;
    } else {
        // split only items longer than the average load of a compute unit: the longest-first
        // schedule then ends within about one item of the average, and shorter pieces would only
        // add merge work. A bf16 piece keeps at least 6 key tiles, so that its set-up (query
        // rotation, page table, the first two staged tiles) stays a small part of it; an fp32
        // key tile takes several times longer (fp32 MFMAs), and one tile is enough.
        const int64_t min_tiles = cfg.dtype == PIC_DTYPE_BF16 ? 6 : 1;
        max_pages = std::max<int64_t>(min_tiles * ppt, align_up((total + s->num_cus - 1) / s->num_cus, ppt));
    }
    // an item's page table is staged in LDS by the attention kernel
    max_pages = std::min<int64_t>(max_pages, kMaxItemPages);
    std::vector<Item> split;
    for (const Item &it : items) {
        if (it.len <= max_pages) {
            split.push_back(it);
            continue;
        }
        const int32_t n_split = (int32_t)((it.len + max_pages - 1) / max_pages);
        const int32_t step = (int32_t)align_up((it.len + n_split - 1) / n_split, ppt);
        const int32_t slot0 = plan->n_slots;
        int32_t used = 0;
        for (int32_t b = 0; b < it.len; b += step) {
            Item piece = it;
            piece.w.page_begin = b;
            piece.w.page_end = std::min(it.len, b + step);
            piece.w.partial = plan->n_slots++;
            piece.len = piece.w.page_end - b;
            split.push_back(piece);
            ++used;
        }
        plan->merge.push_back({it.w.row0, it.w.n_rows, it.w.kv_head, used, slot0, 0, 0, 0});
        plan->n_split_items += used;
    }
    std::stable_sort(split.begin(), split.end(), [](const Item &a, const Item &b) { return a.len > b.len; });
    constexpr int kXcds = kMaxWorkQueues;
    if (cfg.num_kv_heads % kXcds == 0) {
        // work groups are dispatched round-robin over the XCDs: slot i runs on XCD i % 8, so
        // bucket the items by KV head and interleave the buckets. The persistent kernel takes the
        // buckets as queues, work group i from queue i % 8 first.
        plan->work_queues = kXcds;
        std::vector<std::vector<WorkDesc>> bucket(kXcds);
        for (const Item &it : split) bucket[it.w.kv_head % kXcds].push_back(it.w);
        size_t depth = 0;
        for (auto &b : bucket) depth = std::max(depth, b.size());
        plan->work.assign(depth * kXcds, WorkDesc{0, 0, 0, 0, 0, 0, -1, 0});
        for (int x = 0; x < kXcds; ++x)
            for (size_t i = 0; i < bucket[x].size(); ++i) plan->work[i * kXcds + x] = bucket[x][i];
    } else {
        for (const Item &it : split) plan->work.push_back(it.w);
    }

    // ---- decode work list: every (request, KV head) cut into page ranges, about two items per
    // compute unit over the whole batch; each range's partial result goes to its own slot
    if (o.decode) {
        plan->decode = true;
        plan->dec_steps = o.decode;
        for (int r = 0; r < n_reqs; ++r) {
            // the decode tokens sit in the request's last segment, after its suffix rows
            const Seg &g = all[r].back();
            const int32_t seg_pages = (g.length + B - 1) / B;
            plan->dec_req.push_back(
                {ends[r], plan->cu_pages[r + 1] - seg_pages, g.length - o.decode, (int32_t)(g.start - c_off)});
        }
        // about two ranges per compute unit over the batch; where that makes ranges shorter than
        // kDecodeMinPages and one per unit still fills every unit, one per unit, so that fewer,
        // longer ranges carry the set-up and the merge has fewer partial results. A range's page
        // table sits in LDS: at most kMaxDecodePages pages.
        int64_t per_item = (page_heads + 2 * s->num_cus - 1) / (2 * s->num_cus);
        if (per_item < kDecodeMinPages && page_heads >= (int64_t)kDecodeMinPages * s->num_cus)
            per_item = (page_heads + s->num_cus - 1) / s->num_cus;
        per_item = std::min<int64_t>(kMaxDecodePages, std::max<int64_t>(4, per_item));
        // partial slots: (request, KV head) major, ranges in order, as the merge reads them
        std::vector<std::vector<DecodeDesc>> by_range;   // [request's range][KV head]
        int32_t n_slots = 0;
        for (int r = 0; r < n_reqs; ++r) {
            const int32_t n = plan->cu_pages[r + 1] - plan->cu_pages[r];
            const int32_t n_split = n > 0 ? (int32_t)((n + per_item - 1) / per_item) : 0;
            const int32_t step = n_split > 0 ? (n + n_split - 1) / n_split : 1;
            const size_t g0 = by_range.size();
            for (int32_t b = 0; b < n; b += step) by_range.emplace_back();
            const int32_t used = (int32_t)(by_range.size() - g0);
            for (int h = 0; h < cfg.num_kv_heads; ++h) {
                plan->dec_merge.push_back({r, h, used, n_slots, plan->dec_req[r]});
                int32_t i = 0;
                for (int32_t b = 0; b < n; b += step, ++i)
                    by_range[g0 + i].push_back(
                        {plan->cu_pages[r], b, std::min(n, b + step), r, h, n_slots + i, plan->dec_req[r].pos, 0});
                n_slots += used;
            }
        }
        // work groups are dispatched round-robin over the XCDs (slot i on XCD i % 8): the KV heads
        // of one page range go to one XCD, one after another, so that the cos/sin rows of the
        // range's keys are read into that XCD's L2 once. Empty slots (partial -1) exit at once.
        constexpr int kXcds = 8;
        std::vector<std::vector<DecodeDesc>> bucket(kXcds);
        for (size_t g = 0; g < by_range.size(); ++g)
            for (const DecodeDesc &d : by_range[g]) bucket[g % kXcds].push_back(d);
        size_t depth = 0;
        for (auto &b : bucket) depth = std::max(depth, b.size());
        int n_used = 0;
        for (auto &b : bucket) n_used += b.empty() ? 0 : 1;
        if (n_used == 1 || (int64_t)depth * kXcds > 2 * (int64_t)n_slots) {
            // too few ranges to fill the XCDs evenly: plain order
            for (auto &b : by_range)
                for (const DecodeDesc &d : b) plan->dec_work.push_back(d);
        } else {
            plan->dec_work.assign(depth * kXcds, DecodeDesc{0, 0, 0, 0, 0, -1, 0, 0});
            for (int x = 0; x < kXcds; ++x)
                for (size_t i = 0; i < bucket[x].size(); ++i) plan->dec_work[i * kXcds + x] = bucket[x][i];
        }
        plan->n_dec_slots = n_slots;
    }

    // ---- workspace layout
    int64_t off = 0;
    auto place = [&](int64_t bytes) {
        const int64_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    plan->off_pages = place((int64_t)plan->pages.size() * sizeof(PageDesc));
    plan->off_page_scatter = place((int64_t)plan->page_scatter.size() * sizeof(int32_t));
    plan->off_row_pos = place((int64_t)plan->row_pos.size() * sizeof(int32_t));
    plan->off_scatter = place((int64_t)plan->scatter.size() * sizeof(ScatterDesc));
    plan->off_work = place((int64_t)plan->work.size() * sizeof(WorkDesc));
    plan->off_merge = place((int64_t)plan->merge.size() * sizeof(MergeDesc));
    // the attention launch's work counters: zero in the uploaded tables, and back to zero at the
    // end of every launch
    plan->off_ticket = place((kMaxWorkQueues + 1) * sizeof(uint32_t));
    plan->off_dec_work = place((int64_t)plan->dec_work.size() * sizeof(DecodeDesc));
    plan->off_dec_merge = place((int64_t)plan->dec_merge.size() * sizeof(DecodeMergeDesc));
    plan->table_bytes = off;
    // the link call's scratch (split partials, rotated keys) and decode's partials share one
    // region: decode runs after the link call, in stream order, and reads neither, unless the keys
    // are rotated ahead: decode then reads the rotated copy, and its partials follow it
    const int64_t scratch0 = off;
    const int64_t tq = tile_qrows(cfg.dtype);
    plan->off_part_o = place((int64_t)plan->n_slots * tq * cfg.head_dim * sizeof(float));
    plan->off_part_lse = place((int64_t)plan->n_slots * tq * sizeof(float));
    const int64_t elem = cfg.dtype == PIC_DTYPE_BF16 ? 2 : 4;
    plan->off_k_rot = place(plan->rotate_keys ? (int64_t)plan->pages.size() * s->shape.page_elems * elem : 0);
    plan->off_link_end = off;
    if (!plan->rotate_keys) off = scratch0;
    plan->off_dec_o = place((int64_t)plan->n_dec_slots * G * cfg.head_dim * sizeof(float));
    plan->off_dec_lse = place((int64_t)plan->n_dec_slots * G * sizeof(float));
    plan->off_dec_end = off;
    off = std::max(plan->off_link_end, plan->off_dec_end);
    plan->off_end = off;
    plan->workspace_bytes = std::max<int64_t>(off, 256);
    return plan;
}

void release_plan(pic_store *s, pic_plan *plan) {
    for (int32_t p : plan->page_refs) store_unref(s, p);
    s->live_plans -= 1;
    delete plan;
}

}  // namespace piclink
