// Randomised driver of the C ABI on metadata-only stores (no device): stores, chunk storage up to
// pool exhaustion, link plans with valid and invalid requests and options, exports checked
// against the plan's invariants, releases while plans are alive, frees in random order. Built
// with the sanitizers by tests/test_host_sanitizers.py; exits non-zero on a broken invariant.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "piclink.h"

#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #c);    \
            exit(2);                                                               \
        }                                                                          \
    } while (0)

static void check_plan(const pic_plan *plan, int page_size) {
    pic_plan_sizes z;
    CHECK(pic_plan_info(plan, &z) == PIC_OK);
    std::vector<int32_t> row_pos(z.rows), row_dst(z.rows), bt(z.pages), pm(z.pages * page_size);
    std::vector<int32_t> cu_rows(z.requests + 1), cu_pages(z.requests + 1), cs(z.cow_pages), cd(z.cow_pages);
    CHECK(pic_plan_export(plan, row_pos.data(), row_dst.data(), bt.data(), pm.data(), cu_rows.data(),
                          cu_pages.data(), cs.data(), cd.data()) == PIC_OK);
    CHECK(cu_rows[0] == 0 && cu_rows[z.requests] == z.rows);
    CHECK(cu_pages[0] == 0 && cu_pages[z.requests] == z.pages);
    for (int64_t r = 0; r < z.requests; ++r) {
        CHECK(cu_rows[r] <= cu_rows[r + 1] && cu_pages[r] <= cu_pages[r + 1]);
        for (int32_t i = cu_rows[r] + 1; i < cu_rows[r + 1]; ++i) CHECK(row_pos[i] > row_pos[i - 1]);
        // every selected row's position appears in its request's position map
        for (int32_t i = cu_rows[r]; i < cu_rows[r + 1]; ++i) {
            bool found = false;
            for (int64_t s = (int64_t)cu_pages[r] * page_size; s < (int64_t)cu_pages[r + 1] * page_size && !found; ++s)
                found = pm[s] == row_pos[i];
            CHECK(found);
        }
    }
    for (int32_t p : bt) CHECK(p >= 0);
    CHECK(z.workspace_bytes >= 256 && z.workspace_bytes % 256 == 0);
    CHECK(z.rotated_pages == 0 || z.rotated_pages == z.pages);
}

int main(int argc, char **argv) {
    const unsigned seed = argc > 1 ? (unsigned)atoi(argv[1]) : 1u;
    const int iters = argc > 2 ? atoi(argv[2]) : 200;
    std::mt19937 g(seed);
    auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(g); };
    int plans_made = 0, errors_seen = 0;
    for (int it = 0; it < iters; ++it) {
        pic_store_config cfg{};
        const int hkv = 1 << U(0, 3), grp = 1 << U(0, 3);
        cfg.num_kv_heads = hkv;
        cfg.num_q_heads = hkv * grp;
        cfg.head_dim = U(0, 1) ? 128 : 64;
        cfg.page_size = 16 << U(0, 2);
        cfg.num_pages = U(1, 600);
        cfg.dtype = U(0, 3) ? PIC_DTYPE_BF16 : PIC_DTYPE_F32;
        cfg.rope_theta = U(0, 1) ? 5e5 : 1e4;
        cfg.max_position = U(1, 1 << 14);
        cfg.key_layout = U(0, 1) ? PIC_KEYS_SEGMENT_ROPE : PIC_KEYS_POSITION_FREE;
        if (U(0, 15) == 0) cfg.head_dim = 96;   // invalid
        if (U(0, 31) == 0) cfg.key_layout = U(0, 1) ? 2 : -1;   // invalid
        pic_store *s = nullptr;
        const pic_status cs = pic_store_create(&cfg, nullptr, nullptr, nullptr, nullptr, &s);
        if (cs != PIC_OK) {
            CHECK(cs == PIC_ERR_INVALID && s == nullptr && pic_last_error()[0] != 0);
            ++errors_seen;
            continue;
        }
        std::vector<uint64_t> ids;
        const int n_chunks = U(0, 12);
        for (int c = 0; c < n_chunks; ++c) {
            const uint64_t id = (uint64_t)U(0, 20);
            const pic_status st = pic_store_chunk(s, id, nullptr, nullptr, U(0, 400), nullptr);
            if (st == PIC_OK) {
                ids.push_back(id);
            } else {
                CHECK(st == PIC_ERR_EXISTS || st == PIC_ERR_OOM || st == PIC_ERR_INVALID);
                ++errors_seen;
            }
        }
        std::vector<pic_plan *> live;
        for (int p = 0; p < U(0, 5); ++p) {
            const int n_req = U(0, 4);
            std::vector<std::vector<uint64_t>> lists(n_req);
            std::vector<pic_request> reqs(n_req);
            for (int r = 0; r < n_req; ++r) {
                for (int i = 0; i < U(0, 5); ++i)
                    lists[r].push_back(ids.empty() || U(0, 9) == 0 ? (uint64_t)U(0, 30) : ids[U(0, (int)ids.size() - 1)]);
                reqs[r].has_prefix = !ids.empty() && U(0, 2) == 0;
                reqs[r].prefix_id = ids.empty() ? 0 : ids[U(0, (int)ids.size() - 1)];
                reqs[r].chunk_ids = lists[r].data();
                reqs[r].n_chunks = (int32_t)lists[r].size();
                reqs[r].suffix_len = U(0, 3) == 0 ? 0 : U(0, 70);
            }
            pic_link_options o{};
            // mostly valid options, now and then an invalid one
            o.k = U(0, 15) == 0 ? -1 : U(0, 40);
            o.block_level = U(0, 3) == 0;
            o.pos_offset = U(0, 5) == 0 ? U(-2, 3000) : 0;
            o.recompute_all = U(0, 7) == 0;
            o.split_pages = U(0, 3) == 0 ? U(1, 200) : U(-1, 0);
            o.rope_keys = U(0, 15) == 0 ? 3 : U(0, 2);
            o.decode = U(0, 15) == 0 ? -1 : U(0, 2) == 0 ? U(1, 40) : 0;
            pic_plan *plan = nullptr;
            const pic_status st = pic_link_plan(s, reqs.data(), n_req, &o, &plan);
            if (st == PIC_OK) {
                check_plan(plan, cfg.page_size);
                live.push_back(plan);
                ++plans_made;
            } else {
                CHECK(plan == nullptr);
                CHECK(st == PIC_ERR_INVALID || st == PIC_ERR_NOT_FOUND || st == PIC_ERR_OOM);
                ++errors_seen;
            }
            // evict towards a random free-page target: success reaches it, failure changes nothing
            if (U(0, 4) == 0) {
                const int target = U(-1, cfg.num_pages + 1);
                int32_t f0 = 0, c0 = 0, f1 = 0, c1 = 0, n = -1;
                CHECK(pic_store_stats(s, &f0, &c0, nullptr) == PIC_OK);
                const pic_status es = pic_store_evict(s, target, &n);
                CHECK(pic_store_stats(s, &f1, &c1, nullptr) == PIC_OK);
                if (es == PIC_OK) {
                    CHECK(f1 >= target && c0 - c1 == n && n >= 0);
                } else {
                    CHECK((es == PIC_ERR_INVALID || es == PIC_ERR_OOM) && f1 == f0 && c1 == c0);
                    ++errors_seen;
                }
                // chunks that eviction released are gone from the id list
                std::vector<uint64_t> kept;
                for (uint64_t id : ids) {
                    int32_t np = 0, nt = 0;
                    if (pic_store_chunk_pages(s, id, nullptr, 0, &np, &nt) == PIC_OK) kept.push_back(id);
                }
                ids = kept;
                pic_store_usage_info u;
                CHECK(pic_store_usage(s, &u) == PIC_OK);
                CHECK(u.pages_free + u.pages_chunks + u.pages_plans_only == u.pages_total && u.pages_plans_only >= 0);
            }
            // release a chunk that live plans may still reference
            if (!ids.empty() && U(0, 3) == 0) {
                const int i = U(0, (int)ids.size() - 1);
                CHECK(pic_store_release(s, ids[i]) == PIC_OK);
                ids.erase(ids.begin() + i);
            }
        }
        // device calls on a metadata-only store fail cleanly
        if (!live.empty()) {
            CHECK(pic_plan_upload(s, live[0], nullptr, 0, nullptr) == PIC_ERR_STATE);
            CHECK(pic_link_attend(s, live[0], nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
                  PIC_ERR_STATE);
            CHECK(pic_link_decode(s, live[0], nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
                  PIC_ERR_STATE);
        }
        if (!live.empty()) CHECK(pic_store_destroy(s) == PIC_ERR_STATE);
        std::shuffle(live.begin(), live.end(), g);
        for (pic_plan *pl : live) CHECK(pic_plan_free(s, pl) == PIC_OK);
        for (uint64_t id : ids) CHECK(pic_store_release(s, id) == PIC_OK);
        int32_t free_pages = -1, chunks = -1, plans = -1;
        CHECK(pic_store_stats(s, &free_pages, &chunks, &plans) == PIC_OK);
        CHECK(free_pages == cfg.num_pages && chunks == 0 && plans == 0);   // every page came back
        CHECK(pic_store_destroy(s) == PIC_OK);
    }
    printf("ok: %d iterations, %d plans, %d rejected calls\n", iters, plans_made, errors_seen);
    return 0;
}
