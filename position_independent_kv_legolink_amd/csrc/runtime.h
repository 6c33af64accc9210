// Host-side state behind the C ABI: the paged chunk store and link plans.
#pragma once

#include <stdint.h>

#include <new>
#include <set>
#include <stdexcept>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/piclink.h"
#include "launch.h"
#include "layout.h"
#include "ledger.h"

namespace piclink {

// Status + message carried back to the C ABI.
struct Error {
    pic_status status;
    std::string message;
};

[[noreturn]] void fail(pic_status status, const std::string &message);
void check_hip(hipError_t e, const char *what);

extern thread_local std::string g_last_error;

// Runs f, turning every C++ exception into a status and the thread's last-error message; no
// exception crosses the C ABI.
template <typename F>
pic_status guarded(F &&f) {
    try {
        f();
        return PIC_OK;
    } catch (const Error &e) {
        g_last_error = e.message;
        return e.status;
    } catch (const std::bad_alloc &) {
        g_last_error = "host allocation failed";
        return PIC_ERR_OOM;
    } catch (const std::exception &e) {
        g_last_error = e.what();
        return PIC_ERR_INVALID;
    } catch (...) {
        g_last_error = "unknown error";
        return PIC_ERR_INVALID;
    }
}

struct Chunk {
    int32_t n_tokens = 0;
    std::vector<int32_t> pages;
    uint64_t last_use = 0;   // store clock at ingest or at the last plan that linked it
};

struct ProfileMarks {
    hipEvent_t ev[5];   // before scatter, before key rotation, before attention, before merge, after merge
};

}  // namespace piclink

struct pic_store {
    pic_store_config cfg{};
    piclink::LayerShape shape{};
    void *k_pool = nullptr;
    void *v_pool = nullptr;
    float *rope = nullptr;
    std::vector<int32_t> refs;          // references per physical page (chunk table + live plans)
    std::set<int32_t> free_pages;       // lowest id first
    std::unordered_map<uint64_t, piclink::Chunk> chunks;
    int32_t live_plans = 0;
    uint64_t use_clock = 0;             // advanced by every chunk ingest and every link plan
    int64_t evictions = 0;              // chunks released by pic_store_evict
    int32_t num_cus = 256;              // compute units used by the work-list split policy
    bool profiling = false;
    int32_t profiled_calls = 0;
    double profiled_ms[4] = {0, 0, 0, 0};   // scatter, attention, merge, key rotation
    std::vector<piclink::ProfileMarks> pending;
    std::vector<hipEvent_t> spare_events;
    // pinned host buffer the plan tables are uploaded from, and the event recorded after the last
    // upload's copy out of it
    void *staging = nullptr;
    int64_t staging_bytes = 0;
    hipEvent_t staging_done = nullptr;
    piclink::WorkspaceLedger<pic_plan> ledger;   // which plan's tables each workspace region holds
};

struct pic_plan {
    pic_store *owner = nullptr;
    int32_t n_requests = 0;
    std::vector<int32_t> row_pos, row_dst, cu_rows, cu_pages;
    std::vector<piclink::PageDesc> pages;
    std::vector<piclink::ScatterDesc> scatter;
    std::vector<int32_t> page_scatter;  // per logical page: its scatter entry, or -1 (shared page)
    std::vector<int32_t> cow_src, cow_dst;
    std::vector<piclink::WorkDesc> work;
    int32_t work_queues = 1;            // queues interleaved in `work` (its size is a multiple)
    std::vector<piclink::MergeDesc> merge;
    std::vector<int32_t> page_refs;     // every physical page this plan holds a reference on
    int32_t n_slots = 0;
    int64_t n_split_items = 0;
    // workspace layout (byte offsets)
    int64_t off_pages = 0, off_page_scatter = 0, off_row_pos = 0, off_scatter = 0, off_work = 0, off_merge = 0, off_ticket = 0;
    int64_t off_part_o = 0, off_part_lse = 0, table_bytes = 0, workspace_bytes = 0;
    bool rotate_keys = false;           // keys rotated into the workspace before attention
    int64_t off_k_rot = 0;
    // decode after link (plans made with opts.decode)
    bool decode = false;
    int32_t dec_steps = 0;              // decode steps reserved per request
    int32_t dec_next = 0;               // the next decode step (reset by pic_link_attend)
    std::vector<piclink::DecodeReq> dec_req;   // host only: copied into the decode and merge descriptors
    std::vector<piclink::DecodeDesc> dec_work;
    std::vector<piclink::DecodeMergeDesc> dec_merge;
    int32_t n_dec_slots = 0;            // decode partial slots: the items of dec_work that are not empty
    int64_t off_dec_work = 0, off_dec_merge = 0, off_dec_o = 0, off_dec_lse = 0, off_end = 0;
    // the link call's scratch [off_part_o, off_link_end) and decode's partials [off_dec_o,
    // off_dec_end) start at the same offset
    int64_t off_link_end = 0, off_dec_end = 0;
    const void *attended_ws = nullptr;  // workspace of the last pic_link_attend since the last upload
};

namespace piclink {

void store_check_config(const pic_store_config &cfg);
int32_t store_alloc_page(pic_store *s);
void store_ref(pic_store *s, int32_t page);
void store_unref(pic_store *s, int32_t page);
const Chunk &store_find(const pic_store *s, uint64_t id);

pic_plan *build_plan(pic_store *s, const pic_request *reqs, int32_t n_reqs, const pic_link_options &opts);
void release_plan(pic_store *s, pic_plan *plan);

// Shared by the link calls (abi.cpp) and the layer executor (forward.cpp).
void upload_tables(pic_store *s, pic_plan *plan, void *workspace, int64_t workspace_bytes, hipStream_t stream);
void check_link_call(pic_store *s, const pic_plan *plan, const void *q_new, const void *k_new, const void *v_new,
                     const void *out);
void launch_link(pic_store *s, const pic_plan *plan, int layer, const void *q_new, const void *k_new,
                 const void *v_new, void *out, float *lse, uint8_t *ws, bool prof, hipStream_t stream);

}  // namespace piclink
