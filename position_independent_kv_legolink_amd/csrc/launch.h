// Host-side launchers of the HIP kernels (kernels.hip). Internal to the library.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "layout.h"

namespace piclink {

struct LayerShape {
    int hq, hkv, d, page_size, dtype;
    int64_t page_elems;   // elements of one page in one pool: Hkv * page_size * d
    int key_layout;       // PIC_KEYS_POSITION_FREE or PIC_KEYS_SEGMENT_ROPE
};

constexpr int kMaxFillPages = 480;

struct FillPages {
    int32_t count;
    int32_t first_token;   // token index of slot 0 of ids[0] within the chunk
    int32_t n_tokens;      // tokens of the whole chunk
    int32_t ids[kMaxFillPages];
};

// Copy one chunk's [n][Hkv][d] K and V into its pages ([Hkv][page][d] each), zeroing padding.
hipError_t launch_store_fill(const LayerShape &s, void *k_pool, void *v_pool, const void *k, const void *v,
                             const FillPages &pages, hipStream_t stream);

// Scatter kernel over `n` private pages described in `table` (device). In a store of
// segment-rotated keys, new keys are rotated at their position inside their segment (rope).
hipError_t launch_scatter(const LayerShape &s, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                          const float *rope, const ScatterDesc *table, int n, hipStream_t stream);

// The scatter of `n_scatter` private pages and the keys of `n_pages` logical pages (device
// PageDesc table) rotated to their absolute positions into k_rot ([logical page][Hkv][page][d]),
// in one launch: by each key's position, or by its segment's start when the store's keys are
// rotated inside their segment. page_scatter[i] is logical page i's entry in `table`, or -1 for a
// shared page. bfloat16 layers only.
hipError_t launch_prepare(const LayerShape &s, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                          const float *rope, const PageDesc *pages, const int32_t *page_scatter, int n_pages,
                          const ScatterDesc *table, int n_scatter, void *k_rot, hipStream_t stream);

struct AttnTables {
    const PageDesc *pages;
    const int32_t *row_pos;
    const WorkDesc *work;
    int n_work;
    uint32_t *ticket;              // kMaxWorkQueues + 1 work counters (zero between launches)
    int n_queues;                  // queues of the work list (its items interleaved)
    int n_groups;                  // work groups of a persistent attention launch
    const MergeDesc *merge;
    int n_merge;
    float *part_o;
    float *part_lse;
    const void *k_rot = nullptr;   // pre-rotated keys (bf16), or null: keys rotated inside attention
};

hipError_t launch_attention(const LayerShape &s, const void *q, const void *k_pool, const void *v_pool,
                            const float *rope, const AttnTables &t, void *out, float *lse, hipStream_t stream);

hipError_t launch_merge(const LayerShape &s, const AttnTables &t, void *out, float *lse, hipStream_t stream);

struct DecodeTables {
    const PageDesc *pages;
    int step;                        // decode step: token `step` of every request
    const DecodeDesc *work;
    int n_work;
    const DecodeMergeDesc *merge;    // one per (request, KV head)
    int n_merge;
    float *part_o;                   // [item][G][d]: normalised partial outputs
    float *part_lse;                 // [item][G]: their log2-sum-exp (scores in log2 units)
    int max_pos;                     // rows of the RoPE table
    void *k_rot;                     // keys rotated ahead [logical page][Hkv][page][d], or null: decode
                                     // then rotates the pool's keys itself
};

// Decode attention (split-KV over the pre-rotated keys and the pool's values), then the merge of
// each (request, KV head)'s partial results with the new token's own key and value, which the
// merge also writes into the token's decode slot (pools and rotated keys) for later steps (bf16).
hipError_t launch_decode(const LayerShape &s, const void *q, const void *k, const void *v, void *k_pool, void *v_pool,
                         const float *rope, const DecodeTables &t, void *out, float *lse, hipStream_t stream);

// Address, on the current device, of the library's static device scratch (kStaticScratchBytes,
// one array per GPU, held until the process ends), looked up once per device.
hipError_t static_scratch(void **ptr);

}  // namespace piclink
