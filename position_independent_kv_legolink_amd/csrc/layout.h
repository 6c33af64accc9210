// Device-side plan tables shared by the host planner and the HIP kernels.
// Every struct is plain int32 data, uploaded once per plan into the caller's
// workspace and read by the kernels of one link call.
#pragma once

#include <stdint.h>

namespace piclink {

// One logical page of a request: where it lives and which positions it holds.
struct PageDesc {
    int32_t phys;    // physical page id in the pools
    int32_t pos0;    // absolute position of slot 0
    int32_t valid;   // slots [0, valid) hold tokens, the rest are padding
    int32_t seg0;    // keys rotated inside their segment: the rotation that places them, the
                     // segment's start minus the store's compile offset (negative when the segment
                     // starts before that offset)
};

// One private page written by the scatter kernel before attention:
// slots [0, n_new) take new rows row0.., slots [n_new, n_valid) are copied
// from page `src` (copy-on-write, src >= 0), slots [n_valid, page) are zeroed.
// local0 is the rotation of slot 0's new key in a store whose keys are rotated at their position
// inside their segment: that position plus the store's compile offset.
struct ScatterDesc {
    int32_t dst;
    int32_t src;
    int32_t n_new;
    int32_t row0;
    int32_t n_valid;
    int32_t local0;
    int32_t pad1, pad2;
};

// One attention work item: a tile of consecutive selected rows of one request
// (all query heads of one KV head) over the logical pages [page_begin,
// page_end) of that request.
struct WorkDesc {
    int32_t page_base;   // index of the request's logical page 0 in the PageDesc table
    int32_t page_begin;
    int32_t page_end;
    int32_t row0;        // first selected row (global index)
    int32_t n_rows;      // selected rows in the tile; 0 = empty slot, exit
    int32_t kv_head;
    int32_t partial;     // -1: final output; else partial-result slot of this split
    int32_t pad;
};

// Combine the partial results of the splits of one (row tile, KV head).
struct MergeDesc {
    int32_t row0;
    int32_t n_rows;
    int32_t kv_head;
    int32_t n_split;
    int32_t slot0;
    int32_t pad0, pad1, pad2;
};

// One decode work item: the new token of request `request` (the G query heads of KV head
// kv_head) over the logical pages [page_begin, page_end) of that request. Every item writes a
// partial result into slot `partial` (-1: an empty slot of the work list, which does nothing).
struct DecodeDesc {
    int32_t page_base;   // index of the request's logical page 0 in the PageDesc table
    int32_t page_begin;
    int32_t page_end;
    int32_t request;
    int32_t kv_head;
    int32_t partial;
    int32_t pos;         // the request's first decode position (its DecodeReq's), read with the rest
    int32_t pad0;
};

// Decode slots of one request: its first decode token's position and where its decode tokens
// are written (token i at logical page lpage0 + (off + i) / page, slot (off + i) % page).
struct DecodeReq {
    int32_t pos;
    int32_t lpage0;
    int32_t off;
    int32_t seg0;    // start of the segment holding the slots minus the store's compile offset: a decode
                     // key at position p is written rotated at p - seg0 in a store of keys rotated
                     // inside their segment
};

// Combine the partial results of one (request, KV head) with the new token's own key. `req` is a
// copy of the request's DecodeReq, so that the merge starts its loads after one descriptor read.
struct DecodeMergeDesc {
    int32_t request;
    int32_t kv_head;
    int32_t n_split;
    int32_t slot0;
    DecodeReq req;
};

constexpr int kKeysPerTile = 64;   // keys staged in LDS per attention iteration
constexpr int kMaxWorkQueues = 8;    // queues of an attention work list (one per XCD)
constexpr int kMaxItemPages = 2048;  // longest KV range of one attention work item (its page table sits in LDS)
constexpr int kMaxDecodePages = 1024;  // longest KV range of one decode work item (its page table sits in LDS)
constexpr int kDecodeMinPages = 96;    // decode ranges shorter than this give way to one range per compute unit
// Positions are packed with a page's valid count into one 32-bit word (pos0 << 7 | valid) and
// cos/sin rows are addressed with 32-bit byte offsets: both hold below this bound.
constexpr int kMaxPosition = 1 << 22;
// Largest compile offset (leading tokens a chunk was compiled after) a store takes.
constexpr int kMaxCompileOffset = 4096;
// Most decoder layers a store holds K/V pools for.
constexpr int kMaxLayers = 1024;
constexpr int kThreads = 256;      // page writers, merge and the fp32 attention kernel
// Automatic key rotation mode: rotate once per link call when the work list reads each key page
// at least this many times on average (else inside attention). The rotation pass costs about as
// much as 5 reads' worth of rotation inside attention.
constexpr int kRotateReuse = 5;

// Device scratch of the allocation-free link call: the largest plan workspace it takes.
constexpr int64_t kStaticScratchBytes = int64_t(64) << 20;

// (row, head) pairs handled by one attention work group: 8 waves x 32 rows (bf16), 4 x 32 (fp32).
constexpr int tile_qrows(int dtype) { return dtype == 0 ? 256 : 128; }

}  // namespace piclink
