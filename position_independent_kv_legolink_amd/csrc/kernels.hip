// HIP kernels of the link step for gfx950 (CDNA4).
//
//   store_fill     chunk K/V [n][Hkv][d] -> page-aligned pool pages (compile-step product in)
//   link_scatter   recomputed rows' K/V -> request-private pages, copy-on-write of cached rows
//   rotate_keys    optional: K of every logical page rotated once at its absolute positions, for
//                  link calls whose key tiles are read by many row tiles
//   link_attention causal attention of the selected rows over their request's linked pages,
//                  RoPE applied in registers at each token's absolute position, grouped-query
//                  rows of one KV head per work group, MFMA for QK^T and PV, online softmax
//   link_merge     log-sum-exp combination of split KV ranges
//   link_decode    decode after link: each request's new token over its linked pages (split-KV),
//                  then the merge of the ranges with the token's own key
//
// Method: EPIC (atlas.scime.ai summary, "Approach": chunks compiled from position 0, the first
// k tokens of every chunk recomputed at link time) and MEPIC (searcharxiv.org abstract:
// page-aligned position-free chunk KV, RoPE fused in the attention kernel, first block
// request-specific, other blocks shared).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "launch.h"
#include "lds_dma.h"

namespace piclink {
namespace {

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// The running softmax maximum is moved lazily: exact for any stale maximum as long as the
// exponentials stay bounded, here by 2^kRescaleLog2, so the output accumulator is rescaled rarely.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kInitMax = -1.0e30f;    // fp32 kernel: maximum before the first key
constexpr int kNeverAttended = INT_MAX;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    floatx2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// A page (or any block under 4 GiB) as a buffer resource: base address and size in SGPRs, so that
// loads from it take a 32-bit per-lane offset (no per-load 64-bit address add); reads at offsets
// at or past `bytes` return zeros. Data format 32, the format of untyped loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, (int)bytes, 0x00020000);
}

// Work-group barrier that orders LDS only. A plain __syncthreads() also waits for every
// outstanding global load of the wave (vmcnt(0)), which would expose the latency of loads that
// are prefetched for later tiles and are read by their own wave only.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int swap_bits23(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

struct AttnParams {
    const void *q;
    const void *k_pool;
    const void *v_pool;
    const float *rope;          // [max_position][d]: d/2 cosines, then d/2 sines
    const void *k_rot;          // pre-rotated keys [logical page][Hkv][page][d], or null
    const PageDesc *pages;
    const int32_t *row_pos;
    const WorkDesc *work;
    uint32_t *ticket;           // n_queues + 1 work counters: zero at launch, left at zero
    int n_work;                 // a multiple of n_queues
    int n_queues;
    int persistent;             // one work group per compute unit over the queues, else one per item
    void *out;
    float *lse;
    float *part_o;
    float *part_lse;
    int hq, hkv, gshift, pshift;
    int64_t page_elems;
    float scale_log2;           // log2(e) / sqrt(d)
    float scale;                // 1 / sqrt(d)
    int seg_keys;               // keys stored rotated inside their segment: rotate by its start
};

// Work items of an attention launch. With more items than compute units the launch is persistent
// (p.persistent: one work group per compute unit). The list then holds p.n_queues queues
// interleaved: item i of queue q is p.work[i * n_queues + q], each queue longest first, with its
// counter in ticket[q]. A work group takes items from the queue of its XCD (work groups are
// dispatched round-robin over the 8 XCDs, and the planner puts one KV head's items in one queue,
// so that they share that XCD's L2) and, once that queue is empty, from the queue with the most
// items left: compute units that run faster take more items. Otherwise work group i runs item i
// alone. `state` is the caller's (thread 0's): 0 before its first item, 1 while its own queue
// has items, 2 after. Returns -1 when the work group is done.
__device__ __forceinline__ int next_work_item(const AttnParams &p, int &state) {
    if (!p.persistent) return state++ == 0 ? (int)blockIdx.x : -1;
    const int nq = p.n_queues;
    const uint32_t depth = (uint32_t)(p.n_work / nq);
    const int home = (int)(blockIdx.x % (uint32_t)nq);
    if (state < 2) {
        state = 1;
        const uint32_t t = atomicAdd(p.ticket + home, 1u);
        if (t < depth) return (int)t * nq + home;
        state = 2;
    }
    // every counter read at once; an item from the fullest queue, or none left. Counters only
    // grow, so this ends.
    for (;;) {
        uint32_t c[kMaxWorkQueues];
#pragma unroll
        for (int q = 0; q < kMaxWorkQueues; ++q)
            c[q] = q < nq ? __hip_atomic_load(p.ticket + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : depth;
        uint32_t least = depth;
        int best = -1;
#pragma unroll
        for (int q = 0; q < kMaxWorkQueues; ++q)
            if (c[q] < least) {
                least = c[q];
                best = q;
            }
        if (best < 0) return -1;
        const uint32_t t = atomicAdd(p.ticket + best, 1u);
        if (t < depth) return (int)t * nq + best;
    }
}

// End of a persistent launch (thread 0 of each work group, after its last item): the last work
// group to get here puts the queue counters and the exit count (ticket[n_queues]) back to zero
// for the next launch.
__device__ __forceinline__ void release_work_queues(const AttnParams &p) {
    if (!p.persistent) return;
    if (atomicAdd(p.ticket + p.n_queues, 1u) == gridDim.x - 1)
        for (int q = 0; q <= p.n_queues; ++q) atomicExch(p.ticket + q, 0u);
}

// A callable that issues piece j of a tile's loads, with the number of pieces as a constant
// (zero: no loads).
template <int N, typename F>
struct Loads {
    static constexpr int count = N;
    F f;
    __device__ __forceinline__ void operator()(int j) const { f(j); }
};

// Rotate 8 bf16 pairs (x_i, x_{i+d/2}) by (cos, sin); returns rounded bf16 words.
__device__ __forceinline__ void rope8_bf16(const u32x4 &lo, const u32x4 &hi, const floatx4 c[2],
                                           const floatx4 s[2], u32x4 &olo, u32x4 &ohi) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float x0 = bf_lo(lo[w]), x1 = bf_hi(lo[w]);
        const float y0 = bf_lo(hi[w]), y1 = bf_hi(hi[w]);
        const float c0 = c[w >> 1][2 * (w & 1)], c1 = c[w >> 1][2 * (w & 1) + 1];
        const float s0 = s[w >> 1][2 * (w & 1)], s1 = s[w >> 1][2 * (w & 1) + 1];
        olo[w] = pack_bf16(fmaf(x0, c0, -y0 * s0), fmaf(x1, c1, -y1 * s1));
        ohi[w] = pack_bf16(fmaf(y0, c0, x0 * s0), fmaf(y1, c1, x1 * s1));
    }
}

// ---------------------------------------------------------------------------------------------
// bf16 attention. Work group = 8 waves; wave w owns M-rows [32w, 32w + 32) as one 32-row MFMA
// block; M-row m is (tile row m / G, query head m % G of the work item's KV head).
//   S^T = K' Q'^T   (v_mfma_f32_32x32x16_bf16; A = rotated K rows from LDS, B = rotated Q in VGPRs)
//   O^T += V^T P^T  (A = V^T built by transposing LDS reads of V, B = P straight from the S^T
//                    accumulators)
// Ping-pong schedule: waves 0-3 (group A, one per SIMD) and waves 4-7 (group B) run the same
// per-tile sequence one phase apart, so that one wave's MFMA phase meets the other wave's VALU
// phase on every SIMD:
//   Y(t): LDS staging of tile t+2 (with the RoPE rotation of its keys unless KR), then the
//         softmax of tile t with the global loads of tile t+3 spread between its
//         exponentials; with pre-rotated keys (KR) each staged piece is written to LDS just
//         before the load that reuses its registers, so the staging writes are spread over
//         the exponentials too instead of meeting the other wave's operand reads at once (VALU)
//   X(t): PV of tile t, QK^T of tile t+1 (MFMAs and their LDS operand reads only)   (MFMA)
// with a work-group barrier after each phase; group B passes one extra barrier at the start
// (and group A one at the end), so B's phase k overlaps A's phase k+1. Tile buffers are deep
// enough for the one-phase skew: K' and key positions x3, V x4. Q carries the softmax scale and
// log2(e), and the running maximum enters S^T through one bias MFMA per 32-key block, so the
// common softmax path is exp2, a row sum and the bf16 packing. A wave past the last key tile its
// rows attend keeps staging tiles for the others, with the same barriers, and computes nothing.
// KR: keys come pre-rotated (rotate_keys, indexed by logical page) and are staged as loaded;
// otherwise they are rotated here, with the same table values and arithmetic: by each key's
// absolute position, or (SEG: the store holds keys rotated at their position inside their
// segment) by the start of the key's segment, one cos/sin row per page.
template <int D, bool KR, bool SEG>
__global__ __launch_bounds__(512, 1) void link_attention_bf16(AttnParams p) {
    static_assert(!(KR && SEG), "pre-rotated keys need no segment starts");
    constexpr int NT = 512;
    constexpr int KT = kKeysPerTile;
    constexpr int KS = D + 8;          // K' row stride in LDS (bf16): conflict-free A-fragment reads
    constexpr int VS = D + 32;         // V row stride in LDS (bf16): 16 banks mod 64, so the 4 keys x 2 column
                                       // halves of one transposing read cover all 64 banks
    constexpr int NS = D / 16;         // k-steps of QK^T
    constexpr int NDB = D / 32;        // 32-wide d blocks of PV
    constexpr int KPAIRS = KT * (D / 16);          // (key, 8 dims of each half) per tile
    constexpr int VCHUNKS = KT * (D / 8);          // (key, 8 dims) per tile
    constexpr int NKP = (KPAIRS + NT - 1) / NT;
    constexpr int NVC = (VCHUNKS + NT - 1) / NT;
    constexpr int TQ = 256;
    static_assert(KT == 64, "one key per lane when deciding the tile mask");

    constexpr int KBUF = KT * KS, VBUF = KT * VS;
    __shared__ __attribute__((aligned(16))) uint16_t ks[3 * KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t vs[4 * VBUF];
    __shared__ __attribute__((aligned(16))) int kpos_s[3 * KT];
    __shared__ int pg_phys[kMaxItemPages], pg_pv[kMaxItemPages];
    __shared__ int pg_seg[SEG ? kMaxItemPages : 1];

    // the work group's items, one after the other (next_work_item)
    __shared__ int item_s;
    int wstate = 0;   // thread 0's
    for (;;) {
        __syncthreads();   // every wave is done with the previous item's LDS, item_s included
        if (threadIdx.x == 0) item_s = next_work_item(p, wstate);
        __syncthreads();
        const int item = __builtin_amdgcn_readfirstlane(item_s);
        if (item < 0) break;
        const WorkDesc w = p.work[item];
        if (w.n_rows <= 0) continue;

        // the lane's index as an opaque value per item: values derived from it are computed inside
        // the loop instead of being held in registers across it
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));

        const int wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
        const int G = 1 << p.gshift;
        const int page_size = 1 << p.pshift;
        const int ppt = KT >> p.pshift;
        const PageDesc *pg = p.pages + w.page_base;
        const int64_t head_off = (int64_t)w.kv_head * page_size * D;

        // ---- rotated Q fragments, held for the whole key range
        u32x4 qf[NS];
        int rpos;
        {
            const int m = wave * 32 + ln;
            const int ti = m >> p.gshift;
            const bool valid = ti < w.n_rows;
            const int row = w.row0 + (valid ? ti : 0);
            const int qh = w.kv_head * G + (m & (G - 1));
            const int rp = valid ? p.row_pos[row] : -1;
            rpos = rp;
            const uint16_t *qrow = static_cast<const uint16_t *>(p.q) + ((int64_t)row * p.hq + qh) * D;
            const float *cs = p.rope + (int64_t)(valid ? rp : 0) * D;
#pragma unroll
            for (int s = 0; s < NS / 2; ++s) {
                const int e0 = 16 * s + 8 * lg;
                u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
                if (valid) {
                    lo = *reinterpret_cast<const u32x4 *>(qrow + e0);
                    hi = *reinterpret_cast<const u32x4 *>(qrow + D / 2 + e0);
                }
                floatx4 c[2], sn[2];
                c[0] = *reinterpret_cast<const floatx4 *>(cs + e0);
                c[1] = *reinterpret_cast<const floatx4 *>(cs + e0 + 4);
                sn[0] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + e0);
                sn[1] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + e0 + 4);
                // the softmax scale and log2(e) ride on Q: scores come out of the MFMA in log2 units
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    c[h] *= p.scale_log2;
                    sn[h] *= p.scale_log2;
                }
                rope8_bf16(lo, hi, c, sn, qf[s], qf[s + NS / 2]);
            }
        }

        // position of the wave's first row: its rows are consecutive selected rows of one request, in
        // increasing position, so a key tile needs no mask for this wave when no key lies after it (a
        // wave without rows never needs the mask: its outputs are not written)
        const int rpos0 = __builtin_amdgcn_readfirstlane(rpos);
        const int wave_rpos0 = rpos0 < 0 ? INT_MAX : rpos0;
        // ... and of its last row (-1: no rows)
        int rlast = rpos;
        // the wave's largest row position: XOR swizzles within each half (no lane-address
        // registers), then the two halves
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (16 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (8 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (4 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (2 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (1 << 10)));
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(rlast, rlast, false, false);
            rlast = max((int)sw[0], (int)sw[1]);
        }
        const int wave_rpos1 = __builtin_amdgcn_readfirstlane(rlast);

        // ---- staging registers of one key tile (global -> registers -> LDS)
        u32x4 k_lo[NKP], k_hi[NKP];
        int k_pos[NKP];
        uint32_t k_sgn[NKP];               // SEG: sign bit of the rotation (a negative angle flips the sines)
        floatx4 k_c[NKP][2], k_s[NKP][2];
        u32x4 v_r[NVC];
        u32x4 k_olo[NKP], k_ohi[NKP];      // rotated K halves on their way to LDS
        int kp_stage = kNeverAttended;
        unsigned mask_ring = 7u;           // bit (t % 3): tile t needs the causal/padding mask

        // Loop-invariant byte offsets of this thread's pieces inside a page (and inside a cos/sin
        // row), so that each load is a scalar page base plus a 32-bit lane offset.
        const char *kpool_b = static_cast<const char *>(KR ? p.k_rot : p.k_pool);
        const char *vpool_b = static_cast<const char *>(p.v_pool);
        const char *rope_b = reinterpret_cast<const char *>(p.rope);
        const uint32_t page_bytes = (uint32_t)p.page_elems * 2u;
        const int lpage0 = w.page_base + w.page_begin;   // logical page of the item's first page
        uint32_t k_loff[NKP], k_cs_off[NKP], v_loff[NVC];
        int k_slot[NKP];
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int pi = tid + NT * u;
            const int key = pi / (D / 16), c = pi % (D / 16);
            k_slot[u] = key & (page_size - 1);
            k_loff[u] = (uint32_t)(head_off + k_slot[u] * D + 8 * c) * 2u;
            k_cs_off[u] = (uint32_t)(8 * c) * 4u;
        }
#pragma unroll
        for (int u = 0; u < NVC; ++u) {
            const int pi = tid + NT * u;
            const int key = pi / (D / 8), c16 = pi % (D / 8);
            v_loff[u] = (uint32_t)(head_off + (key & (page_size - 1)) * D + 8 * c16) * 2u;
        }

        // The work item's page table is staged in LDS once: the physical page, and the page's first
        // position and valid token count packed as pos0 << 7 | valid (pos0 < 2^22, valid <= 64).
        // The descriptors of a tile's KT / page pages are read from LDS early in the MFMA phase and
        // moved to SGPRs where the loads of the same phase use them. Keys of one wave's K pieces (and
        // of each of its V pieces) lie in one page (page >= 16 tokens). Keys past the work item's
        // range or in page padding read real, finite pool data (the last page, or the zeroed padding
        // slots) and are removed by the mask (position kNeverAttended).
        const int n_pages = w.page_end - w.page_begin;
        for (int i = tid; i < n_pages; i += NT) {
            const PageDesc d = pg[w.page_begin + i];
            pg_phys[i] = d.phys;
            pg_pv[i] = (d.pos0 << 7) | d.valid;
            if constexpr (SEG) pg_seg[i] = d.seg0;
        }
        lds_barrier();
        // descriptor values read ahead from LDS: the wave's K page and V pages (uniform) and the
        // page of key `lane` (for the mask positions). The reads are unconditional (clamped to the
        // last page) and the range test is applied where the values are used: a conditional read
        // becomes a branch whose join waits for the LDS result at once.
        int rk_phys[NKP], rk_pv[NKP], rk_seg[NKP], rv_phys[NVC], rl_pv;
        bool rk_in[NKP], rl_in;
        auto load_desc = [&](int t) __attribute__((always_inline)) {
            const int r0 = t * ppt;
            const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
            for (int u = 0; u < NKP; ++u) {
                const int rq = r0 + (((NT * u + 64 * wv) / (D / 16)) >> p.pshift);
                const int r = min(rq, n_pages - 1);
                if constexpr (KR) {
                    rk_phys[u] = lpage0 + r;
                } else {
                    rk_phys[u] = pg_phys[r];
                    rk_pv[u] = pg_pv[r];
                    if constexpr (SEG) rk_seg[u] = pg_seg[r];
                    rk_in[u] = rq < n_pages;
                }
            }
#pragma unroll
            for (int u = 0; u < NVC; ++u)
                rv_phys[u] = pg_phys[min(r0 + (((NT * u + 64 * wv) / (D / 8)) >> p.pshift), n_pages - 1)];
            const int rq = r0 + (lane >> p.pshift);
            rl_pv = pg_pv[min(rq, n_pages - 1)];
            rl_in = rq < n_pages;
        };
        // the loads of one tile, one instruction per piece so that they can be spread between MFMAs:
        // piece 0 takes the page descriptors into SGPRs, sets the keys' positions and loads the K low
        // halves, 1 the K high halves, then V, then (keys rotated here) the cos/sin rows at the keys'
        // positions
        constexpr int NLOAD = 2 + NVC + (KR ? 0 : 4);
        __amdgpu_buffer_rsrc_t k_page[NKP];   // the key pages of this thread's pieces, as buffers
        auto load_piece = [&](int j) __attribute__((always_inline)) {
            if (j == 0) {
#pragma unroll
                for (int u = 0; u < NKP; ++u) {
                    const uint32_t phys = (uint32_t)__builtin_amdgcn_readfirstlane(rk_phys[u]);
                    if constexpr (!KR) {
                        const int pv = __builtin_amdgcn_readfirstlane(rk_pv[u]);
                        const int pos0 = pv >> 7, valid = pv & 127;
                        const int pi = tid + NT * u;
                        const bool ok = (KPAIRS % NT == 0 || pi < KPAIRS) && rk_in[u] && k_slot[u] < valid;
                        // the cos/sin row of the key's rotation (padding slots hold zeros, which
                        // rotate to zeros with any row)
                        if constexpr (SEG) {
                            // the segment's rotation may be negative (keys compiled after leading tokens
                            // linked before them): the row of its magnitude, sines negated
                            const int r = __builtin_amdgcn_readfirstlane(rk_seg[u]);
                            k_pos[u] = r < 0 ? -r : r;
                            k_sgn[u] = r < 0 ? 0x80000000u : 0u;
                        } else {
                            k_pos[u] = ok ? pos0 + k_slot[u] : pos0;
                        }
                    }
                    k_page[u] = page_rsrc(kpool_b + (uint64_t)phys * page_bytes, page_bytes);
                    k_lo[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(k_page[u], (int)k_loff[u], 0, 0));
                }
                const int slot = lane & (page_size - 1);
                kp_stage = rl_in && slot < (rl_pv & 127) ? (rl_pv >> 7) + slot : kNeverAttended;
            } else if (j == 1) {
#pragma unroll
                for (int u = 0; u < NKP; ++u)
                    k_hi[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(k_page[u], (int)(k_loff[u] + D), 0, 0));
            } else if (j < 2 + NVC) {
                const int u = j - 2;
                const char *page = vpool_b + (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(rv_phys[u]) * page_bytes;
                v_r[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(page_rsrc(page, page_bytes), (int)v_loff[u], 0, 0));
            } else {
                const int q = j - 2 - NVC;   // 0: cos lo, 1: cos hi, 2: sin lo, 3: sin hi
#pragma unroll
                for (int u = 0; u < NKP; ++u) {
                    const uint32_t off = (uint32_t)k_pos[u] * (uint32_t)(D * 4) + k_cs_off[u];
                    const floatx4 v = *reinterpret_cast<const floatx4 *>(rope_b + off + (q >> 1) * (D * 2) + (q & 1) * 16);
                    if (q < 2) k_c[u][q & 1] = v;
                    else k_s[u][q & 1] = v;
                }
            }
        };
        auto load_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NLOAD; ++j) load_piece(j);
        };

        // staging of one tile, in pieces that fit between MFMAs: the rotation of word wd (two
        // (x_i, x_{i+d/2}) pairs) of every K piece, then the LDS writes. K', V and key positions of a
        // tile share ring slot sl (of 3); the mask bit of the slot records whether any key of the tile
        // lies after the wave's first row.
        // step k rotates pair k & 1 of word k >> 1 (the even pair is held until the odd one is ready
        // to be packed with it)
        float rx[NKP], ry[NKP];
        auto rope_step = [&](int k) __attribute__((always_inline)) {
            const int wd = k >> 1, h = k & 1;
            if constexpr (SEG) {
                // a negative rotation: sines negated here, where the rotation first needs them (done
                // right after their load it would wait for the load there); k_sgn is wave-uniform
                if (k == 0) {
#pragma unroll
                    for (int u = 0; u < NKP; ++u)
                        if (k_sgn[u])
#pragma unroll
                            for (int i = 0; i < 2; ++i)
                                k_s[u][i] = __builtin_bit_cast(floatx4, __builtin_bit_cast(u32x4, k_s[u][i]) ^ k_sgn[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < NKP; ++u) {
                const float x = h ? bf_hi(k_lo[u][wd]) : bf_lo(k_lo[u][wd]);
                const float y = h ? bf_hi(k_hi[u][wd]) : bf_lo(k_hi[u][wd]);
                const float c = k_c[u][wd >> 1][2 * (wd & 1) + h], sn = k_s[u][wd >> 1][2 * (wd & 1) + h];
                const float xr = fmaf(x, c, -y * sn), yr = fmaf(y, c, x * sn);
                if (h == 0) {
                    rx[u] = xr;
                    ry[u] = yr;
                } else {
                    k_olo[u][wd] = pack_bf16(rx[u], xr);
                    k_ohi[u][wd] = pack_bf16(ry[u], yr);
                }
            }
        };
        auto write_k = [&](int sl) __attribute__((always_inline)) {
            uint16_t *kb = ks + sl * KBUF;
#pragma unroll
            for (int u = 0; u < NKP; ++u) {
                const int pi = tid + NT * u;
                if (KPAIRS % NT != 0 && pi >= KPAIRS) break;
                const int key = pi / (D / 16), c = pi % (D / 16);
                *reinterpret_cast<u32x4 *>(&kb[key * KS + 8 * c]) = k_olo[u];
                *reinterpret_cast<u32x4 *>(&kb[key * KS + D / 2 + 8 * c]) = k_ohi[u];
            }
        };
        auto write_v = [&](int vsl, int sl) __attribute__((always_inline)) {
            uint16_t *vb = vs + vsl * VBUF;
#pragma unroll
            for (int u = 0; u < NVC; ++u) {
                const int pi = tid + NT * u;
                if (VCHUNKS % NT != 0 && pi >= VCHUNKS) break;
                const int key = pi / (D / 8), c16 = pi % (D / 8);
                *reinterpret_cast<u32x4 *>(&vb[key * VS + 8 * c16]) = v_r[u];
            }
            kpos_s[sl * KT + lane] = kp_stage;   // every wave writes the same 64 values
            const unsigned bit = 1u << sl;
            mask_ring = __any(kp_stage > wave_rpos0) ? (mask_ring | bit) : (mask_ring & ~bit);
        };
        auto write_piece = [&](int j, int sl, int vsl) __attribute__((always_inline)) {
            if (j == 0) {
                kpos_s[sl * KT + lane] = kp_stage;
                const unsigned bit = 1u << sl;
                mask_ring = __any(kp_stage > wave_rpos0) ? (mask_ring | bit) : (mask_ring & ~bit);
                uint16_t *kb = ks + sl * KBUF;
#pragma unroll
                for (int u = 0; u < NKP; ++u) {
                    const int pi = tid + NT * u;
                    if (KPAIRS % NT != 0 && pi >= KPAIRS) break;
                    const int key = pi / (D / 16), c = pi % (D / 16);
                    *reinterpret_cast<u32x4 *>(&kb[key * KS + 8 * c]) = k_lo[u];
                }
            } else if (j == 1) {
                uint16_t *kb = ks + sl * KBUF;
#pragma unroll
                for (int u = 0; u < NKP; ++u) {
                    const int pi = tid + NT * u;
                    if (KPAIRS % NT != 0 && pi >= KPAIRS) break;
                    const int key = pi / (D / 16), c = pi % (D / 16);
                    *reinterpret_cast<u32x4 *>(&kb[key * KS + D / 2 + 8 * c]) = k_hi[u];
                }
            } else {
                const int u = j - 2;
                const int pi = tid + NT * u;
                if (VCHUNKS % NT == 0 || pi < VCHUNKS) {
                    const int key = pi / (D / 8), c16 = pi % (D / 8);
                    *reinterpret_cast<u32x4 *>(&(vs + vsl * VBUF)[key * VS + 8 * c16]) = v_r[u];
                }
            }
        };
        auto store_tile = [&](int sl, int vsl) __attribute__((always_inline)) {
            if constexpr (KR) {
#pragma unroll
                for (int u = 0; u < NKP; ++u) {
                    k_olo[u] = k_lo[u];
                    k_ohi[u] = k_hi[u];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) rope_step(r);
            }
            write_k(sl);
            write_v(vsl, sl);
        };

        // S^T of one tile: two 32-key blocks, NS k-steps each
        auto qk = [&](int sl, floatx16 (&sacc)[2]) {
            const uint16_t *kb = ks + sl * KBUF;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[b][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&kb[(b * 32 + ln) * KS + 16 * s + 8 * lg]);
                    sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, qf[s]), sacc[b],
                                                                       0, 0, 0);
                }
        };

        floatx16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
        // Online softmax with a lazily moved maximum carried as an MFMA bias. mrow is the running
        // maximum in log2 units of the scaled scores, kept on bf16 values, and one extra MFMA per
        // 32-key block adds -mrow to every S^T entry before the K'Q'^T k-steps (A = a unit vector
        // along one k, B = -mrow of each row along the same k), so the accumulators hold s - mrow and
        // the weights are plain exp2 of them. mrow moves only when a lane's partial sum of one tile's
        // weights leaves (0, 2^kRescaleLog2] (a weight may exceed 2^kRescaleLog2, or overflowed),
        // while the row has no maximum yet, or on tiles that need the causal/padding mask.
        float mrow = 0.0f, lrow = 0.0f;
        bool have_max = false;
        const bf16x8 bias_a = __builtin_bit_cast(bf16x8, u32x4{lg == 0 ? 0x3f80u : 0u, 0u, 0u, 0u});   // e_0
        u32x4 bias_b = {0u, 0u, 0u, 0u};   // -mrow at k = 0 (lanes 0-31 hold k 0..7 of their row)
        floatx16 sacc[2];   // S^T - mrow of the tile in flight
        u32x4 pf[2][2];     // its bf16 softmax weights, the B operands of PV

        auto tile_sum = [&](const float (&e)[2][16]) -> float {
            float part[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part[i] = e[i >> 1][8 * (i & 1)];
#pragma unroll
                for (int r = 1; r < 8; ++r) part[i] += e[i >> 1][8 * (i & 1) + r];
            }
            return (part[0] + part[1]) + (part[2] + part[3]);
        };
        // the row sum adds the fp32 weights with plain adds (a v_dot2 shares the matrix pipe and
        // would stall behind the other wave's MFMAs)
        auto apply_mask = [&](int sl) __attribute__((always_inline)) {
            const int *kp = kpos_s + sl * KT;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const i32x4 kp4 = *reinterpret_cast<const i32x4 *>(&kp[b * 32 + 8 * i + 4 * lg]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) sacc[b][4 * i + j] = kp4[j] > rpos ? -INFINITY : sacc[b][4 * i + j];
                }
        };

        // `loads(j)` issues load piece j of the next tile; the pieces are spread between the
        // exponentials so that the wave group's loads do not queue up in the vector memory pipeline
        auto softmax = [&](bool masked, int kc, auto loads) __attribute__((always_inline)) {
            constexpr int NL = decltype(loads)::count;
            float e[2][16];
            float lsum = 0.0f;
            bool exact = masked;
            if (!masked) {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    e[i >> 4][i & 15] = __builtin_amdgcn_exp2f(sacc[i >> 4][i & 15]);
                    if (NL > 0 && (i & 3) == 3 && (i >> 2) < NL) {
                        loads(i >> 2);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                lsum = tile_sum(e);
                const bool ok = have_max && lsum <= (float)(1 << (int)kRescaleLog2);   // false for inf, NaN
                exact = __any(!ok);
            }
            if (exact) {
                if (masked) {
#pragma unroll
                    for (int j = 0; j < NL; ++j) loads(j);
                    apply_mask(kc);
                }
                // the tile's maximum relative to mrow, over both lane halves of the row
                float mx = sacc[0][0];
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[b][r]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                float target = mrow;
                bool first = false;
                if (mx != -INFINITY) {            // the row sees a key of this tile
                    if (!have_max) {
                        target = mrow + mx;       // nothing accumulated yet
                        first = true;
                        have_max = true;
                    } else if (mx > 0.0f) {
                        target = mrow + mx;
                    }
                }
                // the new maximum is a bf16 value (it enters the MFMA as a bf16 operand); the shift
                // between two bf16 values is exact in fp32
                const uint32_t tb = pack_bf16(-target, 0.0f) & 0xffffu;
                const float mnew = -bf_lo(tb);
                const float shift = mnew - mrow;
                const float alpha = first ? 1.0f : __builtin_amdgcn_exp2f(-shift);
                mrow = mnew;
                bias_b[0] = lg == 0 ? tb : 0u;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) e[b][r] = __builtin_amdgcn_exp2f(sacc[b][r] - shift);
                lsum = tile_sum(e);
                lrow *= alpha;
                if (__any(alpha != 1.0f)) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                }
            }
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int u = 0; u < 4; ++u) pf[b][s2][u] = pack_bf16(e[b][8 * s2 + 2 * u], e[b][8 * s2 + 2 * u + 1]);
            lrow += lsum;
        };

        // X phase: O^T += V^T P^T for tile t (V^T operands from pairs of transposing 8-byte LDS
        // reads), then S^T = K' Q'^T for tile t+1. Only MFMAs and their operand reads: a wave issues
        // one instruction per four cycles at best, so every other instruction in this phase would
        // delay the MFMAs. Every MFMA's LDS operand is read three MFMAs ahead; the slots are
        // separated by scheduling barriers, so the order below is the issue order.
        typedef short v4s __attribute__((ext_vector_type(4)));
        constexpr int NPV = 4 * NDB;       // PV MFMAs per tile
        constexpr int NQK = 2 * NS;        // QK^T k-step MFMAs per tile
        constexpr int NBIAS = 2;           // bias MFMAs (one per 32-key block) ahead of them
        constexpr int AHEAD = 3;
        v4s vlo[NPV], vhi[NPV];
        bf16x8 ka[NQK];
        auto xphase = [&](int vsl, int ksl, auto with_qk) __attribute__((always_inline)) {
            constexpr bool QK = decltype(with_qk)::value;
            constexpr int NM = NPV + (QK ? NBIAS + NQK : 0);
            const int gi = lane >> 4, jj = (lane >> 2) & 3, qq = lane & 3;
            const uint16_t *vb = vs + vsl * VBUF + (4 * lg + jj) * VS + 16 * (gi & 1) + 4 * qq;
            const uint16_t *kb = ks + ksl * KBUF + ln * KS + 8 * lg;
            // PV MFMA i takes d block i % NDB and k-step i / NDB (32-key block b, half s2), so that
            // consecutive MFMAs accumulate into different output blocks; each block still takes its
            // k-steps in the same order
            auto read = [&](int i) __attribute__((always_inline)) {
                if (i < NPV) {
                    const int db = i % NDB, b = (i / NDB) >> 1, s2 = (i / NDB) & 1;
                    const uint16_t *a = vb + (b * 32 + 16 * s2) * VS + db * 32;
                    vlo[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)a);
                    vhi[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(a + 8 * VS));
                } else if (i >= NPV + NBIAS) {
                    const int j = i - NPV - NBIAS, s = j >> 1, b = j & 1;
                    ka[j] = *reinterpret_cast<const bf16x8 *>(kb + b * 32 * KS + 16 * s);
                }
            };
            auto mma = [&](int i) __attribute__((always_inline)) {
                if (i < NPV) {
                    const int db = i % NDB, b = (i / NDB) >> 1, s2 = (i / NDB) & 1;
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[i], vhi[i], 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pf[b][s2]), oacc[db],
                                                                       0, 0, 0);
                } else if (i < NPV + NBIAS) {
                    const floatx16 zero = {};
                    sacc[i - NPV] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bias_a, __builtin_bit_cast(bf16x8, bias_b), zero,
                                                                            0, 0, 0);
                } else {
                    const int j = i - NPV - NBIAS, s = j >> 1, b = j & 1;
                    sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], __builtin_bit_cast(bf16x8, qf[s]), sacc[b], 0, 0, 0);
                }
            };
#pragma unroll
            for (int i = 0; i < AHEAD; ++i) read(i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                mma(i);
                if (i + AHEAD < NM) read(i + AHEAD);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        const int ntiles = (w.page_end - w.page_begin + ppt - 1) / ppt;
        const bool group_b = wave >= 4;
        // Key tiles this wave attends: those whose first key is at or before its last row, a prefix
        // [0, n_act) of the item's tiles (page positions increase). Past it the wave only stages tiles
        // for the other waves, and its SIMD partner runs alone.
        int n_act;
        {
            int lo = 0, hi = n_pages;   // first page whose first position lies after the last row
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((pg_pv[mid] >> 7) <= wave_rpos1) lo = mid + 1;
                else hi = mid;
            }
            n_act = __builtin_amdgcn_readfirstlane((lo + ppt - 1) / ppt);
        }

        load_desc(0);
        load_tile();
        store_tile(0, 0);
        load_desc(1);
        load_tile();
        store_tile(1, 1);
        lds_barrier();
        qk(0, sacc);
        load_desc(2);
        load_tile();
        load_desc(3);
        if (group_b) lds_barrier();

        // ring slots of tiles t, t+1, t+2: K' and key positions in a ring of 3, V in a ring of 4 (the
        // one-phase skew between the wave groups keeps a V tile in use one phase longer)
        int kc = 0, kn = 1, ks2 = 2, vc = 0;
        // one tile. Y(t): LDS staging of tile t+2 from the registers loaded one step earlier and
        // the loads of tile t+3 into the freed registers (a whole step ahead of their use), with the
        // softmax of tile t. X(t): PV of tile t, QK^T of tile t+1, and the page descriptors of the
        // next step's loads.
        auto step = [&](int t, auto next_qk, auto staging, auto next_staging) __attribute__((always_inline)) {
            constexpr bool STAGE = decltype(staging)::value;
            if constexpr (KR) {
                // each staged piece goes to LDS just before the load that reuses its registers, so the
                // tile's LDS writes are spread over the exponentials
                const int wsl = ks2, wvsl = (vc + 2) & 3;
                const bool masked = (mask_ring >> kc) & 1u;   // read before piece 0 updates the ring
                auto stage_load = [&](int j) __attribute__((always_inline)) {
                    write_piece(j, wsl, wvsl);
                    load_piece(j);
                };
                softmax(masked, kc, Loads<STAGE ? NLOAD : 0, decltype(stage_load) &>{stage_load});
            } else {
                if constexpr (STAGE) store_tile(ks2, (vc + 2) & 3);
                softmax((mask_ring >> kc) & 1u, kc, Loads<STAGE ? NLOAD : 0, decltype(load_piece) &>{load_piece});
            }
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            xphase(vc, kn, next_qk);
            if constexpr (decltype(next_staging)::value) load_desc(t + 4);
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            const int old = kc;
            kc = kn;
            kn = ks2;
            ks2 = old;
            vc = (vc + 1) & 3;
        };
        // a step of a wave past its last key tile: the staging of tile t+2 and the loads of tile t+3,
        // with the same two barriers as `step`
        auto idle_step = [&](int t, auto staging, auto next_staging) __attribute__((always_inline)) {
            if constexpr (decltype(staging)::value) {
                store_tile(ks2, (vc + 2) & 3);
#pragma unroll
                for (int j = 0; j < NLOAD; ++j) load_piece(j);
            }
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            if constexpr (decltype(next_staging)::value) load_desc(t + 4);
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            const int old = kc;
            kc = kn;
            kn = ks2;
            ks2 = old;
            vc = (vc + 1) & 3;
        };
        using yes = std::integral_constant<bool, true>;
        using no = std::integral_constant<bool, false>;
        // every wave passes 2 barriers per tile for all ntiles tiles, active or not
        int t = 0;
        const int t_main = min(n_act, ntiles - 3);
        for (; t < t_main; ++t) step(t, yes{}, yes{}, yes{});
        for (; t + 3 < ntiles; ++t) idle_step(t, yes{}, yes{});
        if (t + 2 < ntiles) {
            if (t < n_act) step(t, yes{}, yes{}, no{});
            else idle_step(t, yes{}, no{});
            ++t;
        }
        if (t + 1 < ntiles) {
            if (t < n_act) step(t, yes{}, no{}, no{});
            else idle_step(t, no{}, no{});
            ++t;
        }
        if (t < ntiles) {
            if (t < n_act) step(t, no{}, no{}, no{});
            else idle_step(t, no{}, no{});
        }
        if (!group_b) lds_barrier();

        // ---- epilogue: normalise, write the output (or this split's partial result)
        {
            const int m = wave * 32 + ln;
            const int ti = m >> p.gshift;
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lrow), __float_as_uint(lrow), false, false);
            const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            const float lse_v = lt > 0.0f ? (mrow + __builtin_amdgcn_logf(lt)) * 0.6931471805599453f : -INFINITY;
            if (ti < w.n_rows) {
                const int row = w.row0 + ti;
                const int qh = w.kv_head * G + (m & (G - 1));
                if (w.partial < 0) {
                    uint16_t *orow = static_cast<uint16_t *>(p.out) + ((int64_t)row * p.hq + qh) * D;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int d0 = db * 32 + 8 * i + 4 * lg;
                            u32x2 v;
                            v[0] = pack_bf16(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv);
                            v[1] = pack_bf16(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
                            *reinterpret_cast<u32x2 *>(orow + d0) = v;
                        }
                    if (p.lse && lg == 0) p.lse[(int64_t)row * p.hq + qh] = lse_v;
                } else {
                    float *po = p.part_o + ((int64_t)w.partial * TQ + m) * D;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int d0 = db * 32 + 8 * i + 4 * lg;
                            floatx4 v = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                                         oacc[db][4 * i + 3] * inv};
                            *reinterpret_cast<floatx4 *>(po + d0) = v;
                        }
                    if (lg == 0) p.part_lse[(int64_t)w.partial * TQ + m] = lse_v;
                }
            }
        }
    }
    if (threadIdx.x == 0) release_work_queues(p);
}

// ---------------------------------------------------------------------------------------------
// bf16 attention over keys rotated ahead (KR), d = 128: the schedule of link_attention_bf16 with
// the K' and V tiles loaded straight from global memory into LDS (buffer_load_dwordx4 ... lds over
// one page: lane i of an instruction writes the 16 bytes it loads at the instruction's LDS base +
// 16 i). Staging then costs no registers, no LDS writes and no VALU work in the softmax phase.
//   - Rows are unpadded (256 bytes per key) and XOR-swizzled per 16-byte chunk so that the MFMA
//     operand reads stay free of bank conflicts: K' row r holds chunk c at c ^ (r & 15), so the 16
//     lanes of one b128 read take 16 rows at 16 distinct chunks; V row r holds it at c ^ 4 (r & 3),
//     so the 4 keys x 4 chunks that 32 lanes of one transposing b64 read touch are distinct. Each
//     lane fetches the global chunk that lands in its LDS position.
//   - K', V and key positions use rings of 4 slots; the K' and V slots are separate arrays and the
//     main loop is unrolled by 4, so that every slot is a compile-time constant and the compiler
//     keeps the loads of later tiles in flight past the operand reads of the current ones.
//   - Slot lifetimes under the one-phase skew of the wave groups: K' of tile t+3 is loaded in
//     Y(t) (its slot held tile t-1, read by both groups' QK^T before A's X(t-1)); V of tile t+3 in
//     X(t) (its slot held tile t-1, read by B's PV during A's Y(t)). Per wave and tile: 2 K' and 2
//     V load instructions of 1 KiB.
//   - Before the barrier that opens group A's X(t), every wave waits for its own loads of K'(t+1)
//     and V(t): group A at the end of Y(t) (8 later load instructions may stay in flight), group B
//     at the end of its X(t-1) (6 may).
template <typename T>
struct IsSlot : std::false_type {};
template <int V>
struct IsSlot<std::integral_constant<int, V>> : std::true_type {};

template <int D>
__global__ __launch_bounds__(512, 1) void link_attention_bf16_dl(AttnParams p) {
    static_assert(D == 128, "16 chunks of 16 bytes per key row");
    constexpr int NT = 512;
    constexpr int KT = kKeysPerTile;
    constexpr int NS = D / 16;         // k-steps of QK^T
    constexpr int NDB = D / 32;        // 32-wide d blocks of PV
    constexpr int TQ = 256;
    constexpr int TILE = KT * D;       // elements of one K' or V tile (16 KiB)
    static_assert(KT == 64, "one key per lane when deciding the tile mask");

    __shared__ __attribute__((aligned(16))) uint16_t k0[TILE], k1[TILE], k2[TILE], k3[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t v0[TILE], v1[TILE], v2[TILE], v3[TILE];
    __shared__ __attribute__((aligned(16))) int kpos_s[4 * KT];
    __shared__ int pg_phys[kMaxItemPages], pg_pv[kMaxItemPages];

    // the work group's items, one after the other (next_work_item)
    __shared__ int item_s;
    int wstate = 0;   // thread 0's
    for (;;) {
        barrier_dl();   // every wave is done with the previous item's LDS, item_s included
        if (threadIdx.x == 0) item_s = next_work_item(p, wstate);
        barrier_dl();
        const int item = __builtin_amdgcn_readfirstlane(item_s);
        if (item < 0) break;
        const WorkDesc w = p.work[item];
        if (w.n_rows <= 0) continue;

        // the lane's index as an opaque value per item: values derived from it are computed inside
        // the loop instead of being held in registers across it
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const int G = 1 << p.gshift;
        const int page_size = 1 << p.pshift;
        const int ppt = KT >> p.pshift;
        const PageDesc *pg = p.pages + w.page_base;
        const int64_t head_off = (int64_t)w.kv_head * page_size * D;

        // slots: compile-time (std::integral_constant) in the unrolled main loop, else run-time
        auto kslot = [&](auto s) -> uint16_t * {
            if constexpr (IsSlot<decltype(s)>::value) {
                constexpr int S = decltype(s)::value;
                if constexpr (S == 0) return k0;
                else if constexpr (S == 1) return k1;
                else if constexpr (S == 2) return k2;
                else return k3;
            } else {
                const int S = s & 3;
                return S == 0 ? k0 : S == 1 ? k1 : S == 2 ? k2 : k3;
            }
        };
        auto vslot = [&](auto s) -> uint16_t * {
            if constexpr (IsSlot<decltype(s)>::value) {
                constexpr int S = decltype(s)::value;
                if constexpr (S == 0) return v0;
                else if constexpr (S == 1) return v1;
                else if constexpr (S == 2) return v2;
                else return v3;
            } else {
                const int S = s & 3;
                return S == 0 ? v0 : S == 1 ? v1 : S == 2 ? v2 : v3;
            }
        };
        auto slot_plus = [](auto s, auto k) {
            if constexpr (IsSlot<decltype(s)>::value)
                return std::integral_constant<int, (decltype(s)::value + decltype(k)::value) & 3>{};
            else
                return (int)((s + decltype(k)::value) & 3);
        };
        using one = std::integral_constant<int, 1>;
        using three = std::integral_constant<int, 3>;

        // ---- rotated Q fragments, held for the whole key range
        u32x4 qf[NS];
        int rpos;
        {
            const int m = wave * 32 + ln;
            const int ti = m >> p.gshift;
            const bool valid = ti < w.n_rows;
            const int row = w.row0 + (valid ? ti : 0);
            const int qh = w.kv_head * G + (m & (G - 1));
            const int rp = valid ? p.row_pos[row] : -1;
            rpos = rp;
            const uint16_t *qrow = static_cast<const uint16_t *>(p.q) + ((int64_t)row * p.hq + qh) * D;
            const float *cs = p.rope + (int64_t)(valid ? rp : 0) * D;
#pragma unroll
            for (int s = 0; s < NS / 2; ++s) {
                const int e0 = 16 * s + 8 * lg;
                u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
                if (valid) {
                    lo = *reinterpret_cast<const u32x4 *>(qrow + e0);
                    hi = *reinterpret_cast<const u32x4 *>(qrow + D / 2 + e0);
                }
                floatx4 c[2], sn[2];
                c[0] = *reinterpret_cast<const floatx4 *>(cs + e0);
                c[1] = *reinterpret_cast<const floatx4 *>(cs + e0 + 4);
                sn[0] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + e0);
                sn[1] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + e0 + 4);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    c[h] *= p.scale_log2;
                    sn[h] *= p.scale_log2;
                }
                rope8_bf16(lo, hi, c, sn, qf[s], qf[s + NS / 2]);
            }
        }
        const int rpos0 = __builtin_amdgcn_readfirstlane(rpos);
        const int wave_rpos0 = rpos0 < 0 ? INT_MAX : rpos0;
        int rlast = rpos;
        // the wave's largest row position: XOR swizzles within each half (no lane-address
        // registers), then the two halves
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (16 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (8 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (4 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (2 << 10)));
        rlast = max(rlast, __builtin_amdgcn_ds_swizzle(rlast, 0x1f | (1 << 10)));
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(rlast, rlast, false, false);
            rlast = max((int)sw[0], (int)sw[1]);
        }
        const int wave_rpos1 = __builtin_amdgcn_readfirstlane(rlast);

        // ---- the item's page table in LDS: physical page, and pos0 << 7 | valid
        const int n_pages = w.page_end - w.page_begin;
        for (int i = tid; i < n_pages; i += NT) {
            const PageDesc d = pg[w.page_begin + i];
            pg_phys[i] = d.phys;
            pg_pv[i] = (d.pos0 << 7) | d.valid;
        }
        barrier_dl();

        // ---- direct loads. Instruction m (0, 1) of wave wv covers key rows 8 wv + 4 m .. + 3 of a tile
        // (one page: pages hold at least 16 keys); lane i fetches the global chunk that lands at LDS
        // chunk position i % 16 of row 8 wv + 4 m + i / 16. The page is the load's buffer and the
        // lane's offset in it (k_doff, v_doff) is the same for every tile: the buffer form took 1.3%
        // off attention at the 50k-token request against 64-bit addresses per lane.
        const char *kpool_b = static_cast<const char *>(p.k_rot);
        const char *vpool_b = static_cast<const char *>(p.v_pool);
        const uint32_t page_bytes = (uint32_t)p.page_elems * 2u;
        const int lpage0 = w.page_base + w.page_begin;   // logical page of the item's first page
        const int pg_in_tile = (8 * wv) >> p.pshift;
        uint32_t k_doff[2], v_doff[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int r = 8 * wave + 4 * m + (lane >> 4);
            const int pc = lane & 15;
            const uint32_t row_off = (uint32_t)(head_off + (int64_t)(r & (page_size - 1)) * D) * 2u;
            k_doff[m] = row_off + (uint32_t)((pc ^ (r & 15)) * 16);
            v_doff[m] = row_off + (uint32_t)((pc ^ (4 * (r & 3))) * 16);
        }
        // page of this wave's rows of tile t (keys past the item's range read its last page; the mask
        // removes them)
        auto tile_page = [&](int t) { return min(t * ppt + pg_in_tile, n_pages - 1); };
        auto dma_k = [&](int t, uint16_t *dst, int m) __attribute__((always_inline)) {
            const uint32_t phys = (uint32_t)(lpage0 + tile_page(t));
            dma16_page(kpool_b + (uint64_t)phys * page_bytes, page_bytes, k_doff[m], lds_addr(dst + (8 * wv + 4 * m) * D));
        };
        int v_phys_next = 0;   // V page of the next V tile this wave loads (read from LDS one phase ahead)
        auto dma_v = [&](uint16_t *dst, int m) __attribute__((always_inline)) {
            const uint32_t phys = (uint32_t)__builtin_amdgcn_readfirstlane(v_phys_next);
            dma16_page(vpool_b + (uint64_t)phys * page_bytes, page_bytes, v_doff[m], lds_addr(dst + (8 * wv + 4 * m) * D));
        };
        // key positions of tile t into ring slot sl, and the wave's mask bit of the slot
        unsigned mask_ring = 15u;          // bit sl: the tile in slot sl needs the causal/padding mask
        auto stage_kpos = [&](int t, int sl) __attribute__((always_inline)) {
            const int rq = t * ppt + (lane >> p.pshift);
            const int pv = pg_pv[min(rq, n_pages - 1)];
            const int slot = lane & (page_size - 1);
            const int kp = rq < n_pages && slot < (pv & 127) ? (pv >> 7) + slot : kNeverAttended;
            kpos_s[sl * KT + lane] = kp;   // every wave writes the same 64 values
            const unsigned bit = 1u << sl;
            mask_ring = __any(kp > wave_rpos0) ? (mask_ring | bit) : (mask_ring & ~bit);
        };
        auto wait_loads = [&](auto n) __attribute__((always_inline)) {
            // s_waitcnt vmcnt(n): lgkmcnt and expcnt left at their maxima
            __builtin_amdgcn_s_waitcnt((decltype(n)::value & 15) | ((decltype(n)::value >> 4) << 14) | (7 << 4) |
                                       (15 << 8));
        };

        // per-lane LDS fragment offsets (elements) of the swizzled rows. K' k-step s of key row ln reads
        // chunk (2s + lg) ^ (ln & 15): offset kfo0 ^ 16 s, since the XOR only touches bits 4-6. V^T
        // d block db of key row 4 lg + jj reads chunk (4 db + 2 (gi & 1) + qq / 2) ^ 4 jj: offset
        // vfo0 ^ 32 db (bits 5-6). Written as XORs of a per-lane base, they cost one VALU each where the
        // compiler does not keep them in registers.
        const uint32_t kfo0 = (uint32_t)(ln * D + 8 * (lg ^ (ln & 1)) + 16 * ((ln & 15) >> 1));
        auto kfo = [&](int s) { return kfo0 ^ (uint32_t)(16 * s); };
        const int gi = lane >> 4, jj = (lane >> 2) & 3, qq = lane & 3;
        const uint32_t vfo0 = (uint32_t)((4 * lg + jj) * D + 32 * jj + 16 * (gi & 1) + 4 * qq);
        auto vfo = [&](int db) { return vfo0 ^ (uint32_t)(32 * db); };

        auto qk = [&](auto ksl, floatx16 (&sacc)[2]) {
            const uint16_t *kb = kslot(ksl);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[b][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + kfo(s) + b * 32 * D);
                    sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, qf[s]), sacc[b],
                                                                       0, 0, 0);
                }
        };

        floatx16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
        float mrow = 0.0f, lrow = 0.0f;
        bool have_max = false;
        const bf16x8 bias_a = __builtin_bit_cast(bf16x8, u32x4{lg == 0 ? 0x3f80u : 0u, 0u, 0u, 0u});   // e_0
        u32x4 bias_b = {0u, 0u, 0u, 0u};
        floatx16 sacc[2];
        u32x4 pf[2][2];

        auto tile_sum = [&](const float (&e)[2][16]) -> float {
            float part[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part[i] = e[i >> 1][8 * (i & 1)];
#pragma unroll
                for (int r = 1; r < 8; ++r) part[i] += e[i >> 1][8 * (i & 1) + r];
            }
            return (part[0] + part[1]) + (part[2] + part[3]);
        };
        auto apply_mask = [&](int sl) __attribute__((always_inline)) {
            const int *kp = kpos_s + sl * KT;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const i32x4 kp4 = *reinterpret_cast<const i32x4 *>(&kp[b * 32 + 8 * i + 4 * lg]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) sacc[b][4 * i + j] = kp4[j] > rpos ? -INFINITY : sacc[b][4 * i + j];
                }
        };
        // the softmax of one tile (as link_attention_bf16); `loads(j)` issues load j of a later tile,
        // spread between the exponentials
        auto softmax = [&](bool masked, int kc, auto loads) __attribute__((always_inline)) {
            constexpr int NL = decltype(loads)::count;
            float e[2][16];
            float lsum = 0.0f;
            bool exact = masked;
            if (!masked) {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    e[i >> 4][i & 15] = __builtin_amdgcn_exp2f(sacc[i >> 4][i & 15]);
                    if (NL > 0 && (i & 7) == 7 && (i >> 3) < NL) {
                        loads(i >> 3);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                lsum = tile_sum(e);
                const bool ok = have_max && lsum <= (float)(1 << (int)kRescaleLog2);   // false for inf, NaN
                exact = __any(!ok);
            }
            if (exact) {
                if (masked) {
#pragma unroll
                    for (int j = 0; j < NL; ++j) loads(j);
                    apply_mask(kc);
                }
                float mx = sacc[0][0];
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[b][r]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                float target = mrow;
                bool first = false;
                if (mx != -INFINITY) {
                    if (!have_max) {
                        target = mrow + mx;
                        first = true;
                        have_max = true;
                    } else if (mx > 0.0f) {
                        target = mrow + mx;
                    }
                }
                const uint32_t tb = pack_bf16(-target, 0.0f) & 0xffffu;
                const float mnew = -bf_lo(tb);
                const float shift = mnew - mrow;
                const float alpha = first ? 1.0f : __builtin_amdgcn_exp2f(-shift);
                mrow = mnew;
                bias_b[0] = lg == 0 ? tb : 0u;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) e[b][r] = __builtin_amdgcn_exp2f(sacc[b][r] - shift);
                lsum = tile_sum(e);
                lrow *= alpha;
                if (__any(alpha != 1.0f)) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                }
            }
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int u = 0; u < 4; ++u) pf[b][s2][u] = pack_bf16(e[b][8 * s2 + 2 * u], e[b][8 * s2 + 2 * u + 1]);
            lrow += lsum;
        };

        // X phase: PV of the tile in V slot vsl, QK^T of the tile in K' slot ksl, MFMAs and their
        // operand reads only (operands read three MFMAs ahead), then `vloads` (V of a later tile). The
        // V loads go last: issued at the start they slowed the operand reads of the same phase.
        typedef short v4s __attribute__((ext_vector_type(4)));
        constexpr int NPV = 4 * NDB;
        constexpr int NQK = 2 * NS;
        constexpr int NBIAS = 2;
        constexpr int AHEAD = 3;
        v4s vlo[NPV], vhi[NPV];
        bf16x8 ka[NQK];
        auto xphase = [&](auto vsl, auto ksl, auto with_qk, auto vloads) __attribute__((always_inline)) {
            constexpr bool QK = decltype(with_qk)::value;
            constexpr int NM = NPV + (QK ? NBIAS + NQK : 0);
            const uint16_t *vb = vslot(vsl);
            const uint16_t *kb = kslot(ksl);
            auto read = [&](int i) __attribute__((always_inline)) {
                if (i < NPV) {
                    const int db = i % NDB, b = (i / NDB) >> 1, s2 = (i / NDB) & 1;
                    const uint16_t *a = vb + vfo(db) + (b * 32 + 16 * s2) * D;
                    vlo[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)a);
                    vhi[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(a + 8 * D));
                } else if (i >= NPV + NBIAS) {
                    const int j = i - NPV - NBIAS, s = j >> 1, b = j & 1;
                    ka[j] = *reinterpret_cast<const bf16x8 *>(kb + kfo(s) + b * 32 * D);
                }
            };
            auto mma = [&](int i) __attribute__((always_inline)) {
                if (i < NPV) {
                    const int db = i % NDB, b = (i / NDB) >> 1, s2 = (i / NDB) & 1;
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[i], vhi[i], 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pf[b][s2]), oacc[db],
                                                                       0, 0, 0);
                } else if (i < NPV + NBIAS) {
                    const floatx16 zero = {};
                    sacc[i - NPV] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bias_a, __builtin_bit_cast(bf16x8, bias_b), zero,
                                                                            0, 0, 0);
                } else {
                    const int j = i - NPV - NBIAS, s = j >> 1, b = j & 1;
                    sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], __builtin_bit_cast(bf16x8, qf[s]), sacc[b], 0, 0, 0);
                }
            };
            // issue order: the bias MFMAs first, then PV and QK^T alternating, so that each QK^T MFMA
            // follows the previous one on its accumulator four MFMAs later (two when they ran back to
            // back): 1.25% shorter at the 50k-token request. Each accumulator keeps its order, so the
            // results are those of the plain order bit for bit.
            auto op = [&](int k) -> int {
                if constexpr (!QK) return k;
                if (k < NBIAS) return NPV + k;
                const int r = k - NBIAS;
                return (r & 1) ? NPV + NBIAS + (r >> 1) : (r >> 1);
            };
#pragma unroll
            for (int k = 0; k < AHEAD; ++k) read(op(k));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NM; ++k) {
                mma(op(k));
                if (k + AHEAD < NM) read(op(k + AHEAD));
                __builtin_amdgcn_sched_barrier(0);
            }
            vloads();
            __builtin_amdgcn_sched_barrier(0);
        };

        const int ntiles = (n_pages + ppt - 1) / ppt;
        const bool group_b = wave >= 4;
        int n_act;
        {
            int lo = 0, hi = n_pages;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((pg_pv[mid] >> 7) <= wave_rpos1) lo = mid + 1;
                else hi = mid;
            }
            n_act = __builtin_amdgcn_readfirstlane((lo + ppt - 1) / ppt);
        }

        using yes = std::integral_constant<bool, true>;
        using no = std::integral_constant<bool, false>;
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        using S3 = std::integral_constant<int, 3>;
        using W6 = std::integral_constant<int, 6>;
        using W8 = std::integral_constant<int, 8>;
        using W10 = std::integral_constant<int, 10>;
        using W0 = std::integral_constant<int, 0>;

        // ---- prologue: tiles 0, 1, 2 (K', V, positions) in slots 0, 1, 2; QK^T of tile 0
        auto v_page = [&](int t) { return pg_phys[tile_page(t)]; };
        auto prologue_tile = [&](int t, auto sl) __attribute__((always_inline)) {
            dma_k(t, kslot(sl), 0);
            dma_k(t, kslot(sl), 1);
            v_phys_next = v_page(t);
            dma_v(vslot(sl), 0);
            dma_v(vslot(sl), 1);
            stage_kpos(t, decltype(sl)::value);
        };
        prologue_tile(0, S0{});
        if (ntiles > 1) prologue_tile(1, S1{});
        if (ntiles > 2) prologue_tile(2, S2{});
        if (ntiles > 3) v_phys_next = v_page(3);
        if (ntiles > 2) wait_loads(W10{});
        else wait_loads(W0{});
        barrier_dl();
        qk(S0{}, sacc);
        if (group_b) {
            // A's X(0) needs K'(1) and V(0) of every wave
            if (ntiles > 2) wait_loads(W6{});
            else wait_loads(W0{});
            barrier_dl();
        }

        // one tile. Y(t): softmax of tile t with K'(t+3) loaded between its exponentials, positions of
        // tile t+3; X(t): PV of tile t, QK^T of tile t+1, V(t+3) loaded. `stage`: tile t+3 exists.
        auto step = [&](int t, auto sl, auto next_qk, auto stage, auto active) __attribute__((always_inline)) {
            constexpr bool STAGE = decltype(stage)::value;
            constexpr bool ACT = decltype(active)::value;
            const auto sl1 = slot_plus(sl, one{});
            const auto sl3 = slot_plus(sl, three{});
            uint16_t *kdst = kslot(sl3);
            if constexpr (ACT) {
                const bool masked = (mask_ring >> (int)sl) & 1u;
                auto kload = [&](int j) __attribute__((always_inline)) {
                    if constexpr (STAGE) dma_k(t + 3, kdst, j);
                };
                softmax(masked, (int)sl, Loads<STAGE ? 2 : 0, decltype(kload) &>{kload});
            } else if constexpr (STAGE) {
                dma_k(t + 3, kdst, 0);
                dma_k(t + 3, kdst, 1);
            }
            if constexpr (STAGE) stage_kpos(t + 3, (int)sl3);
            __builtin_amdgcn_sched_barrier(0);
            // group A's X(t) needs K'(t+1) (8 later loads may be in flight); B's X(t) follows this
            // barrier too and needs the same
            if constexpr (STAGE) wait_loads(W8{});
            else wait_loads(W0{});
            barrier_dl();
            uint16_t *vdst = vslot(sl3);
            auto vload = [&]() __attribute__((always_inline)) {
                if constexpr (STAGE) {
                    dma_v(vdst, 0);
                    dma_v(vdst, 1);
                }
            };
            if constexpr (ACT) {
                xphase(sl, sl1, next_qk, vload);
            } else {
                vload();
            }
            // the V page of the next tile this wave loads, read from LDS ahead of its use
            if constexpr (STAGE) {
                if (t + 4 < ntiles) v_phys_next = v_page(t + 4);
            }
            __builtin_amdgcn_sched_barrier(0);
            // the barrier that ends B's X(t) opens A's X(t+1), which needs K'(t+2) (6 later loads may be
            // in flight); for A this is one phase early
            if constexpr (STAGE) wait_loads(W6{});
            else wait_loads(W0{});
            barrier_dl();
        };

        int t = 0;
        const int t_main = min(n_act, ntiles - 3);
        for (; t + 4 <= t_main; t += 4) {
            step(t, S0{}, yes{}, yes{}, yes{});
            step(t + 1, S1{}, yes{}, yes{}, yes{});
            step(t + 2, S2{}, yes{}, yes{}, yes{});
            step(t + 3, S3{}, yes{}, yes{}, yes{});
        }
        if (t < t_main) step(t++, S0{}, yes{}, yes{}, yes{});
        if (t < t_main) step(t++, S1{}, yes{}, yes{}, yes{});
        if (t < t_main) step(t++, S2{}, yes{}, yes{}, yes{});
        // waves past their last key tile keep loading tiles for the others
        for (; t + 3 < ntiles; ++t) step(t, t & 3, no{}, yes{}, no{});
        if (t + 2 < ntiles) {
            if (t < n_act) step(t, t & 3, yes{}, no{}, yes{});
            else step(t, t & 3, no{}, no{}, no{});
            ++t;
        }
        if (t + 1 < ntiles) {
            if (t < n_act) step(t, t & 3, yes{}, no{}, yes{});
            else step(t, t & 3, no{}, no{}, no{});
            ++t;
        }
        if (t < ntiles) {
            if (t < n_act) step(t, t & 3, no{}, no{}, yes{});
            else step(t, t & 3, no{}, no{}, no{});
        }
        if (!group_b) barrier_dl();

        // ---- epilogue: normalise, write the output (or this split's partial result)
        {
            const int m = wave * 32 + ln;
            const int ti = m >> p.gshift;
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lrow), __float_as_uint(lrow), false, false);
            const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            const float lse_v = lt > 0.0f ? (mrow + __builtin_amdgcn_logf(lt)) * 0.6931471805599453f : -INFINITY;
            if (ti < w.n_rows) {
                const int row = w.row0 + ti;
                const int qh = w.kv_head * G + (m & (G - 1));
                if (w.partial < 0) {
                    uint16_t *orow = static_cast<uint16_t *>(p.out) + ((int64_t)row * p.hq + qh) * D;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int d0 = db * 32 + 8 * i + 4 * lg;
                            u32x2 v;
                            v[0] = pack_bf16(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv);
                            v[1] = pack_bf16(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
                            *reinterpret_cast<u32x2 *>(orow + d0) = v;
                        }
                    if (p.lse && lg == 0) p.lse[(int64_t)row * p.hq + qh] = lse_v;
                } else {
                    float *po = p.part_o + ((int64_t)w.partial * TQ + m) * D;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int d0 = db * 32 + 8 * i + 4 * lg;
                            floatx4 v = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                                         oacc[db][4 * i + 3] * inv};
                            *reinterpret_cast<floatx4 *>(po + d0) = v;
                        }
                    if (lg == 0) p.part_lse[(int64_t)w.partial * TQ + m] = lse_v;
                }
            }
        }
    }
    if (threadIdx.x == 0) release_work_queues(p);
}

// ---------------------------------------------------------------------------------------------
// fp32 attention. Work group = 4 waves of one 32-row MFMA block each (128 M-rows).
//   S^T = K' Q'^T   (v_mfma_f32_32x32x2f32; lane group lg supplies dimension 8(s/4) + 4lg + s%4
//                    at k-step s, so each lane reads 4 consecutive dimensions per 4 steps)
//   O^T += V^T P^T  (k-step s of a 32-key block pairs the key held in S^T accumulator s)
template <int D>
__global__ __launch_bounds__(kThreads, 1) void link_attention_f32(AttnParams p) {
    constexpr int KT = kKeysPerTile;
    constexpr int KS = D + 4;
    constexpr int VS = D + 4;
    constexpr int NDB = D / 32;
    constexpr int NQ = D / 8;                       // float4 groups of Q held per lane
    constexpr int NKP = KT * (D / 8) / kThreads;    // K (lo, hi) float4 pairs per thread
    constexpr int NV = KT * (D / 4) / kThreads;     // V float4 chunks per thread
    constexpr int TQ = 128;
    static_assert(NKP >= 1 && NV >= 1, "tile too small for the work group");

    __shared__ __attribute__((aligned(16))) float ks[2][KT * KS];
    __shared__ __attribute__((aligned(16))) float vs[2][KT * VS];
    __shared__ __attribute__((aligned(16))) int kpos_s[2][KT];

    const WorkDesc w = p.work[blockIdx.x];
    if (w.n_rows <= 0) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
    const int G = 1 << p.gshift;
    const int page_size = 1 << p.pshift;
    const int ppt = KT >> p.pshift;
    const PageDesc *pg = p.pages + w.page_base;
    const float *kpool = static_cast<const float *>(p.k_pool);
    const float *vpool = static_cast<const float *>(p.v_pool);
    const int64_t head_off = (int64_t)w.kv_head * page_size * D;

    // rotated Q: qf[g] = Q'[m][8g + 4lg .. +3]
    floatx4 qf[NQ];
    int rpos;
    {
        const int m = wave * 32 + ln;
        const int ti = m >> p.gshift;
        const bool valid = ti < w.n_rows;
        const int row = w.row0 + (valid ? ti : 0);
        const int qh = w.kv_head * G + (m & (G - 1));
        const int rp = valid ? p.row_pos[row] : -1;
        rpos = rp;
        const float *qrow = static_cast<const float *>(p.q) + ((int64_t)row * p.hq + qh) * D;
        const float *cs = p.rope + (int64_t)(valid ? rp : 0) * D;
#pragma unroll
        for (int g = 0; g < NQ / 2; ++g) {
            const int e0 = 8 * g + 4 * lg;
            floatx4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
            if (valid) {
                lo = *reinterpret_cast<const floatx4 *>(qrow + e0);
                hi = *reinterpret_cast<const floatx4 *>(qrow + D / 2 + e0);
            }
            const floatx4 c = *reinterpret_cast<const floatx4 *>(cs + e0);
            const floatx4 sn = *reinterpret_cast<const floatx4 *>(cs + D / 2 + e0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qf[g][j] = fmaf(lo[j], c[j], -hi[j] * sn[j]);
                qf[g + NQ / 2][j] = fmaf(hi[j], c[j], lo[j] * sn[j]);
            }
        }
    }

    // position of the wave's first row (rows of one request in increasing position; a wave
    // without rows never needs the mask)
    const int rpos0 = __builtin_amdgcn_readfirstlane(rpos);
    const int wave_rpos0 = rpos0 < 0 ? INT_MAX : rpos0;

    floatx4 k_lo[NKP], k_hi[NKP], k_c[NKP], k_s[NKP];
    uint32_t k_sgn[NKP];   // sign bit of the rotation: a negative angle flips the sines
    floatx4 v_r[NV];
    int kp_next = kNeverAttended;
    bool mask_next = true;

    auto load_tile = [&](int t) {
        const int lp0 = w.page_begin + t * ppt;
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int pi = tid + kThreads * u;
            const int key = pi / (D / 8), c = pi % (D / 8);
            const int lp = lp0 + (key >> p.pshift), slot = key & (page_size - 1);
            bool ok = false;
            int pos = 0;
            int64_t base = 0;
            if (lp < w.page_end) {
                const PageDesc pd = pg[lp];
                if (slot < pd.valid) {
                    ok = true;
                    pos = p.seg_keys ? pd.seg0 : pd.pos0 + slot;   // the rotation (negative: see below)
                    base = (int64_t)pd.phys * p.page_elems + head_off + (int64_t)slot * D;
                }
            }
            k_lo[u] = ok ? *reinterpret_cast<const floatx4 *>(kpool + base + 4 * c) : floatx4{0, 0, 0, 0};
            k_hi[u] = ok ? *reinterpret_cast<const floatx4 *>(kpool + base + D / 2 + 4 * c) : floatx4{0, 0, 0, 0};
            // a negative rotation takes the row of its magnitude with the sines negated (when the
            // rotation uses them: negated here, they would wait for their load here)
            const float *cs = p.rope + (int64_t)(pos < 0 ? -pos : pos) * D + 4 * c;
            k_c[u] = *reinterpret_cast<const floatx4 *>(cs);
            k_s[u] = *reinterpret_cast<const floatx4 *>(cs + D / 2);
            k_sgn[u] = pos < 0 ? 0x80000000u : 0u;
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int pi = tid + kThreads * u;
            const int key = pi / (D / 4), c = pi % (D / 4);
            const int lp = lp0 + (key >> p.pshift), slot = key & (page_size - 1);
            floatx4 v = {0, 0, 0, 0};
            if (lp < w.page_end) {
                const PageDesc pd = pg[lp];
                if (slot < pd.valid)
                    v = *reinterpret_cast<const floatx4 *>(vpool + (int64_t)pd.phys * p.page_elems + head_off +
                                                           (int64_t)slot * D + 4 * c);
            }
            v_r[u] = v;
        }
        {
            // every wave holds the position of key `lane` of the tile (64 keys, 64 lanes)
            const int lp = lp0 + (lane >> p.pshift), slot = lane & (page_size - 1);
            int kp = kNeverAttended;
            if (lp < w.page_end) {
                const PageDesc pd = pg[lp];
                if (slot < pd.valid) kp = pd.pos0 + slot;
            }
            kp_next = kp;
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int pi = tid + kThreads * u;
            const int key = pi / (D / 8), c = pi % (D / 8);
            floatx4 olo, ohi;
            const floatx4 sn = __builtin_bit_cast(floatx4, __builtin_bit_cast(u32x4, k_s[u]) ^ k_sgn[u]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                olo[j] = fmaf(k_lo[u][j], k_c[u][j], -k_hi[u][j] * sn[j]);
                ohi[j] = fmaf(k_hi[u][j], k_c[u][j], k_lo[u][j] * sn[j]);
            }
            *reinterpret_cast<floatx4 *>(&ks[buf][key * KS + 4 * c]) = olo;
            *reinterpret_cast<floatx4 *>(&ks[buf][key * KS + D / 2 + 4 * c]) = ohi;
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int pi = tid + kThreads * u;
            const int key = pi / (D / 4), c = pi % (D / 4);
            *reinterpret_cast<floatx4 *>(&vs[buf][key * VS + 4 * c]) = v_r[u];
        }
        if (wave == 0) kpos_s[buf][lane] = kp_next;
        // the tile needs the causal/padding mask for this wave iff some key lies after the wave's
        // first row
        mask_next = __any(kp_next > wave_rpos0);
    };

    floatx16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float mrow = kInitMax, lrow = 0.0f;

    const int ntiles = (w.page_end - w.page_begin + ppt - 1) / ppt;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const bool more = t + 1 < ntiles;
        const bool need_mask = mask_next;
        if (more) load_tile(t + 1);

        floatx16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
            for (int g = 0; g < NQ; ++g) {
                const floatx4 a = *reinterpret_cast<const floatx4 *>(&ks[buf][(kb * 32 + ln) * KS + 8 * g + 4 * lg]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], qf[g][j], sacc[kb], 0, 0, 0);
            }
        }
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const i32x4 kp4 = *reinterpret_cast<const i32x4 *>(&kpos_s[buf][kb * 32 + 8 * i + 4 * lg]);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (kp4[j] > rpos) sacc[kb][4 * i + j] = -INFINITY;
                }
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool upd = (mx - mrow) * p.scale_log2 > kRescaleLog2;
        if (__any(upd)) {
            const float mnew = upd ? mx : mrow;
            const float alpha = exp2f((mrow - mnew) * p.scale_log2);
            lrow *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            mrow = mnew;
        }
        const float msc = mrow * p.scale_log2;
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = exp2f(fmaf(sacc[kb][r], p.scale_log2, -msc));
                sacc[kb][r] = e;
                lsum += e;
            }
        lrow += lsum;

#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const int key = kb * 32 + 8 * (s >> 2) + 4 * lg + (s & 3);
                    const float a = vs[buf][key * VS + db * 32 + ln];
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[kb][s], oacc[db], 0, 0, 0);
                }

        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    {
        const int m = wave * 32 + ln;
        const int ti = m >> p.gshift;
        const float lt = lrow + __shfl_xor(lrow, 32);
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const float lse_v = lt > 0.0f ? mrow * p.scale + logf(lt) : -INFINITY;
        if (ti < w.n_rows) {
            const int row = w.row0 + ti;
            const int qh = w.kv_head * G + (m & (G - 1));
            float *dst = w.partial < 0 ? static_cast<float *>(p.out) + ((int64_t)row * p.hq + qh) * D
                                       : p.part_o + ((int64_t)w.partial * TQ + m) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int d0 = db * 32 + 8 * i + 4 * lg;
                    floatx4 v = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                                 oacc[db][4 * i + 3] * inv};
                    *reinterpret_cast<floatx4 *>(dst + d0) = v;
                }
            if (lg == 0) {
                if (w.partial < 0) {
                    if (p.lse) p.lse[(int64_t)row * p.hq + qh] = lse_v;
                } else {
                    p.part_lse[(int64_t)w.partial * TQ + m] = lse_v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Combine the splits of one (row tile, KV head): o = sum_s e^{lse_s - L} o_s / sum_s e^{lse_s - L}.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void link_merge(const MergeDesc *merge, const float *part_o,
                                                       const float *part_lse, T *out, float *lse, int hq,
                                                       int gshift, int tq) {
    // grid: (split tile, block of kThreads / (D / 4) M-rows); one thread per (M-row, 4 dims)
    constexpr int RPB = kThreads / (D / 4);
    const MergeDesc md = merge[blockIdx.x];
    const int G = 1 << gshift;
    const int mrows = md.n_rows << gshift;
    {
        const int m = blockIdx.y * RPB + (int)threadIdx.x / (D / 4), d4 = (int)threadIdx.x % (D / 4);
        if (m >= mrows) return;
        // one pass over the splits, four at a time: the loads of a group (its log-sum-exps and
        // partial outputs) are all issued before any of them is used, then folded into a running
        // maximum L, weight sum and output (rescaled when L moves)
        constexpr int R = 4;
        float L = -INFINITY, wsum = 0.0f;
        floatx4 acc = {0, 0, 0, 0};
        for (int s0 = 0; s0 < md.n_split; s0 += R) {
            float ls[R];
            floatx4 o[R];
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int s = s0 + u;
                const int64_t slot = (int64_t)(md.slot0 + min(s, md.n_split - 1)) * tq + m;
                ls[u] = s < md.n_split ? part_lse[slot] : -INFINITY;
                o[u] = *reinterpret_cast<const floatx4 *>(part_o + slot * D + 4 * d4);
            }
            float mx = L;
#pragma unroll
            for (int u = 0; u < R; ++u) mx = fmaxf(mx, ls[u]);
            if (mx == -INFINITY) continue;
            const float sc = expf(L - mx);   // 0 while L is still -inf
            acc *= sc;
            wsum *= sc;
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const float wgt = ls[u] == -INFINITY ? 0.0f : expf(ls[u] - mx);
                acc += wgt * o[u];
                wsum += wgt;
            }
            L = mx;
        }
        const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
        const int row = md.row0 + (m >> gshift);
        const int qh = md.kv_head * G + (m & (G - 1));
        T *dst = out + ((int64_t)row * hq + qh) * D + 4 * d4;
        if constexpr (sizeof(T) == 2) {
            u32x2 v;
            v[0] = pack_bf16(acc[0] * inv, acc[1] * inv);
            v[1] = pack_bf16(acc[2] * inv, acc[3] * inv);
            *reinterpret_cast<u32x2 *>(dst) = v;
        } else {
            *reinterpret_cast<floatx4 *>(dst) = acc * inv;
        }
        if (lse && d4 == 0) lse[(int64_t)row * hq + qh] = wsum > 0.0f ? L + logf(wsum) : -INFINITY;
    }
}

// ---------------------------------------------------------------------------------------------
// Page writers. One work group per (page, KV head); each thread moves 16-byte pieces.
__global__ __launch_bounds__(kThreads) void store_fill(FillPages pages, uint8_t *k_pool, uint8_t *v_pool,
                                                       const uint8_t *k, const uint8_t *v, int hkv,
                                                       int page_size, int row_bytes, int64_t page_bytes) {
    const int i = blockIdx.x, h = blockIdx.y;
    const int page = pages.ids[i];
    const int tok0 = pages.first_token + i * page_size;
    const int pieces_per_row = row_bytes / 16;
    const int64_t dst0 = (int64_t)page * page_bytes + (int64_t)h * page_size * row_bytes;
    for (int c = threadIdx.x; c < page_size * pieces_per_row; c += kThreads) {
        const int slot = c / pieces_per_row, piece = c % pieces_per_row;
        const int tok = tok0 + slot;
        u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
        if (tok < pages.n_tokens) {
            const int64_t src = ((int64_t)tok * hkv + h) * row_bytes + piece * 16;
            a = *reinterpret_cast<const u32x4 *>(k + src);
            b = *reinterpret_cast<const u32x4 *>(v + src);
        }
        const int64_t dst = dst0 + (int64_t)slot * row_bytes + piece * 16;
        *reinterpret_cast<u32x4 *>(k_pool + dst) = a;
        *reinterpret_cast<u32x4 *>(v_pool + dst) = b;
    }
}

// In a store of keys rotated at their position inside their segment (rotate_new), a new row's
// key is written in that form: rotated at slot position local0 + slot, with the table values and
// the fp32 arithmetic of the attention kernels' key rotation. Cached rows are copied as stored.
__device__ __forceinline__ void scatter_page_head(const ScatterDesc &sd, int h, uint8_t *k_pool, uint8_t *v_pool,
                                                  const uint8_t *k_new, const uint8_t *v_new, const float *rope,
                                                  int rotate_new, int elem, int hkv, int page_size, int row_bytes,
                                                  int64_t page_bytes) {
    const int pieces_per_row = row_bytes / 16;
    const int64_t head_bytes = (int64_t)h * page_size * row_bytes;
    const int64_t dst0 = (int64_t)sd.dst * page_bytes + head_bytes;
    const int n_rot = rotate_new ? sd.n_new : 0;   // new rows whose keys are written rotated below
    for (int c = threadIdx.x; c < page_size * pieces_per_row; c += kThreads) {
        const int slot = c / pieces_per_row, piece = c % pieces_per_row;
        u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
        if (slot < sd.n_new) {
            const int64_t src = ((int64_t)(sd.row0 + slot) * hkv + h) * row_bytes + piece * 16;
            a = *reinterpret_cast<const u32x4 *>(k_new + src);
            b = *reinterpret_cast<const u32x4 *>(v_new + src);
        } else if (slot < sd.n_valid) {
            const int64_t src = (int64_t)sd.src * page_bytes + head_bytes + (int64_t)slot * row_bytes + piece * 16;
            a = *reinterpret_cast<const u32x4 *>(k_pool + src);
            b = *reinterpret_cast<const u32x4 *>(v_pool + src);
        }
        const int64_t dst = dst0 + (int64_t)slot * row_bytes + piece * 16;
        if (slot >= n_rot) *reinterpret_cast<u32x4 *>(k_pool + dst) = a;
        *reinterpret_cast<u32x4 *>(v_pool + dst) = b;
    }
    if (n_rot > 0) {
        // a thread takes pieces c and c + half of one new key: the rotation pairs (i, i + d/2)
        const int half = pieces_per_row / 2, d = row_bytes / elem;
        for (int c = threadIdx.x; c < n_rot * half; c += kThreads) {
            const int slot = c / half, piece = c % half;
            const int64_t src = ((int64_t)(sd.row0 + slot) * hkv + h) * row_bytes + piece * 16;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(k_new + src);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(k_new + src + row_bytes / 2);
            const float *cs = rope + (int64_t)(sd.local0 + slot) * d;
            u32x4 olo, ohi;
            if (elem == 2) {
                const int e0 = piece * 8;
                floatx4 co[2], sn[2];
                co[0] = *reinterpret_cast<const floatx4 *>(cs + e0);
                co[1] = *reinterpret_cast<const floatx4 *>(cs + e0 + 4);
                sn[0] = *reinterpret_cast<const floatx4 *>(cs + d / 2 + e0);
                sn[1] = *reinterpret_cast<const floatx4 *>(cs + d / 2 + e0 + 4);
                rope8_bf16(lo, hi, co, sn, olo, ohi);
            } else {
                const int e0 = piece * 4;
                const floatx4 co = *reinterpret_cast<const floatx4 *>(cs + e0);
                const floatx4 sn = *reinterpret_cast<const floatx4 *>(cs + d / 2 + e0);
                const floatx4 x = __builtin_bit_cast(floatx4, lo), y = __builtin_bit_cast(floatx4, hi);
                floatx4 xr, yr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xr[j] = fmaf(x[j], co[j], -y[j] * sn[j]);
                    yr[j] = fmaf(y[j], co[j], x[j] * sn[j]);
                }
                olo = __builtin_bit_cast(u32x4, xr);
                ohi = __builtin_bit_cast(u32x4, yr);
            }
            const int64_t dst = dst0 + (int64_t)slot * row_bytes + piece * 16;
            *reinterpret_cast<u32x4 *>(k_pool + dst) = olo;
            *reinterpret_cast<u32x4 *>(k_pool + dst + row_bytes / 2) = ohi;
        }
    }
}

__global__ __launch_bounds__(kThreads) void link_scatter(const ScatterDesc *table, uint8_t *k_pool, uint8_t *v_pool,
                                                         const uint8_t *k_new, const uint8_t *v_new, const float *rope,
                                                         int rotate_new, int elem, int hkv, int page_size,
                                                         int row_bytes, int64_t page_bytes) {
    scatter_page_head(table[blockIdx.x], blockIdx.y, k_pool, v_pool, k_new, v_new, rope, rotate_new, elem, hkv,
                      page_size, row_bytes, page_bytes);
}

// The copy-on-write scatter and the key rotation of a plan in one launch (bfloat16 stores whose
// plan rotates its keys ahead of attention). Work groups [0, n_pages) rotate the keys of one
// logical page each; the rest run the scatter, one (private page, KV head) each. The two roles
// touch different memory: a private page's rotation reads the keys the scatter writes into that
// page from where the scatter takes them (the new rows, the copy-on-write source page, zeros),
// so the scatter's small, latency-bound work runs beside the rotation's streaming.
//   Rotation: the keys of a logical page turned once to the page's absolute positions, with the
// attention kernel's table values and arithmetic, into the pool's page layout indexed by logical
// page ([page][Hkv][page_size][d]); padding slots are written as zeros (the pools hold zeros
// there, which rotate to zeros). A position-free key is rotated by its position; a key stored
// rotated at its position inside its segment (SEG) by the segment's start (a new row's key
// first takes the form the scatter stores: rotated at its position inside its segment). A
// thread takes 8 (x_i, x_{i+d/2}) pairs of one slot, loads their cos/sin once, and rotates them
// in every head of its head group (heads hg, hg + n_hg, ...), loading up to HB heads' keys
// before the first store; consecutive threads take consecutive pairs of a row, so every key row
// is read and written in whole 128-byte runs.
struct PrepareParams {
    const PageDesc *pages;
    const int32_t *page_scatter;   // per logical page: its scatter entry, or -1 for a shared page
    const ScatterDesc *scatter;
    uint8_t *k_pool;
    uint8_t *v_pool;
    const uint8_t *k_new;
    const uint8_t *v_new;
    const float *rope;
    uint8_t *k_rot;
    int n_pages, hkv, pshift;
    int64_t page_bytes;
};

// Five waves per SIMD for position-free keys (84 VGPRs), as the rotation pass had on its own;
// keys rotated inside their segment need the second cos/sin row of a new key and keep four.
template <int D, bool SEG>
__global__ __launch_bounds__(kThreads, SEG ? 4 : 5) void link_prepare_bf16(PrepareParams p) {
    constexpr int PPR = D / 16;   // pieces of 8 pairs per row
    constexpr int HB = 4;         // heads loaded ahead of their stores
    const int page_size = 1 << p.pshift;
    if ((int)blockIdx.x >= p.n_pages) {
        const int b = blockIdx.x - p.n_pages;
        scatter_page_head(p.scatter[b / p.hkv], b % p.hkv, p.k_pool, p.v_pool, p.k_new, p.v_new, p.rope,
                          SEG, 2, p.hkv, page_size, D * 2, p.page_bytes);
        return;
    }
    const PageDesc pd = p.pages[blockIdx.x];
    const int si = p.page_scatter[blockIdx.x];
    const ScatterDesc sd = si >= 0 ? p.scatter[si] : ScatterDesc{pd.phys, -1, 0, 0, pd.valid, 0, 0, 0};
    const int items = page_size * PPR;                           // (slot, piece) of one head
    const int n_hg = max(1, min(p.hkv, kThreads / items));       // head groups side by side
    // the page's keys as the pool holds them once the scatter has run: a shared page's own, or a
    // private page's new rows, copy-on-write source rows and zeros
    const uint8_t *page_src = p.k_pool + (int64_t)(si >= 0 ? max(sd.src, 0) : pd.phys) * p.page_bytes;
    uint8_t *dst = p.k_rot + (int64_t)blockIdx.x * p.page_bytes;
    for (int i = threadIdx.x; i < items * n_hg; i += kThreads) {
        const int c = i % PPR, slot = (i / PPR) & (page_size - 1), hg = i / items;
        const bool valid = slot < pd.valid;
        const bool is_new = slot < sd.n_new;                      // a new row (private pages only)
        const bool from_page = !is_new && slot < sd.n_valid;      // the page's or the source page's row
        floatx4 co[2] = {}, sn[2] = {}, cl[2] = {}, sl[2] = {};
        if (valid) {
            // a negative rotation (keys compiled after leading tokens, linked before them) takes the
            // row of its magnitude with the sines negated, as the attention kernels do
            const int rot = SEG ? pd.seg0 : pd.pos0 + slot;
            const float *cs = p.rope + (int64_t)(rot < 0 ? -rot : rot) * D + 8 * c;
            co[0] = *reinterpret_cast<const floatx4 *>(cs);
            co[1] = *reinterpret_cast<const floatx4 *>(cs + 4);
            sn[0] = *reinterpret_cast<const floatx4 *>(cs + D / 2);
            sn[1] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + 4);
            if (rot < 0) {
                sn[0] = -sn[0];
                sn[1] = -sn[1];
            }
            if (SEG && is_new) {
                const float *cw = p.rope + (int64_t)(sd.local0 + slot) * D + 8 * c;
                cl[0] = *reinterpret_cast<const floatx4 *>(cw);
                cl[1] = *reinterpret_cast<const floatx4 *>(cw + 4);
                sl[0] = *reinterpret_cast<const floatx4 *>(cw + D / 2);
                sl[1] = *reinterpret_cast<const floatx4 *>(cw + D / 2 + 4);
            }
        }
        for (int h0 = hg; h0 < p.hkv; h0 += HB * n_hg) {
            u32x4 lo[HB], hi[HB];
#pragma unroll
            for (int j = 0; j < HB; ++j) {
                const int h = h0 + j * n_hg;
                lo[j] = u32x4{0, 0, 0, 0};
                hi[j] = u32x4{0, 0, 0, 0};
                if (valid && h < p.hkv) {
                    if (is_new) {
                        const int64_t off = ((int64_t)(sd.row0 + slot) * p.hkv + h) * D * 2 + c * 16;
                        lo[j] = *reinterpret_cast<const u32x4 *>(p.k_new + off);
                        hi[j] = *reinterpret_cast<const u32x4 *>(p.k_new + off + D);
                    } else if (from_page) {
                        // a buffer load over the page with the non-temporal bit: the pool's keys are
                        // read once per link call, and with the MALL evicted this pass took 57
                        // against 74 us at the 50k-token request (unchanged warm)
                        const uint32_t off = (uint32_t)(((int64_t)h * page_size + slot) * D * 2 + c * 16);
                        const __amdgpu_buffer_rsrc_t rs = page_rsrc(reinterpret_cast<const char *>(page_src),
                                                                     (uint32_t)p.page_bytes);
                        lo[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
                        hi[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + D, 0, 2));
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < HB; ++j) {
                const int h = h0 + j * n_hg;
                if (h >= p.hkv) break;
                u32x4 olo = {0, 0, 0, 0}, ohi = {0, 0, 0, 0};
                if (valid) {
                    if (SEG && is_new) {
                        u32x4 plo, phi;
                        rope8_bf16(lo[j], hi[j], cl, sl, plo, phi);
                        lo[j] = plo;
                        hi[j] = phi;
                    }
                    rope8_bf16(lo[j], hi[j], co, sn, olo, ohi);
                }
                const int64_t off = ((int64_t)h * page_size + slot) * D * 2 + c * 16;
                *reinterpret_cast<u32x4 *>(dst + off) = olo;
                *reinterpret_cast<u32x4 *>(dst + off + D) = ohi;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Decode after link (bf16). One work group (4 waves) per DecodeDesc item: the new token's G query
// heads of one KV head over a page range of its request. The G heads take the columns of the
// 32x32 MFMA blocks (lanes of rows G..31 hold zero queries), so the arithmetic is that of
// link_attention_bf16 with one 32-key block at a time:
//   S^T = K' Q'^T   (A = 32 keys loaded from the pool straight into registers and rotated there:
//                    lane pieces s and s + NS/2 hold the rotation pairs (e, e + d/2) of one key)
//   O^T += V^T P^T  (A = V^T from transposing LDS reads of the block's values, staged per wave)
// Keys come from the link call's rotated copy when it made one (read as they are), else from the
// pools, read as stored and rotated here, so that decode needs no per-request copy of shared
// pages. A key of a store of keys rotated inside their segment turns by its segment's rotation (one
// cos/sin row per page, as the rotation pass turns it). A position-free key at position t = b + o
// (b = its page's first position plus its slot rounded down to 16, o = slot mod 16) turns by
// R(b) R(o): the cos/sin of t come from rows b and o by the angle-addition formulas, so a 32-key
// block reads two rows of the table (one per 16-key group, staged through LDS) and the 16 rows of
// o sit in LDS, instead of one row per key.
// Wave w takes the item's 32-key blocks w, w+4, ... with its own online softmax (fp32, log2
// units; every key of the cache lies before the new token, so only padding is masked). The four
// waves' results are merged through LDS into the item's partial slot: the normalised output and
// its log2-sum-exp.
struct DecodeParams {
    const void *q;
    const void *k_rot;               // keys rotated ahead [logical page][Hkv][page][d], or null
    const void *k_pool;
    const void *v_pool;
    const float *rope;
    const PageDesc *pages;
    const DecodeDesc *work;
    float *part_o;
    float *part_lse;
    int hq, hkv, gshift, pshift, step;
    int64_t page_elems;
    float scale_log2;
    int max_pos;                     // rows of the RoPE table
};

constexpr int kDecRotated = 0, kDecPosition = 1, kDecSegment = 2;   // where decode's keys come from

template <int D, int KM>
__global__ __launch_bounds__(256, 2) void link_decode_bf16(DecodeParams p) {
    constexpr bool KR = KM == kDecRotated, SEG = KM == kDecSegment;
    constexpr int NS = D / 16;          // k-steps of QK^T; also 16-byte V pieces per lane
    constexpr int NDB = D / 32;
    constexpr int VS = D + 32;          // V row stride in LDS, as in link_attention_bf16
    constexpr int NW = 4;
    constexpr int MAXG = 8;
    __shared__ __attribute__((aligned(16))) uint16_t vbuf[NW * 32 * VS];
    __shared__ __attribute__((aligned(16))) int kval[NW * 32];
    __shared__ float obuf[NW * MAXG * D];
    __shared__ float mbuf[NW * MAXG], lbuf[NW * MAXG];
    __shared__ int dpg_phys[kMaxDecodePages], dpg_pv[kMaxDecodePages];
    __shared__ __attribute__((aligned(16))) float slot_cs[KM == kDecPosition ? 16 * D : 4];   // table rows 0..15
    __shared__ __attribute__((aligned(16))) float base_cs[KR ? 4 : NW * 2 * D];   // per wave: the block's 2 rows

    const DecodeDesc w = p.work[blockIdx.x];
    if (w.partial < 0) return;   // empty slot of the work list
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
    const int G = 1 << p.gshift;
    const int page_size = 1 << p.pshift;
    const int n_pages = w.page_end - w.page_begin;
    const int lpage0 = w.page_base + w.page_begin;
    const int64_t head_off = (int64_t)w.kv_head * page_size * D;   // elements
    const uint32_t page_bytes = (uint32_t)p.page_elems * 2u;
    // the range's page table, staged once: the physical page, and the first position and valid
    // count packed as pos0 << 7 | valid (positions below 2^22, valid <= 64)
    for (int i = tid; i < n_pages; i += 256) {
        const PageDesc d = p.pages[lpage0 + i];
        dpg_phys[i] = d.phys;
        dpg_pv[i] = (d.pos0 << 7) | d.valid;
    }
    if constexpr (KM == kDecPosition) {
        for (int i = tid; i < 16 * D; i += 256) slot_cs[i] = i / D < p.max_pos ? p.rope[i] : 0.0f;
    }
    __syncthreads();
    // the new token's position: keys at or after it (this step's token and later decode slots) are
    // masked; the merge adds the token itself
    const int qpos = w.pos + p.step;

    // rotated, scaled query fragments of head ln (zero beyond the G heads)
    u32x4 qf[NS];
    {
        const bool valid = ln < G;
        const uint16_t *qrow =
            static_cast<const uint16_t *>(p.q) + ((int64_t)w.request * p.hq + w.kv_head * G + (valid ? ln : 0)) * D;
        const float *cs = p.rope + (int64_t)qpos * D;
#pragma unroll
        for (int s = 0; s < NS / 2; ++s) {
            const int e0 = 16 * s + 8 * lg;
            u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
            if (valid) {
                lo = *reinterpret_cast<const u32x4 *>(qrow + e0);
                hi = *reinterpret_cast<const u32x4 *>(qrow + D / 2 + e0);
            }
            floatx4 c[2], sn[2];
            c[0] = *reinterpret_cast<const floatx4 *>(cs + e0);
            c[1] = *reinterpret_cast<const floatx4 *>(cs + e0 + 4);
            sn[0] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + e0);
            sn[1] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + e0 + 4);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                c[h] *= p.scale_log2;
                sn[h] *= p.scale_log2;
            }
            rope8_bf16(lo, hi, c, sn, qf[s], qf[s + NS / 2]);
        }
    }

    floatx16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = (floatx16)(0.0f);
    float m_run = -INFINITY, l_run = 0.0f;

    uint16_t *vb = vbuf + wave * 32 * VS;
    int *kv = kval + wave * 32;
    const char *kpool_b = static_cast<const char *>(p.k_pool);
    const char *vpool_b = static_cast<const char *>(p.v_pool);
    const char *rope_b = reinterpret_cast<const char *>(p.rope);
    const int nblk = (n_pages * page_size + 31) >> 5;
    for (int blk = wave; blk < nblk; blk += NW) {
        // the lane's key for the A operand (both lane halves hold key ln)
        const int kk = blk * 32 + ln;
        const int rel = kk >> p.pshift;
        const int slot = kk & (page_size - 1);
        const bool in_range = rel < n_pages;
        const int rc = in_range ? rel : n_pages - 1;
        const int pv = dpg_pv[rc];
        const bool filled = in_range && slot < (pv & 127);
        const bool ok = filled && (pv >> 7) + slot < qpos;
        const uint32_t kpage = KR ? (uint32_t)(lpage0 + rc) : (uint32_t)dpg_phys[rc];
        const char *krow = (KR ? static_cast<const char *>(p.k_rot) : kpool_b) + (uint64_t)kpage * page_bytes +
                           (uint32_t)(head_off + slot * D) * 2u;
        // the cos/sin row of each 16-key group of the block (padding slots hold zeros, which rotate
        // to zeros with any row): its segment's rotation (negative: the row of its magnitude, sines
        // negated), or b, the position of the group's first slot; row o = slot mod 16 of a key's
        // position comes from slot_cs. One 16-byte piece per lane, through LDS.
        constexpr int LPR = D / 4;   // lanes per row
        u32x4 brow_piece = {0u, 0u, 0u, 0u};
        const int bg = lane / LPR;
        if (!KR && bg < 2) {
            const int gk = blk * 32 + 16 * bg;
            const int grc = min(gk >> p.pshift, n_pages - 1);
            int row;
            uint32_t neg = 0u;
            if constexpr (SEG) {
                const int r = p.pages[lpage0 + grc].seg0;
                row = r < 0 ? -r : r;
                neg = r < 0 && (lane % LPR) >= LPR / 2 ? 0x80000000u : 0u;   // the sine half
            } else {
                row = min((dpg_pv[grc] >> 7) + (gk & (page_size - 1)), p.max_pos - 1);
            }
            brow_piece = *reinterpret_cast<const u32x4 *>(rope_b + (uint64_t)(uint32_t)row * (uint32_t)(D * 4) +
                                                          (lane % LPR) * 16);
#pragma unroll
            for (int u = 0; u < 4; ++u) brow_piece[u] ^= neg;
        }
        // K: NS 16-byte pieces of the A operand. V: NS loads, each a contiguous run of RPI rows of
        // the block (a page holds whole runs: RPI <= 8 <= page size), lane = (row, 16-byte chunk)
        constexpr int RPI = 512 / D, CPR = D / 8;
        u32x4 kr[NS];
        u32x4 vr[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) kr[s] = *reinterpret_cast<const u32x4 *>(krow + (16 * s + 8 * lg) * 2);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int vk = blk * 32 + i * RPI + lane / CPR;
            const int vrel = min(vk >> p.pshift, n_pages - 1);
            const char *vrow = vpool_b + (uint64_t)(uint32_t)dpg_phys[vrel] * page_bytes +
                               (uint32_t)(head_off + (vk & (page_size - 1)) * D) * 2u;
            vr[i] = *reinterpret_cast<const u32x4 *>(vrow + (lane % CPR) * 16);
        }
        // the previous block's reads of this wave's LDS buffers are complete
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        float *bcs = base_cs + wave * 2 * D;
        if (!KR && bg < 2) *reinterpret_cast<u32x4 *>(&bcs[bg * D + (lane % LPR) * 4]) = brow_piece;
#pragma unroll
        for (int i = 0; i < NS; ++i) *reinterpret_cast<u32x4 *>(&vb[(i * RPI + lane / CPR) * VS + (lane % CPR) * 8]) = vr[i];
        if (lg == 0) kv[ln] = ok ? 1 : 0;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const float *cs_row = bcs + (ln >> 4) * D;   // the lane's key's group
        const int orow = ln & 15;                    // its slot mod 16
        bf16x8 ka[NS];
#pragma unroll
        for (int s = 0; s < NS / 2 && KR; ++s) {
            ka[s] = __builtin_bit_cast(bf16x8, kr[s]);
            ka[s + NS / 2] = __builtin_bit_cast(bf16x8, kr[s + NS / 2]);
        }
#pragma unroll
        for (int s = 0; s < NS / 2 && !KR; ++s) {
            const int e0 = 16 * s + 8 * lg;
            floatx4 c[2], sn[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                c[h] = *reinterpret_cast<const floatx4 *>(&cs_row[e0 + 4 * h]);
                sn[h] = *reinterpret_cast<const floatx4 *>(&cs_row[D / 2 + e0 + 4 * h]);
            }
            if constexpr (KM == kDecPosition) {
                // cos/sin(b + o) from the rows of b and of o
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const floatx4 c2 = *reinterpret_cast<const floatx4 *>(&slot_cs[orow * D + e0 + 4 * h]);
                    const floatx4 s2 = *reinterpret_cast<const floatx4 *>(&slot_cs[orow * D + D / 2 + e0 + 4 * h]);
                    floatx4 cc, ss;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        cc[u] = fmaf(c[h][u], c2[u], -(sn[h][u] * s2[u]));
                        ss[u] = fmaf(sn[h][u], c2[u], c[h][u] * s2[u]);
                    }
                    c[h] = cc;
                    sn[h] = ss;
                }
            }
            u32x4 lo, hi;
            rope8_bf16(kr[s], kr[s + NS / 2], c, sn, lo, hi);
            ka[s] = __builtin_bit_cast(bf16x8, lo);
            ka[s + NS / 2] = __builtin_bit_cast(bf16x8, hi);
            // one step's cos/sin live at a time
            __builtin_amdgcn_sched_barrier(0);
        }
        floatx16 sacc = (floatx16)(0.0f);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], __builtin_bit_cast(bf16x8, qf[s]), sacc, 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        // S^T lane layout: column ln (head), rows 8 (r / 4) + 4 lg + r % 4 (keys of the block)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const i32x4 k4 = *reinterpret_cast<const i32x4 *>(&kv[8 * i + 4 * lg]);
#pragma unroll
            for (int j = 0; j < 4; ++j) sacc[4 * i + j] = k4[j] ? sacc[4 * i + j] : -INFINITY;
        }
        float mx = sacc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float m_new = fmaxf(m_run, mx);
        const float base = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - base);
        float e[16];
        float lsum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            e[r] = __builtin_amdgcn_exp2f(sacc[r] - base);
            lsum += e[r];
        }
        const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        lsum = __uint_as_float(sl[0]) + __uint_as_float(sl[1]);
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        u32x4 pf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int u = 0; u < 4; ++u) pf[s2][u] = pack_bf16(e[8 * s2 + 2 * u], e[8 * s2 + 2 * u + 1]);
        // O^T += V^T P^T over the block's 32 keys (two k-steps of 16)
        typedef short v4s __attribute__((ext_vector_type(4)));
        const int gi = lane >> 4, jj = (lane >> 2) & 3, qq = lane & 3;
        const uint16_t *vt = vb + (4 * lg + jj) * VS + 16 * (gi & 1) + 4 * qq;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            oacc[db] *= alpha;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint16_t *a = vt + (16 * s2) * VS + db * 32;
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)a);
                const v4s hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(a + 8 * VS));
                const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, pf[s2]), oacc[db], 0,
                                                                   0, 0);
            }
        }
    }

    // the four waves' (m, l, O) of every head, merged through LDS
    if (ln < G) {
        if (lg == 0) {
            mbuf[wave * MAXG + ln] = m_run;
            lbuf[wave * MAXG + ln] = l_run;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) obuf[(wave * MAXG + ln) * D + db * 32 + 8 * i + 4 * lg + j] = oacc[db][4 * i + j];
    }
    __syncthreads();
    for (int t = tid; t < G * D; t += 256) {
        const int h = t / D, d = t % D;
        float m = -INFINITY;
#pragma unroll
        for (int v = 0; v < NW; ++v) m = fmaxf(m, mbuf[v * MAXG + h]);
        float l = 0.0f, o = 0.0f;
        if (m != -INFINITY) {
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float f = __builtin_amdgcn_exp2f(mbuf[v * MAXG + h] - m);
                l += lbuf[v * MAXG + h] * f;
                o += obuf[(v * MAXG + h) * D + d] * f;
            }
        }
        const bool any = l > 0.0f;
        p.part_o[((int64_t)w.partial * G + h) * D + d] = any ? o / l : 0.0f;
        if (d == 0) p.part_lse[(int64_t)w.partial * G + h] = any ? m + __builtin_amdgcn_logf(l) : -INFINITY;
    }
}

// Decode merge: one work group per (request, query head). The new token's own score (its rotated
// query against its rotated key, both rounded to bf16 as the attention kernels round them) joins
// the partial results of the request's page ranges; the output is their log-sum-exp weighted
// mean. Thread (g, d) folds ranges g, g + NG, ... of output dimension d into a running
// (maximum, weight sum, weighted sum), loading R ranges at a time before using them, so the merge
// waits for memory about once; one LDS round then combines the NG groups with the token's score.
struct DecodeMergeParams {
    const void *q, *k, *v;
    const float *rope;
    const DecodeMergeDesc *merge;
    const PageDesc *pages;
    const float *part_o;
    const float *part_lse;
    void *out;
    float *lse;
    void *k_pool, *v_pool, *k_rot;   // the token's decode slot is written here (k_rot: when present)
    int hq, hkv, gshift, pshift, step;
    int64_t page_elems;
    float scale_log2;
    int seg_keys;                    // the pool holds keys rotated at their position in their segment
};

template <int D>
__global__ __launch_bounds__(512) void link_decode_merge(DecodeMergeParams p) {
    constexpr int NT = 512, NG = NT / D;
    constexpr int R = 8;                // ranges a thread loads before folding them in
    __shared__ float part_m[NG * D], part_l[NG * D], part_s[NG * D];
    __shared__ float s_new_sh;
    const int G = 1 << p.gshift;
    const DecodeMergeDesc md = p.merge[blockIdx.x >> p.gshift];
    const int hl = blockIdx.x & (G - 1), h = md.kv_head * G + hl;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = tid % D, grp = tid / D;
    const DecodeReq dr = md.req;
    const int pos = dr.pos + p.step;
    // the token's rows, loaded ahead of the ranges (wave 0 forms its score from them)
    const int i = lane & (D / 2 - 1);   // rotation pair (i, i + D/2); lanes past D/2 repeat it
    const uint16_t *qr = static_cast<const uint16_t *>(p.q) + ((int64_t)md.request * p.hq + h) * D;
    const uint16_t *kr = static_cast<const uint16_t *>(p.k) + ((int64_t)md.request * p.hkv + md.kv_head) * D;
    const uint16_t *vr = static_cast<const uint16_t *>(p.v) + ((int64_t)md.request * p.hkv + md.kv_head) * D;
    float c = 0.0f, sn = 0.0f, qx = 0.0f, qy = 0.0f, kx = 0.0f, ky = 0.0f;
    if (wave == 0) {
        c = p.rope[(int64_t)pos * D + i];
        sn = p.rope[(int64_t)pos * D + D / 2 + i];
        qx = bf_lo(qr[i]);
        qy = bf_lo(qr[i + D / 2]);
        kx = bf_lo(kr[i]);
        ky = bf_lo(kr[i + D / 2]);
    }

    const float *lse_r = p.part_lse + (int64_t)md.slot0 * G + hl;              // range j at lse_r[j * G]
    const float *po = p.part_o + ((int64_t)md.slot0 * G + hl) * D + d;         // range j at po[j * G * D]
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    for (int j0 = grp; j0 < md.n_split; j0 += NG * R) {
        float lv[R], ov[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int j = j0 + u * NG;
            const bool in = j < md.n_split;
            lv[u] = in ? lse_r[(int64_t)j * G] : -INFINITY;
            ov[u] = in ? po[(int64_t)j * G * D] : 0.0f;
        }
        float mx = m;
#pragma unroll
        for (int u = 0; u < R; ++u) mx = fmaxf(mx, lv[u]);
        if (mx != -INFINITY) {
            const float sc = __builtin_amdgcn_exp2f(m - mx);   // 0 while m is -inf
            l *= sc;
            o *= sc;
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const float f = __builtin_amdgcn_exp2f(lv[u] - mx);
                l += f;
                o += f * ov[u];
            }
            m = mx;
        }
    }
    part_m[grp * D + d] = m;
    part_l[grp * D + d] = l;
    part_s[grp * D + d] = o;
    if (wave == 0) {
        const float cq = c * p.scale_log2, sq = sn * p.scale_log2;
        const uint32_t qp = pack_bf16(fmaf(qx, cq, -qy * sq), fmaf(qy, cq, qx * sq));
        const uint32_t kp = pack_bf16(fmaf(kx, c, -ky * sn), fmaf(ky, c, kx * sn));
        float dot = lane < D / 2 ? bf_lo(qp) * bf_lo(kp) + bf_hi(qp) * bf_hi(kp) : 0.0f;
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) dot += __shfl_xor(dot, o2);
        if (lane == 0) s_new_sh = dot;   // log2 units
        // the first query head of the KV head writes the token into its decode slot, for the
        // later steps: its key (in the pool's key form) and value into the pools, and its rotated
        // key into the rotated copy when decode reads keys from there
        if (hl == 0 && lane < D / 2) {
            const int page_size = 1 << p.pshift;
            const int lp = dr.lpage0 + ((dr.off + p.step) >> p.pshift);
            const int slot = (dr.off + p.step) & (page_size - 1);
            const int64_t row = (int64_t)(md.kv_head * page_size + slot) * D;
            const int64_t phys_row = (int64_t)p.pages[lp].phys * p.page_elems + row;
            uint16_t *kp_ = static_cast<uint16_t *>(p.k_pool), *vp_ = static_cast<uint16_t *>(p.v_pool);
            uint32_t krot = kp;   // the rotated copy's form: as the link call rotates the pool's key
            if (p.seg_keys) {
                // the pool's form: rotated at the token's position inside its segment; the copy
                // turns that by the segment's rotation (negative: the row of its magnitude, sines
                // negated), as the link call turns every stored key
                const float *cl = p.rope + (int64_t)(pos - dr.seg0) * D;
                const float c2 = cl[i], s2 = cl[D / 2 + i];
                const uint32_t kl = pack_bf16(fmaf(kx, c2, -ky * s2), fmaf(ky, c2, kx * s2));
                kp_[phys_row + i] = (uint16_t)(kl & 0xffffu);
                kp_[phys_row + i + D / 2] = (uint16_t)(kl >> 16);
                const int r = dr.seg0;
                const float *cr = p.rope + (int64_t)(r < 0 ? -r : r) * D;
                const float c3 = cr[i], s3 = r < 0 ? -cr[D / 2 + i] : cr[D / 2 + i];
                const float lx = bf_lo(kl), ly = bf_hi(kl);
                krot = pack_bf16(fmaf(lx, c3, -ly * s3), fmaf(ly, c3, lx * s3));
            } else {
                kp_[phys_row + i] = kr[i];
                kp_[phys_row + i + D / 2] = kr[i + D / 2];
            }
            vp_[phys_row + i] = vr[i];
            vp_[phys_row + i + D / 2] = vr[i + D / 2];
            if (p.k_rot) {
                uint16_t *kr_ = static_cast<uint16_t *>(p.k_rot);
                const int64_t rot_row = (int64_t)lp * p.page_elems + row;
                kr_[rot_row + i] = (uint16_t)(krot & 0xffffu);
                kr_[rot_row + i + D / 2] = (uint16_t)(krot >> 16);
            }
        }
    }
    __syncthreads();
    if (tid < D) {
        const float s_new = s_new_sh;
        float mm = s_new;
#pragma unroll
        for (int g = 0; g < NG; ++g) mm = fmaxf(mm, part_m[g * D + tid]);
        const float f_new = __builtin_amdgcn_exp2f(s_new - mm);
        float den = f_new, osum = f_new * bf_lo(vr[tid]);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float f = __builtin_amdgcn_exp2f(part_m[g * D + tid] - mm);   // 0 for a group without ranges
            den += part_l[g * D + tid] * f;
            osum += part_s[g * D + tid] * f;
        }
        uint16_t *orow = static_cast<uint16_t *>(p.out) + ((int64_t)md.request * p.hq + h) * D;
        orow[tid] = (uint16_t)(pack_bf16(osum / den, 0.0f) & 0xffffu);
        if (tid == 0 && p.lse)
            p.lse[(int64_t)md.request * p.hq + h] = (mm + __builtin_amdgcn_logf(den)) * 0.6931471805599453f;
    }
}

int log2_exact(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

}  // namespace

hipError_t launch_store_fill(const LayerShape &s, void *k_pool, void *v_pool, const void *k, const void *v,
                             const FillPages &pages, hipStream_t stream) {
    if (pages.count <= 0) return hipSuccess;
    const int elem = s.dtype == 0 ? 2 : 4;
    dim3 grid(pages.count, s.hkv);
    hipLaunchKernelGGL(store_fill, grid, dim3(kThreads), 0, stream, pages, static_cast<uint8_t *>(k_pool),
                       static_cast<uint8_t *>(v_pool), static_cast<const uint8_t *>(k),
                       static_cast<const uint8_t *>(v), s.hkv, s.page_size, s.d * elem, s.page_elems * elem);
    return hipGetLastError();
}

hipError_t launch_scatter(const LayerShape &s, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                          const float *rope, const ScatterDesc *table, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int elem = s.dtype == 0 ? 2 : 4;
    dim3 grid(n, s.hkv);
    hipLaunchKernelGGL(link_scatter, grid, dim3(kThreads), 0, stream, table, static_cast<uint8_t *>(k_pool),
                       static_cast<uint8_t *>(v_pool), static_cast<const uint8_t *>(k_new),
                       static_cast<const uint8_t *>(v_new), rope, s.key_layout, elem, s.hkv, s.page_size, s.d * elem,
                       s.page_elems * elem);
    return hipGetLastError();
}

hipError_t launch_prepare(const LayerShape &s, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                          const float *rope, const PageDesc *pages, const int32_t *page_scatter, int n_pages,
                          const ScatterDesc *table, int n_scatter, void *k_rot, hipStream_t stream) {
    if (s.dtype != 0) return hipErrorInvalidValue;
    const int n_groups = n_pages + n_scatter * s.hkv;
    if (n_groups <= 0) return hipSuccess;
    PrepareParams p;
    p.pages = pages;
    p.page_scatter = page_scatter;
    p.scatter = table;
    p.k_pool = static_cast<uint8_t *>(k_pool);
    p.v_pool = static_cast<uint8_t *>(v_pool);
    p.k_new = static_cast<const uint8_t *>(k_new);
    p.v_new = static_cast<const uint8_t *>(v_new);
    p.rope = rope;
    p.k_rot = static_cast<uint8_t *>(k_rot);
    p.n_pages = n_pages;
    p.hkv = s.hkv;
    p.pshift = log2_exact(s.page_size);
    p.page_bytes = s.page_elems * 2;
    const dim3 grid(n_groups);
    if (s.key_layout) {
        if (s.d == 128) hipLaunchKernelGGL((link_prepare_bf16<128, true>), grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((link_prepare_bf16<64, true>), grid, dim3(kThreads), 0, stream, p);
    } else {
        if (s.d == 128) hipLaunchKernelGGL((link_prepare_bf16<128, false>), grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((link_prepare_bf16<64, false>), grid, dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_attention(const LayerShape &s, const void *q, const void *k_pool, const void *v_pool,
                            const float *rope, const AttnTables &t, void *out, float *lse, hipStream_t stream) {
    if (t.n_work <= 0) return hipSuccess;
    if (t.k_rot && s.dtype != 0) return hipErrorInvalidValue;
    AttnParams p;
    p.q = q;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.rope = rope;
    p.k_rot = t.k_rot;
    p.pages = t.pages;
    p.row_pos = t.row_pos;
    p.work = t.work;
    p.ticket = t.ticket;
    p.n_work = t.n_work;
    p.n_queues = t.n_queues;
    p.persistent = t.n_groups < t.n_work;
    p.out = out;
    p.lse = lse;
    p.part_o = t.part_o;
    p.part_lse = t.part_lse;
    p.hq = s.hq;
    p.hkv = s.hkv;
    p.gshift = log2_exact(s.hq / s.hkv);
    p.pshift = log2_exact(s.page_size);
    p.page_elems = s.page_elems;
    p.scale = 1.0f / sqrtf((float)s.d);
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)s.d);
    p.seg_keys = s.key_layout;
    dim3 grid(t.n_work);
    const dim3 groups(t.n_groups);   // the bf16 kernels: persistent when there are fewer groups than items
    if (s.dtype == 0) {
        if (t.k_rot) {
            if (s.d == 128) hipLaunchKernelGGL(link_attention_bf16_dl<128>, groups, dim3(512), 0, stream, p);
            else hipLaunchKernelGGL((link_attention_bf16<64, true, false>), groups, dim3(512), 0, stream, p);
        } else if (s.key_layout) {
            if (s.d == 128) hipLaunchKernelGGL((link_attention_bf16<128, false, true>), groups, dim3(512), 0, stream, p);
            else hipLaunchKernelGGL((link_attention_bf16<64, false, true>), groups, dim3(512), 0, stream, p);
        } else {
            if (s.d == 128) hipLaunchKernelGGL((link_attention_bf16<128, false, false>), groups, dim3(512), 0, stream, p);
            else hipLaunchKernelGGL((link_attention_bf16<64, false, false>), groups, dim3(512), 0, stream, p);
        }
    } else {
        if (s.d == 128) hipLaunchKernelGGL(link_attention_f32<128>, grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL(link_attention_f32<64>, grid, dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const LayerShape &s, const void *q, const void *k, const void *v, void *k_pool, void *v_pool,
                         const float *rope, const DecodeTables &t, void *out, float *lse, hipStream_t stream) {
    if (s.dtype != 0) return hipErrorInvalidValue;
    const int gshift = log2_exact(s.hq / s.hkv);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)s.d);
    if (t.n_work > 0) {
        DecodeParams p;
        p.q = q;
        p.k_rot = t.k_rot;
        p.k_pool = k_pool;
        p.v_pool = v_pool;
        p.rope = rope;
        p.pages = t.pages;
        p.step = t.step;
        p.work = t.work;
        p.part_o = t.part_o;
        p.part_lse = t.part_lse;
        p.hq = s.hq;
        p.hkv = s.hkv;
        p.gshift = gshift;
        p.pshift = log2_exact(s.page_size);
        p.page_elems = s.page_elems;
        p.scale_log2 = scale_log2;
        p.max_pos = t.max_pos;
        const dim3 grid(t.n_work);
        if (t.k_rot) {
            if (s.d == 128) hipLaunchKernelGGL((link_decode_bf16<128, kDecRotated>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((link_decode_bf16<64, kDecRotated>), grid, dim3(256), 0, stream, p);
        } else if (s.key_layout) {
            if (s.d == 128) hipLaunchKernelGGL((link_decode_bf16<128, kDecSegment>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((link_decode_bf16<64, kDecSegment>), grid, dim3(256), 0, stream, p);
        } else {
            if (s.d == 128) hipLaunchKernelGGL((link_decode_bf16<128, kDecPosition>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((link_decode_bf16<64, kDecPosition>), grid, dim3(256), 0, stream, p);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (t.n_merge <= 0) return hipSuccess;
    DecodeMergeParams m;
    m.q = q;
    m.k = k;
    m.v = v;
    m.rope = rope;
    m.merge = t.merge;
    m.pages = t.pages;
    m.k_pool = k_pool;
    m.v_pool = v_pool;
    m.k_rot = t.k_rot;
    m.pshift = log2_exact(s.page_size);
    m.step = t.step;
    m.page_elems = s.page_elems;
    m.part_o = t.part_o;
    m.part_lse = t.part_lse;
    m.out = out;
    m.lse = lse;
    m.hq = s.hq;
    m.hkv = s.hkv;
    m.gshift = gshift;
    m.scale_log2 = scale_log2;
    m.seg_keys = s.key_layout;
    const dim3 grid(t.n_merge << gshift);
    if (s.d == 128) hipLaunchKernelGGL(link_decode_merge<128>, grid, dim3(512), 0, stream, m);
    else hipLaunchKernelGGL(link_decode_merge<64>, grid, dim3(512), 0, stream, m);
    return hipGetLastError();
}

// Device scratch of the allocation-free link call (pic_link_attend_static): the plan tables, split
// partials and rotated keys of one call. Each GPU the library runs on holds its own copy, at its own
// address, until the process ends. In host code `scratch` names a host-side stand-in: its device
// address comes from hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex lock;
    static void *address[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> hold(lock);
    if (!address[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        address[dev] = p;
    }
    *ptr = address[dev];
    return hipSuccess;
}

hipError_t launch_merge(const LayerShape &s, const AttnTables &t, void *out, float *lse, hipStream_t stream) {
    if (t.n_merge <= 0) return hipSuccess;
    const int gshift = log2_exact(s.hq / s.hkv);
    const int tq = tile_qrows(s.dtype);
    dim3 grid(t.n_merge, tq / (kThreads / (s.d / 4)));
    if (s.dtype == 0) {
        typedef uint16_t T;
        if (s.d == 128)
            hipLaunchKernelGGL((link_merge<T, 128>), grid, dim3(kThreads), 0, stream, t.merge, t.part_o, t.part_lse,
                               static_cast<T *>(out), lse, s.hq, gshift, tq);
        else
            hipLaunchKernelGGL((link_merge<T, 64>), grid, dim3(kThreads), 0, stream, t.merge, t.part_o, t.part_lse,
                               static_cast<T *>(out), lse, s.hq, gshift, tq);
    } else {
        if (s.d == 128)
            hipLaunchKernelGGL((link_merge<float, 128>), grid, dim3(kThreads), 0, stream, t.merge, t.part_o,
                               t.part_lse, static_cast<float *>(out), lse, s.hq, gshift, tq);
        else
            hipLaunchKernelGGL((link_merge<float, 64>), grid, dim3(kThreads), 0, stream, t.merge, t.part_o,
                               t.part_lse, static_cast<float *>(out), lse, s.hq, gshift, tq);
    }
    return hipGetLastError();
}

}  // namespace piclink
