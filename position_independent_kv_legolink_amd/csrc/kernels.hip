// HIP kernels of the link step for gfx950 (CDNA4).
//
//   store_fill     chunk K/V [n][Hkv][d] -> page-aligned pool pages (compile-step product in)
//   link_scatter   recomputed rows' K/V -> request-private pages, copy-on-write of cached rows
//   link_attention causal attention of the selected rows over their request's linked pages,
//                  RoPE applied in registers at each token's absolute position, grouped-query
//                  rows of one KV head per work group, MFMA for QK^T and PV, online softmax
//   link_merge     log-sum-exp combination of split KV ranges
//
// Method: EPIC (atlas.scime.ai summary, "Approach": chunks compiled from position 0, the first
// k tokens of every chunk recomputed at link time) and MEPIC (searcharxiv.org abstract:
// page-aligned position-free chunk KV, RoPE fused in the attention kernel, first block
// request-specific, other blocks shared).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

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

// Scores are kept in raw q.k units; the running maximum is only moved when a
// row's maximum grows by more than 2^kRescaleLog2 in softmax units, so the
// accumulator is rescaled rarely. Exact for any stale maximum: exponentials
// stay <= 2^kRescaleLog2.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kInitMax = -1.0e30f;
constexpr int kNeverAttended = INT_MAX;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    floatx2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
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
    const PageDesc *pages;
    const int32_t *row_pos;
    const WorkDesc *work;
    void *out;
    float *lse;
    float *part_o;
    float *part_lse;
    int hq, hkv, gshift, pshift;
    int64_t page_elems;
    float scale_log2;           // log2(e) / sqrt(d)
    float scale;                // 1 / sqrt(d)
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
//   Y(t): softmax of tile t, RoPE + LDS staging of tile t+2, global loads of tile t+3  (VALU)
//   X(t): PV of tile t, QK^T of tile t+1                                             (MFMA)
// with a work-group barrier after each phase; group B passes one extra barrier at the start
// (and group A one at the end), so B's phase k overlaps A's phase k+1. Tile buffers are deep
// enough for the one-phase skew: K' and key positions x3, V x4.
template <int D>
__global__ __launch_bounds__(512, 1) void link_attention_bf16(AttnParams p) {
    constexpr int NT = 512;
    constexpr int KT = kKeysPerTile;
    constexpr int KS = D + 8;          // K' row stride in LDS (bf16): conflict-free A-fragment reads
    constexpr int VS = D + 16;         // V row stride in LDS (bf16): conflict-free transposing reads
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
    __shared__ int pg_phys[kMaxItemPages], pg_pos0[kMaxItemPages], pg_valid[kMaxItemPages];

    const WorkDesc w = p.work[blockIdx.x];
    if (w.n_rows <= 0) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
    const int G = 1 << p.gshift;
    const int page_size = 1 << p.pshift;
    const int ppt = KT >> p.pshift;
    const PageDesc *pg = p.pages + w.page_base;
    const uint16_t *kpool = static_cast<const uint16_t *>(p.k_pool);
    const uint16_t *vpool = static_cast<const uint16_t *>(p.v_pool);
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
            rope8_bf16(lo, hi, c, sn, qf[s], qf[s + NS / 2]);
        }
    }

    // ---- staging registers of one key tile (global -> registers -> LDS)
    u32x4 k_lo[NKP], k_hi[NKP];
    int k_pos[NKP];
    floatx4 k_c[NKP][2], k_s[NKP][2];
    u32x4 v_r[NVC];
    int kp_stage = kNeverAttended;
    unsigned mask_ring = 7u;           // bit (t % 3): tile t needs the causal/padding mask

    // The work item's page table is staged in LDS once. The descriptors of a tile's KT / page
    // pages are read from LDS at the start of the VALU phase (their latency hides behind the
    // softmax) and moved to SGPRs where the global loads use them. Keys of one wave's K pieces
    // (and of each of its V pieces) lie in one page (page >= 16 tokens): each piece picks its page
    // with a scalar select. Keys past the work item's range or in page padding read real, finite
    // pool data (the last page, or the zeroed padding slots) and are removed by the mask
    // (position kNeverAttended).
    const int n_pages = w.page_end - w.page_begin;
    for (int i = tid; i < n_pages; i += NT) {
        const PageDesc d = pg[w.page_begin + i];
        pg_phys[i] = d.phys;
        pg_pos0[i] = d.pos0;
        pg_valid[i] = d.valid;
    }
    lds_barrier();
    // descriptor values read ahead from LDS: the wave's K page and V pages (uniform) and the
    // page of key `lane` (for the mask positions)
    int rk_phys[NKP], rk_pos0[NKP], rk_valid[NKP], rv_phys[NVC], rl_pos0, rl_valid;
    auto load_desc = [&](int t) {
        const int r0 = t * ppt;
        const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int rq = r0 + (((NT * u + 64 * wv) / (D / 16)) >> p.pshift);
            const int r = min(rq, n_pages - 1);
            rk_phys[u] = pg_phys[r];
            rk_pos0[u] = pg_pos0[r];
            rk_valid[u] = rq < n_pages ? pg_valid[r] : 0;
        }
#pragma unroll
        for (int u = 0; u < NVC; ++u)
            rv_phys[u] = pg_phys[min(r0 + (((NT * u + 64 * wv) / (D / 8)) >> p.pshift), n_pages - 1)];
        const int rq = r0 + (lane >> p.pshift);
        const int r = min(rq, n_pages - 1);
        rl_pos0 = pg_pos0[r];
        rl_valid = rq < n_pages ? pg_valid[r] : 0;
    };
    auto load_tile = [&]() {
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int pi = tid + NT * u;
            const int key = pi / (D / 16), c = pi % (D / 16);
            const int phys = __builtin_amdgcn_readfirstlane(rk_phys[u]);
            const int pos0 = __builtin_amdgcn_readfirstlane(rk_pos0[u]);
            const int valid = __builtin_amdgcn_readfirstlane(rk_valid[u]);
            const int slot = key & (page_size - 1);
            const bool ok = (KPAIRS % NT == 0 || pi < KPAIRS) && slot < valid;
            const int64_t base = (int64_t)phys * p.page_elems + head_off + (int64_t)slot * D;
            k_lo[u] = *reinterpret_cast<const u32x4 *>(kpool + base + 8 * c);
            k_hi[u] = *reinterpret_cast<const u32x4 *>(kpool + base + D / 2 + 8 * c);
            k_pos[u] = ok ? pos0 + slot : pos0;
        }
#pragma unroll
        for (int u = 0; u < NVC; ++u) {
            const int pi = tid + NT * u;
            const int key = pi / (D / 8), c16 = pi % (D / 8);
            const int slot = key & (page_size - 1);
            const int64_t base =
                (int64_t)__builtin_amdgcn_readfirstlane(rv_phys[u]) * p.page_elems + head_off + (int64_t)slot * D;
            v_r[u] = *reinterpret_cast<const u32x4 *>(vpool + base + 8 * c16);
        }
        const int slot = lane & (page_size - 1);
        kp_stage = slot < rl_valid ? rl_pos0 + slot : kNeverAttended;
    };

    // cos/sin of the staged keys; issued ahead of the MFMAs that hide their latency
    auto load_rope = [&]() {
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int pi = tid + NT * u;
            const int c = pi % (D / 16);
            const float *cs = p.rope + (int64_t)k_pos[u] * D + 8 * c;
            k_c[u][0] = *reinterpret_cast<const floatx4 *>(cs);
            k_c[u][1] = *reinterpret_cast<const floatx4 *>(cs + 4);
            k_s[u][0] = *reinterpret_cast<const floatx4 *>(cs + D / 2);
            k_s[u][1] = *reinterpret_cast<const floatx4 *>(cs + D / 2 + 4);
        }
    };

    // slots: K' and key positions in ring slot ksl (of 3), V in slot vsl (of 4)
    auto store_tile = [&](int ksl, int vsl, int t) {
        uint16_t *kb = ks + ksl * KBUF;
        uint16_t *vb = vs + vsl * VBUF;
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int pi = tid + NT * u;
            if (KPAIRS % NT != 0 && pi >= KPAIRS) break;
            const int key = pi / (D / 16), c = pi % (D / 16);
            u32x4 olo, ohi;
            rope8_bf16(k_lo[u], k_hi[u], k_c[u], k_s[u], olo, ohi);
            *reinterpret_cast<u32x4 *>(&kb[key * KS + 8 * c]) = olo;
            *reinterpret_cast<u32x4 *>(&kb[key * KS + D / 2 + 8 * c]) = ohi;
        }
#pragma unroll
        for (int u = 0; u < NVC; ++u) {
            const int pi = tid + NT * u;
            if (VCHUNKS % NT != 0 && pi >= VCHUNKS) break;
            const int key = pi / (D / 8), c16 = pi % (D / 8);
            *reinterpret_cast<u32x4 *>(&vb[key * VS + 8 * c16]) = v_r[u];
        }
        kpos_s[ksl * KT + lane] = kp_stage;   // every wave writes the same 64 values
        const unsigned bit = 1u << ksl;
        mask_ring = __any(kp_stage > w.rpos_min) ? (mask_ring | bit) : (mask_ring & ~bit);
    };

    // S^T of one tile: two 32-key blocks, NS k-steps each
    auto qk = [&](int ksl, floatx16 (&sacc)[2]) {
        const uint16_t *kb = ks + ksl * KBUF;
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
    float mrow = kInitMax, lrow = 0.0f;

    // online softmax, part 1: row maximum over the tile and the running maximum (moved only when
    // it grows by more than 2^kRescaleLog2); returns the factor that rescales the running sums
    auto softmax_max = [&](floatx16 (&sacc)[2]) -> float {
        float mx = sacc[0][0];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[b][r]);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const bool upd = (mx - mrow) * p.scale_log2 > kRescaleLog2;
        const float mnew = upd ? mx : mrow;
        const float alpha = __builtin_amdgcn_exp2f((mrow - mnew) * p.scale_log2);
        mrow = mnew;
        lrow *= alpha;
        return alpha;
    };

    // part 2: exponentials straight into the bf16 P fragments; the row sum adds the rounded
    // weights (v_dot2 against (1, 1)), i.e. exactly the weights the PV MFMA multiplies
    auto softmax_exp = [&](const floatx16 (&sacc)[2], u32x4 (&pf)[2][2]) {
        const float msc = mrow * p.scale_log2;
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float lsum[2] = {0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[b][8 * s2 + 2 * u], p.scale_log2, -msc));
                    const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[b][8 * s2 + 2 * u + 1], p.scale_log2, -msc));
                    const uint32_t w2 = pack_bf16(e0, e1);
                    pf[b][s2][u] = w2;
                    lsum[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones,
                                                                  lsum[u & 1], false);
                }
        lrow += lsum[0] + lsum[1];
    };

    auto apply_mask = [&](int ksl, floatx16 (&sacc)[2]) {
        const int *kp = kpos_s + ksl * KT;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const i32x4 kp4 = *reinterpret_cast<const i32x4 *>(&kp[b * 32 + 8 * i + 4 * lg]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (kp4[j] > rpos) sacc[b][4 * i + j] = -INFINITY;
            }
    };

    auto rescale = [&](float alpha) {
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
    };

    // O^T += V^T P^T for one tile; V^T operands come from two transposing 8-byte LDS reads
    auto pv = [&](int vsl, const u32x4 (&pf)[2][2]) {
        const uint16_t *vb = vs + vsl * VBUF;
        const int gi = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int key = b * 32 + 16 * s2 + 4 * lg + j;
                    const int d = db * 32 + 16 * (gi & 1) + 4 * q;
                    typedef short v4s __attribute__((ext_vector_type(4)));
                    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(vb + key * VS + d));
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(vb + (key + 8) * VS + d));
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pf[b][s2]),
                                                                       oacc[db], 0, 0, 0);
                }
    };

    const int ntiles = (w.page_end - w.page_begin + ppt - 1) / ppt;
    const bool group_b = wave >= 4;
    floatx16 sacc[2];
    u32x4 pf[2][2];

    load_desc(0);
    load_tile();
    load_rope();
    store_tile(0, 0, 0);
    load_desc(1);
    load_tile();
    load_rope();
    store_tile(1, 1, 1);
    lds_barrier();
    qk(0, sacc);
    load_desc(2);
    load_tile();
    if (group_b) lds_barrier();

    // ring slots of tile t (K', positions: t % 3; V: t % 4) and of tiles t+1, t+2
    int k_cur = 0, k_nxt = 1, k_st = 2, v_cur = 0;
    for (int t = 0; t < ntiles; ++t) {
        // Y(t): softmax of tile t; staging of tile t+2; loads of tile t+3. The cos/sin loads of
        // the staged keys go first so that the softmax hides their latency.
        const bool stage = t + 2 < ntiles;
        if (stage) {
            load_rope();
            load_desc(t + 3);
        }
        if (mask_ring & (1u << k_cur)) apply_mask(k_cur, sacc);
        rescale(softmax_max(sacc));
        softmax_exp(sacc, pf);
        if (stage) {
            store_tile(k_st, v_cur ^ 2, t + 2);
            load_tile();
        }
        lds_barrier();
        // X(t): PV of tile t; QK^T of tile t+1
        pv(v_cur, pf);
        if (t + 1 < ntiles) qk(k_nxt, sacc);
        lds_barrier();
        const int k_old = k_cur;
        k_cur = k_nxt;
        k_nxt = k_st;
        k_st = k_old;
        v_cur = (v_cur + 1) & 3;
    }
    if (!group_b) lds_barrier();

    // ---- epilogue: normalise, write the output (or this split's partial result)
    {
        const int m = wave * 32 + ln;
        const int ti = m >> p.gshift;
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lrow), __float_as_uint(lrow), false, false);
        const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const float lse_v = lt > 0.0f ? mrow * p.scale + logf(lt) : -INFINITY;
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

    floatx4 k_lo[NKP], k_hi[NKP], k_c[NKP], k_s[NKP];
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
                    pos = pd.pos0 + slot;
                    base = (int64_t)pd.phys * p.page_elems + head_off + (int64_t)slot * D;
                }
            }
            k_lo[u] = ok ? *reinterpret_cast<const floatx4 *>(kpool + base + 4 * c) : floatx4{0, 0, 0, 0};
            k_hi[u] = ok ? *reinterpret_cast<const floatx4 *>(kpool + base + D / 2 + 4 * c) : floatx4{0, 0, 0, 0};
            const float *cs = p.rope + (int64_t)pos * D + 4 * c;
            k_c[u] = *reinterpret_cast<const floatx4 *>(cs);
            k_s[u] = *reinterpret_cast<const floatx4 *>(cs + D / 2);
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
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                olo[j] = fmaf(k_lo[u][j], k_c[u][j], -k_hi[u][j] * k_s[u][j]);
                ohi[j] = fmaf(k_hi[u][j], k_c[u][j], k_lo[u][j] * k_s[u][j]);
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
        // the tile needs the causal/padding mask iff some key lies after the tile's first row
        mask_next = __any(kp_next > w.rpos_min);
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
    const MergeDesc md = merge[blockIdx.x];
    const int G = 1 << gshift;
    const int mrows = md.n_rows << gshift;
    for (int idx = threadIdx.x; idx < mrows * (D / 4); idx += kThreads) {
        const int m = idx / (D / 4), d4 = idx % (D / 4);
        float L = -INFINITY;
        for (int s = 0; s < md.n_split; ++s) L = fmaxf(L, part_lse[(int64_t)(md.slot0 + s) * tq + m]);
        floatx4 acc = {0, 0, 0, 0};
        float wsum = 0.0f;
        for (int s = 0; s < md.n_split; ++s) {
            const float ls = part_lse[(int64_t)(md.slot0 + s) * tq + m];
            const float wgt = ls == -INFINITY ? 0.0f : expf(ls - L);
            const floatx4 o = *reinterpret_cast<const floatx4 *>(part_o + ((int64_t)(md.slot0 + s) * tq + m) * D + 4 * d4);
            acc += wgt * o;
            wsum += wgt;
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

__global__ __launch_bounds__(kThreads) void link_scatter(const ScatterDesc *table, uint8_t *k_pool, uint8_t *v_pool,
                                                         const uint8_t *k_new, const uint8_t *v_new, int hkv,
                                                         int page_size, int row_bytes, int64_t page_bytes) {
    const ScatterDesc sd = table[blockIdx.x];
    const int h = blockIdx.y;
    const int pieces_per_row = row_bytes / 16;
    const int64_t head_bytes = (int64_t)h * page_size * row_bytes;
    const int64_t dst0 = (int64_t)sd.dst * page_bytes + head_bytes;
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
        *reinterpret_cast<u32x4 *>(k_pool + dst) = a;
        *reinterpret_cast<u32x4 *>(v_pool + dst) = b;
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
                          const ScatterDesc *table, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int elem = s.dtype == 0 ? 2 : 4;
    dim3 grid(n, s.hkv);
    hipLaunchKernelGGL(link_scatter, grid, dim3(kThreads), 0, stream, table, static_cast<uint8_t *>(k_pool),
                       static_cast<uint8_t *>(v_pool), static_cast<const uint8_t *>(k_new),
                       static_cast<const uint8_t *>(v_new), s.hkv, s.page_size, s.d * elem, s.page_elems * elem);
    return hipGetLastError();
}

hipError_t launch_attention(const LayerShape &s, const void *q, const void *k_pool, const void *v_pool,
                            const float *rope, const AttnTables &t, void *out, float *lse, hipStream_t stream) {
    if (t.n_work <= 0) return hipSuccess;
    AttnParams p;
    p.q = q;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.rope = rope;
    p.pages = t.pages;
    p.row_pos = t.row_pos;
    p.work = t.work;
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
    dim3 grid(t.n_work);
    if (s.dtype == 0) {
        if (s.d == 128) hipLaunchKernelGGL(link_attention_bf16<128>, grid, dim3(512), 0, stream, p);
        else hipLaunchKernelGGL(link_attention_bf16<64>, grid, dim3(512), 0, stream, p);
    } else {
        if (s.d == 128) hipLaunchKernelGGL(link_attention_f32<128>, grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL(link_attention_f32<64>, grid, dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_merge(const LayerShape &s, const AttnTables &t, void *out, float *lse, hipStream_t stream) {
    if (t.n_merge <= 0) return hipSuccess;
    const int gshift = log2_exact(s.hq / s.hkv);
    const int tq = tile_qrows(s.dtype);
    dim3 grid(t.n_merge);
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
