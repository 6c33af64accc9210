// HIP kernels of the decoder layers around the link step, for gfx950 (CDNA4).
//
//   linear_bf16   C = A W^T for the selected rows: A [M][K] activations, W [N][K] weights, fp32
//                 accumulation on MFMA, with the epilogue of its place in the layer: the q/k/v
//                 split of the QKV projection, the residual add of the output and down
//                 projections, or SiLU(gate) * up of the MLP's gate and up projections
//   rmsnorm_bf16  y = x / sqrt(mean(x^2) + eps) * w per row
//
// Only the selected rows of a link go through these layers: the cached chunks' K/V of every layer
// come from the compile step (EPIC, atlas.scime.ai summary, "Approach": the first k tokens of each
// chunk, and the suffix, are recomputed through the model; the rest of the chunk is reused).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_dma.h"
#include "model.h"

namespace piclink {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef float floatx2 __attribute__((ext_vector_type(2)));
    floatx2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// ---------------------------------------------------------------------------------------------
// linear_bf16. Work group = 4 waves, tile BM x BN = 128 x 128 of C over K in steps of BK = 64.
// Wave (wm, wn) owns C rows [64 wm, 64 wm + 64) and columns [64 wn, 64 wn + 64) of the tile, as
// 2 x 2 blocks of 32 x 32. Each block is computed transposed, C^T = W A^T, with
// v_mfma_f32_32x32x16_bf16 (A operand: 32 rows of W, B operand: 32 rows of A; both K-contiguous,
// read with one 16-byte LDS load per lane), so that a lane holds four consecutive columns of one
// row of C per group of accumulators and writes them with one 8-byte store.
// A and W tiles are double-buffered in LDS (row stride BK + 8: conflict-free fragment reads); the
// next K step's tiles are loaded into registers while the current one is multiplied.
constexpr int BM = 128, BN = 128, BK = 64, KS = BK + 8, NT = 256;

struct LinearParams {
    const uint16_t *a;        // [M][K]
    const uint16_t *w;        // [N][K]
    int m, n, k;
    int epilogue;             // LinearEpilogue
    uint16_t *out[3];         // outputs; kSplit3: column ranges [0, n0), [n0, n0 + n1), [n0 + n1, n)
    int ld_out[3];            // row stride of each output (elements)
    int split0, split1;       // kSplit3: columns of the first and second output
    const uint16_t *residual; // kResidual: [M][N] added to the product (may alias out[0])
    int tiles_m, tiles_n;
};

// The epilogue of both GEMM kernels: the wave's 64 x 64 slice of C at rows m0 + 64 wm, columns
// n0 + 64 wn, from its 2 x 2 accumulator blocks (n block i, m block j).
__device__ __forceinline__ void store_tile(const LinearParams &p, const floatx16 (&acc)[2][2], int m0, int n0, int wm,
                                           int wn, int ln, int lg) {
    // epilogue: lane (ln, lg) of block (i, j) holds C[row][col .. col + 3] in accumulators
    // 4g .. 4g + 3, row = m0 + 64 wm + 32 j + ln, col = n0 + 64 wn + 32 i + 8 g + 4 lg
    if (p.epilogue == kSwiGlu) {
        // W rows alternate 32 gate rows and 32 up rows: block i = 0 holds gate, i = 1 up, for the
        // output columns (n0 + 64 wn) / 2 + 8 g + 4 lg .. + 3
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = m0 + 64 * wm + 32 * j + ln;
            if (row >= p.m) continue;
            uint16_t *orow = p.out[0] + (int64_t)row * p.ld_out[0] + (n0 + 64 * wn) / 2;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gt = acc[0][j][4 * g + e], up = acc[1][j][4 * g + e];
                    v[e] = gt / (1.0f + __expf(-gt)) * up;
                }
                u32x2 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
                *reinterpret_cast<u32x2 *>(orow + 8 * g + 4 * lg) = o;
            }
        }
        return;
    }
    // column ranges of the split outputs (a 32-column block never straddles two of them)
    int which = 0, col_base = 0;
    if (p.epilogue == kSplit3) {
        const int c0 = n0 + 64 * wn;
        which = c0 >= p.split0 + p.split1 ? 2 : c0 >= p.split0 ? 1 : 0;
        col_base = which == 2 ? p.split0 + p.split1 : which == 1 ? p.split0 : 0;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = m0 + 64 * wm + 32 * j + ln;
        if (row >= p.m) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int col = n0 + 64 * wn + 32 * i - col_base;
            uint16_t *orow = p.out[which] + (int64_t)row * p.ld_out[which] + col;
            const uint16_t *rrow = p.residual ? p.residual + (int64_t)row * p.n + n0 + 64 * wn + 32 * i : nullptr;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
                if (p.epilogue == kResidual) {
                    const u32x2 r = *reinterpret_cast<const u32x2 *>(rrow + 8 * g + 4 * lg);
                    v[0] += bf_lo(r[0]);
                    v[1] += bf_hi(r[0]);
                    v[2] += bf_lo(r[1]);
                    v[3] += bf_hi(r[1]);
                }
                u32x2 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
                *reinterpret_cast<u32x2 *>(orow + 8 * g + 4 * lg) = o;
            }
        }
    }
}

__global__ __launch_bounds__(NT, 2) void linear_bf16(LinearParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t as[2][BM * KS];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN * KS];

    // work groups are dealt round-robin over the 8 XCDs: give each XCD a contiguous run of tiles,
    // N-major, so that the work groups sharing one W tile run on one XCD and share its L2
    const int tiles = p.tiles_m * p.tiles_n;
    const int per_xcd = (tiles + 7) / 8;
    const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= tiles) return;
    const int tn = t / p.tiles_m, tm = t % p.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    // global -> register staging: 4 pieces of 16 bytes of A and 4 of W per thread per K step
    // (row = tid / 8 + 32 i, 8 elements at column 8 (tid % 8)); rows of A past M read row M - 1
    const int srow = tid >> 3, scol = (tid & 7) * 8;
    const uint16_t *a_src[4];
    const uint16_t *w_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(m0 + srow + 32 * i, p.m - 1);
        a_src[i] = p.a + (int64_t)r * p.k + scol;
        w_src[i] = p.w + (int64_t)(n0 + srow + 32 * i) * p.k + scol;
    }
    u32x4 a_reg[4], w_reg[4];
    auto load = [&](int kt) __attribute__((always_inline)) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a_reg[i] = *reinterpret_cast<const u32x4 *>(a_src[i] + k0);
            w_reg[i] = *reinterpret_cast<const u32x4 *>(w_src[i] + k0);
        }
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u32x4 *>(&as[buf][(srow + 32 * i) * KS + scol]) = a_reg[i];
            *reinterpret_cast<u32x4 *>(&ws[buf][(srow + 32 * i) * KS + scol]) = w_reg[i];
        }
    };

    floatx16 acc[2][2];   // [n block][m block]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int n_kt = p.k / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < n_kt) load(kt + 1);
        const uint16_t *wb = &ws[buf][(64 * wn + ln) * KS + 8 * lg];
        const uint16_t *ab = &as[buf][(64 * wm + ln) * KS + 8 * lg];
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            bf16x8 wf[2], af[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                wf[i] = *reinterpret_cast<const bf16x8 *>(wb + 32 * i * KS + 16 * s);
                af[i] = *reinterpret_cast<const bf16x8 *>(ab + 32 * i * KS + 16 * s);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < n_kt) store(buf ^ 1);
        __syncthreads();
    }

    store_tile(p, acc, m0, n0, wm, wn, ln, lg);
}

// ---------------------------------------------------------------------------------------------
// linear_bf16_dl: the same product and epilogues with a tile of 128 rows of A x 256 rows of W
// (8 waves, each the 64 x 64 slice of linear_bf16) whose operand tiles are loaded straight from
// global memory into LDS (global_load_lds_dwordx4: lane i of an instruction writes its 16 bytes at
// the instruction's LDS base + 16 i), in a ring of 3 K steps of 64 loaded two steps ahead.
//   - Rows are unpadded (128 bytes) and chunk c of row r sits at c ^ ((r >> 1) & 7): the 16 lanes
//     of one fragment read take 16 consecutive rows at 16 distinct 16-byte bank groups. Each lane
//     of a load fetches the global chunk that lands at its LDS position.
//   - A K step is 48 load instructions of 8 rows (32 of W, 16 of A), 6 per wave. Before the one
//     barrier of step kt each wave waits for its own loads of step kt (the 6 of step kt+1 may stay
//     in flight); after it, step kt+2's loads go into the slot that step kt-1 used.
constexpr int DBM = 128, DBN = 256, DNT = 512, DSTAGES = 3, DLOADS = 6;

__global__ __launch_bounds__(DNT, 1) void linear_bf16_dl(LinearParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t wsm[DSTAGES][DBN * BK];
    __shared__ __attribute__((aligned(16))) uint16_t asm_[DSTAGES][DBM * BK];

    const int tiles = p.tiles_m * p.tiles_n;
    const int per_xcd = (tiles + 7) / 8;
    const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= tiles) return;
    const int tn = t / p.tiles_m, tm = t % p.tiles_m;
    const int m0 = tm * DBM, n0 = tn * DBN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
    const int wn = wave & 3, wm = wave >> 2;
    const int wv = __builtin_amdgcn_readfirstlane(wave);

    // this wave's loads: instruction i is 8-row group q = 6 wave + i (q < 32: W rows 8q..; else A
    // rows 8 (q - 32)..); lane -> row 8q + lane / 8, LDS chunk lane % 8, global chunk swizzled
    const char *src[DLOADS];
#pragma unroll
    for (int i = 0; i < DLOADS; ++i) {
        const int q = DLOADS * wv + i;
        const bool is_w = q < DBN / 8;
        const int r = 8 * (is_w ? q : q - DBN / 8) + (lane >> 3);
        const int gc = (lane & 7) ^ ((r >> 1) & 7);
        const uint16_t *row = is_w ? p.w + (int64_t)(n0 + r) * p.k : p.a + (int64_t)min(m0 + r, p.m - 1) * p.k;
        src[i] = reinterpret_cast<const char *>(row + 8 * gc);
    }
    auto issue = [&](int kt, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DLOADS; ++i) {
            const int q = DLOADS * wv + i;
            uint16_t *dst = q < DBN / 8 ? &wsm[st][q * 8 * BK] : &asm_[st][(q - DBN / 8) * 8 * BK];
            dma16(src[i] + (int64_t)kt * BK * 2, lds_addr(dst));
        }
    };

    // fragment reads: rows 64 wn + 32 i + ln of W and 64 wm + 32 j + ln of A, chunk 2 s + lg at
    // (2 s + lg) ^ ((row >> 1) & 7) = x0 ^ 2 s (the row's bits 1-3 are those of ln)
    const int x0 = lg ^ ((ln >> 1) & 7);
    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int n_kt = p.k / BK;
    issue(0, 0);
    if (n_kt > 1) issue(1, 1);
    int st = 0;
    for (int kt = 0; kt < n_kt; ++kt) {
        if (kt + 1 < n_kt) wait_vmcnt<DLOADS>();
        else wait_vmcnt<0>();
        barrier_dl();
        if (kt + 2 < n_kt) issue(kt + 2, st == 0 ? 2 : st - 1);
        const uint16_t *wb = &wsm[st][(64 * wn + ln) * BK];
        const uint16_t *ab = &asm_[st][(64 * wm + ln) * BK];
        bf16x8 wf[4][2], af[4][2];
#pragma unroll
        for (int s = 0; s < BK / 16; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                wf[s][i] = *reinterpret_cast<const bf16x8 *>(wb + 32 * i * BK + 8 * (x0 ^ (2 * s)));
                af[s][i] = *reinterpret_cast<const bf16x8 *>(ab + 32 * i * BK + 8 * (x0 ^ (2 * s)));
            }
#pragma unroll
        for (int s = 0; s < BK / 16; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s][i], af[s][j], acc[i][j], 0, 0, 0);
        st = st == 2 ? 0 : st + 1;
    }
    store_tile(p, acc, m0, n0, wm, wn, ln, lg);
}

// ---------------------------------------------------------------------------------------------
// linear_bf16_big: the same product and epilogues for large grids, with a tile of 256 rows of A x
// 256 rows of W (8 waves, each 64 columns x 128 rows: 2 x 4 blocks of 32 x 32), so that each byte
// loaded into LDS feeds 1.5 times the MFMA work of linear_bf16_dl. Operand tiles go straight
// into LDS in a ring of 4 K steps of 32, loaded three steps ahead.
//   - Rows of a K step are 64 bytes (4 chunks); chunk c of row r sits at c ^ ((r >> 2) & 3), so the
//     16 lanes of one fragment read (16 consecutive rows) take 16 distinct 16-byte bank groups.
//   - A K step is 32 load instructions of 16 rows (16 of W, 16 of A), 4 per wave; each wave waits
//     for its own loads of step kt before the step's barrier (those of the later steps in flight
//     may stay), and issues step kt+3 into the slot that step kt-1 used after it.
constexpr int GBM = 256, GBN = 256, GBK = 32, GNT = 512, GSTAGES = 4, GLOADS = 4;

__global__ __launch_bounds__(GNT, 1) void linear_bf16_big(LinearParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t wsm[GSTAGES][GBN * GBK];
    __shared__ __attribute__((aligned(16))) uint16_t asm_[GSTAGES][GBM * GBK];

    const int tiles = p.tiles_m * p.tiles_n;
    const int per_xcd = (tiles + 7) / 8;
    const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= tiles) return;
    const int tn = t / p.tiles_m, tm = t % p.tiles_m;
    const int m0 = tm * GBM, n0 = tn * GBN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 31, lg = lane >> 5;
    const int wn = wave & 3, wm = wave >> 2;
    const int wv = __builtin_amdgcn_readfirstlane(wave);

    // this wave's loads: instruction i is 16-row group q = 4 wave + i (q < 16: W rows 16q..; else
    // A rows 16 (q - 16)..); lane -> row 16q + lane / 4, LDS chunk lane % 4, global chunk swizzled
    const char *src[GLOADS];
#pragma unroll
    for (int i = 0; i < GLOADS; ++i) {
        const int q = GLOADS * wv + i;
        const bool is_w = q < GBN / 16;
        const int r = 16 * (is_w ? q : q - GBN / 16) + (lane >> 2);
        const int gc = (lane & 3) ^ ((r >> 2) & 3);
        const uint16_t *row = is_w ? p.w + (int64_t)(n0 + r) * p.k : p.a + (int64_t)min(m0 + r, p.m - 1) * p.k;
        src[i] = reinterpret_cast<const char *>(row + 8 * gc);
    }
    auto issue = [&](int kt, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < GLOADS; ++i) {
            const int q = GLOADS * wv + i;
            uint16_t *dst = q < GBN / 16 ? &wsm[st][q * 16 * GBK] : &asm_[st][(q - GBN / 16) * 16 * GBK];
            dma16(src[i] + (int64_t)kt * GBK * 2, lds_addr(dst));
        }
    };

    // fragment reads: rows 64 wn + 32 i + ln of W and 128 wm + 32 j + ln of A, chunk 2 s + lg at
    // (2 s + lg) ^ ((row >> 2) & 3) = x0 ^ 2 s (the row's bits 2-3 are those of ln)
    const int x0 = lg ^ ((ln >> 2) & 3);
    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int n_kt = p.k / GBK;
#pragma unroll
    for (int k = 0; k < GSTAGES - 1; ++k)
        if (k < n_kt) issue(k, k);
    int st = 0;
    for (int kt = 0; kt < n_kt; ++kt) {
        // loads of later steps this wave has in flight: steps kt+1, kt+2 when they exist
        const int later = min(GSTAGES - 2, n_kt - 1 - kt);
        if (later >= 2) wait_vmcnt<2 * GLOADS>();
        else if (later == 1) wait_vmcnt<GLOADS>();
        else wait_vmcnt<0>();
        barrier_dl();
        if (kt + GSTAGES - 1 < n_kt) issue(kt + GSTAGES - 1, st == 0 ? GSTAGES - 1 : st - 1);
        const uint16_t *wb = &wsm[st][(64 * wn + ln) * GBK];
        const uint16_t *ab = &asm_[st][(128 * wm + ln) * GBK];
#pragma unroll
        for (int s = 0; s < GBK / 16; ++s) {
            bf16x8 wf[2], af[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) wf[i] = *reinterpret_cast<const bf16x8 *>(wb + 32 * i * GBK + 8 * (x0 ^ (2 * s)));
#pragma unroll
            for (int j = 0; j < 4; ++j) af[j] = *reinterpret_cast<const bf16x8 *>(ab + 32 * j * GBK + 8 * (x0 ^ (2 * s)));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
        }
        st = st == GSTAGES - 1 ? 0 : st + 1;
    }
    // the wave's 128 rows as two 64-row slices of the shared epilogue
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const floatx16 sub[2][2] = {{acc[0][2 * h], acc[0][2 * h + 1]}, {acc[1][2 * h], acc[1][2 * h + 1]}};
        store_tile(p, sub, m0 + 128 * wm + 64 * h, n0, 0, wn, ln, lg);
    }
}

// ---------------------------------------------------------------------------------------------
// rmsnorm_bf16: one wave per row. y = x * rsqrt(mean(x^2) + eps) * w, the sum of squares in fp32.
template <int PER_LANE>
__global__ __launch_bounds__(256) void rmsnorm_bf16(const uint16_t *x, const uint16_t *w, uint16_t *y, int rows,
                                                    int dm, float eps) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const uint16_t *xr = x + (int64_t)row * dm;
    u32x4 v[PER_LANE];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int c = (i * 64 + lane) * 8;
        v[i] = c < dm ? *reinterpret_cast<const u32x4 *>(xr + c) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = bf_lo(v[i][e]), b = bf_hi(v[i][e]);
            ss = fmaf(a, a, ss);
            ss = fmaf(b, b, ss);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = rsqrtf(ss / (float)dm + eps);
    uint16_t *yr = y + (int64_t)row * dm;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int c = (i * 64 + lane) * 8;
        if (c >= dm) continue;
        const u32x4 wv = *reinterpret_cast<const u32x4 *>(w + c);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16(bf_lo(v[i][e]) * inv * bf_lo(wv[e]), bf_hi(v[i][e]) * inv * bf_hi(wv[e]));
        *reinterpret_cast<u32x4 *>(yr + c) = o;
    }
}

}  // namespace

hipError_t launch_linear(const LinearCall &c, hipStream_t stream) {
    if (c.m <= 0) return hipSuccess;
    if (c.n % BN != 0 || c.k % BK != 0 || c.k <= 0) return hipErrorInvalidValue;
    LinearParams p{};
    p.a = static_cast<const uint16_t *>(c.a);
    p.w = static_cast<const uint16_t *>(c.w);
    p.m = c.m;
    p.n = c.n;
    p.k = c.k;
    p.epilogue = c.epilogue;
    for (int i = 0; i < 3; ++i) {
        p.out[i] = static_cast<uint16_t *>(c.out[i]);
        p.ld_out[i] = c.ld_out[i];
    }
    p.split0 = c.split0;
    p.split1 = c.split1;
    p.residual = static_cast<const uint16_t *>(c.residual);
    // the 256 x 256 tile where it needs fewer rounds of the 256 compute units, each round weighed
    // 1.7 times a round of 128 x 256 tiles (twice the work at 1.5 times the MFMA work per byte
    // loaded: 15% faster per FLOP). At 3,200 rows that picks it for the output and down
    // projections (208 tiles: one round against two, 12% and 9% faster) and for gate/up, and
    // keeps 128 x 256 for the QKV projection (two rounds against three; 256 x 256 was 9% slower)
    const int64_t big_rounds = ((int64_t)((c.m + GBM - 1) / GBM) * (c.n / GBN) + 255) / 256;
    const int64_t dl_rounds = ((int64_t)((c.m + DBM - 1) / DBM) * (c.n / DBN) + 255) / 256;
    if (c.n % GBN == 0 && 17 * big_rounds < 10 * dl_rounds) {
        p.tiles_m = (c.m + GBM - 1) / GBM;
        p.tiles_n = c.n / GBN;
        const int grid = 8 * ((p.tiles_m * p.tiles_n + 7) / 8);
        hipLaunchKernelGGL(linear_bf16_big, dim3(grid), dim3(GNT), 0, stream, p);
        return hipGetLastError();
    }
    if (c.n % DBN == 0) {
        p.tiles_m = (c.m + DBM - 1) / DBM;
        p.tiles_n = c.n / DBN;
        const int grid = 8 * ((p.tiles_m * p.tiles_n + 7) / 8);
        hipLaunchKernelGGL(linear_bf16_dl, dim3(grid), dim3(DNT), 0, stream, p);
        return hipGetLastError();
    }
    p.tiles_m = (c.m + BM - 1) / BM;
    p.tiles_n = c.n / BN;
    const int tiles = p.tiles_m * p.tiles_n;
    const int grid = 8 * ((tiles + 7) / 8);
    hipLaunchKernelGGL(linear_bf16, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const void *x, const void *w, void *y, int rows, int dm, float eps, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (dm % 8 != 0 || dm > 64 * 8 * 16) return hipErrorInvalidValue;
    const dim3 grid((rows + 3) / 4);
    const int per_lane = (dm + 511) / 512;
    auto *xp = static_cast<const uint16_t *>(x);
    auto *wp = static_cast<const uint16_t *>(w);
    auto *yp = static_cast<uint16_t *>(y);
    if (per_lane <= 1) hipLaunchKernelGGL(rmsnorm_bf16<1>, grid, dim3(256), 0, stream, xp, wp, yp, rows, dm, eps);
    else if (per_lane <= 2) hipLaunchKernelGGL(rmsnorm_bf16<2>, grid, dim3(256), 0, stream, xp, wp, yp, rows, dm, eps);
    else if (per_lane <= 4) hipLaunchKernelGGL(rmsnorm_bf16<4>, grid, dim3(256), 0, stream, xp, wp, yp, rows, dm, eps);
    else if (per_lane <= 8) hipLaunchKernelGGL(rmsnorm_bf16<8>, grid, dim3(256), 0, stream, xp, wp, yp, rows, dm, eps);
    else hipLaunchKernelGGL(rmsnorm_bf16<16>, grid, dim3(256), 0, stream, xp, wp, yp, rows, dm, eps);
    return hipGetLastError();
}

}  // namespace piclink
