// pkv_prefill.hip -- paged prefill and mixed prefill + decode steps on gfx950
// (MI355X): several new query rows per entry, appended to the paged cache and
// attended causally over it.
//
// Entry b brings n_b = qo_indptr[b+1] - qo_indptr[b] new rows (a decode row
// is n_b = 1); after the append its L tokens end with them, so row j sits at
// position p = L - n_b + j and attends tokens 0 .. p ("Adding a Model",
// "How a program runs": prefill runs several rows per request over the same
// paged cache; "Supported Models", Qwen3-Omni / Qwen3-TTS notes: new prompts
// ride a decode step as one mixed step).
//
// Several rows against the same keys make a dense contraction, so the
// products run on the matrix cores (v_mfma_f32_16x16x32_bf16).  The query
// columns of an entry and KV head are its (row, query head) pairs, column
// j G + g for row j and head g of the head group (the G heads of a row share
// the keys and values), cut into column tiles of 128.  Four waves take the
// 128 columns of a tile, 32 per wave in two blocks of 16, and walk the
// entry's tokens up to the tile's last position in token tiles of 32:
//   S^T[t][c] = sum_d K[t][d] Q[c][d]     K rows as the A operand (LDS),
//                                         Q^T as the B operand (registers)
//   O^T[d][c] += sum_t V^T[d][t] P^T[t][c] V^T as the A operand, read
//                                         transposed from V rows in LDS
// The MFMA gives lane l the scores of column l % 16 at tokens 4 (l / 16) + r
// of each 16-token half of the tile, which is exactly a B operand of the
// second product when its contraction index k = 8 (l / 16) + e names token
// 4 (l / 16) + e (e < 4) or 16 + 4 (l / 16) + e - 4 (e >= 4) (the order of a
// sum is free).  V^T in that token order is what ds_read_b64_tr_b16 returns
// from V rows: within each 16 lanes it hands lane i element i % 4 of the
// 8 bytes that lane 4 e + i / 4 addressed, so four lanes addressing four
// consecutive d of one token row give lane i four tokens of one d.  The
// online softmax of a column stays within its four lanes.  P goes in as a
// bf16 high part and a bf16 remainder (two products): with a single bf16 P
// some outputs of unit-variance inputs already miss the per-element bar
// (half a bf16 step of the output plus 1e-3).
//
// Balance.  Column tile j of an entry needs about j + 1 token tiles (its
// rows' prefixes grow with j), so a workgroup of eight waves takes the pair
// of column tiles (k, T-1-k) as two chains of four waves that walk about the
// same number of token tiles: chain A all of tile k and then the first
// token tiles of tile T-1-k, chain B the rest of tile T-1-k.  Chain A's wave
// w and chain B's wave w hold the same columns of tile T-1-k, and at the end
// B merges A's partial (running maximum, weight sum, outputs) from LDS.  The
// middle tile of an odd T is split the same way.  Each SIMD holds one wave of
// each chain.
//
// Each chain stages its token tiles through a ring of three LDS slots with
// direct-to-LDS copies (global_load_lds_dwordx4, 1 KiB a copy), so no
// registers hold tiles in flight; a tile read from cached pages has its page
// ids read a step ahead by scalar loads.  Rows sit unpadded in LDS with their
// 16-byte chunks permuted by an XOR of the row index, chosen so that the
// operand reads of a wave (K rows, and the transposed V reads) meet distinct
// banks.  New rows are read from k_new / v_new, and the workgroups of an
// entry and KV head share writing them into the cache.
//
// The grid lists (entry, KV head, pair) with the pairs of one (entry, KV
// head) adjacent, dealt so that they run on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kInitMax = -1e30f;       // running maximum before any token (log2 domain)
constexpr float kTau = 8.0f;             // lazy-rescale threshold, log2 units
constexpr int kTileTok = 32;             // tokens per token tile
constexpr int kCols = 128;               // query columns per column tile
constexpr int kWaves = 8;                // two chains of four waves
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 3;                 // LDS slots per chain

// LDS layout: per chain kRing tile slots (K rows, then V rows, 2 D bytes a
// row), the two chains side by side, then the q rows of chain A's second
// column tile.  After the walk the same memory holds chain A's partials.
template <int D>
struct Geo {
    static constexpr int CPR = D / 8;               // 16-byte chunks per row
    static constexpr int RPC = 64 / CPR;            // rows per 1 KiB copy
    static constexpr int CPW = kTileTok / RPC / 4;  // copies per wave, per tensor and tile
    static constexpr int TILE = kTileTok * 2 * D;   // bytes of K (or V) in a tile
    static constexpr int SLOT = 2 * TILE;
    static constexpr int RING = kRing * SLOT;
    static constexpr int QA = 4 * 32 * 2 * D;        // chain A's second q tile
    static constexpr int LDS = 2 * RING + QA;
    static constexpr int DC = D / 32;               // 32-value chunks of d (first product)
    static constexpr int DB = D / 16;               // 16-row blocks of d (second product)
    static constexpr int MQ = 2 * DB + 1;           // 16-byte words of a lane's partial
    static_assert(CPW >= 1 && 4 * CPW * RPC == kTileTok, "unsupported head_dim");
    static_assert(4 * MQ * 64 * 16 <= LDS, "partials do not fit");
};

// Chunk permutations (XOR of the chunk index) of K and V rows in LDS.  K is
// read as 16 rows x one 16-byte chunk per 16 lanes, V (transposed) as 4
// consecutive rows x two chunks per 16 lanes and 8 rows per 32 lanes; both
// land on 16 distinct 4-bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    return D == 128 ? ((r << 1) & 14) : (r & 6);
}

// s_waitcnt immediate for "at most n vector memory operations outstanding"
// (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maximum).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Direct-to-LDS copies: 16 (or 4) bytes from each lane's global address to
// LDS at lds + 16 * lane (4 * lane); lds is wave-uniform and goes through M0.
// They are inline assembly, so the compiler does not track them: the kernel
// waits for them itself.
__device__ __forceinline__ void copy16_to_lds(const void *src, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
// The same from a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void copy16_to_lds_s(const void *base, uint32_t off, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// two fp32 -> two bf16 (round to nearest even), packed low-first: one
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo_up(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_up(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Maximum (sum) over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column's
// lanes), with the gfx950 cross-row lane swaps.
__device__ __forceinline__ float column_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float column_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8_t, u32x4_t{v.x, v.y, v.z, v.w});
}

// ---------------------------------------------------------------------------
// Causal attention of the new rows (and their append); see the file comment.
// One work item: the column tile pair kk of entry b at KV head h, taken by
// the whole workgroup (every wave returns from it; the exits are uniform).
template <int D>
__device__ __forceinline__ void tile_pair(const PrefillArgs &a, const int b, const int h,
                                          const int kk) {
    using Gm = Geo<D>;
    constexpr int DC = Gm::DC, DB = Gm::DB, CPR = Gm::CPR, RPC = Gm::RPC, CPW = Gm::CPW;
    constexpr int RB = 2 * D;   // bytes per row in LDS
    __shared__ __attribute__((aligned(1024))) char smem[Gm::LDS];
    const int G = a.num_qo_heads / a.num_kv_heads;

    const int r0 = a.qo_indptr[b];
    const int n = a.qo_indptr[b + 1] - r0;
    if (n < 1 || (n == 1 && a.skip_single))
        return;
    const int nc = min(n, a.max_rows);   // rows computed (and appended)
    const int ncols = nc * G;
    const int T = (ncols + kCols - 1) / kCols;
    if (kk >= (T + 1) / 2)
        return;
    const int p0 = a.indptr[b];
    const int np = a.indptr[b + 1] - p0;
    const int last = a.last_len[b];
    if (np < 1 || last < 1 || last > a.page_size ||
        (int64_t)(np - 1) * a.page_size + last > 0x7fffff00LL)
        return;
    const int len = (np - 1) * a.page_size + last;
    if (n > len)
        return;
    const int base_pos = len - n;   // position of the entry's first new row
    const int32_t *pages = a.indices + p0;

    // the two chains: A = column tile jl over token tiles [0, nA1), then
    // column tile jh over [0, nA2); B = column tile jh over [xB, xB + nB)
    auto tiles_of = [&](int j) {   // token tiles column tile j walks
        return (base_pos + (min(ncols, kCols * (j + 1)) - 1) / G) / kTileTok + 1;
    };
    const int jl = kk, jh = T - 1 - kk;
    int nA1, nA2, xB, nB;
    if (jl < jh) {
        const int w1 = tiles_of(jl), w2 = tiles_of(jh);
        const int x = max(0, (w1 + w2) / 2 - w1);
        nA1 = w1; nA2 = x; xB = x; nB = w2 - x;
    } else {   // the middle tile, halved
        const int w = tiles_of(jl);
        nA1 = w / 2; nA2 = 0; xB = w / 2; nB = w - w / 2;
    }
    // B merges A's partial when A walked part of B's column tile
    const bool merge = jl < jh ? nA2 > 0 : nA1 > 0;
    const int lenA = nA1 + nA2;

    const int tid = threadIdx.x;
    // wave-uniform by construction; readfirstlane lets the compiler know it,
    // so the walk's branches (and its waits) stay scalar
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int chain = wv >> 2, w4 = wv & 3;
    const int q = lane >> 4, c = lane & 15;
    const int my_len = chain ? nB : lenA;
    char *ring = smem + chain * Gm::RING;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
    auto tok_tile = [&](int s) { return chain ? xB + s : (s < nA1 ? s : s - nA1); };

    // fold a negative scale into q (exact: a sign flip of bf16)
    const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(a.scale_log2);

    // ---- the wave's columns and running state
    int cpos[2];
    int cur_j = 0;   // the wave's column tile
    bool cok[2];
    bf16x8_t qb[2][DC];
    f32x4_t o[2][DB];
    float m[2], lsum[2];
    int wmin = 0, wmax = -1;   // first and last position among the wave's valid columns
    // column c of the wave's 32 in column tile j -> its row, head and q row
    auto column_of = [&](int j, int cw, int &row, int &head) {
        const int col = min(kCols * j + 32 * w4 + cw, ncols - 1);
        row = col / G;
        head = h * G + col % G;
    };
    auto set_geometry = [&](int j) {
        const int colw = kCols * j + 32 * w4;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            cok[cb] = colw + 16 * cb + c < ncols;
            int row, head;
            column_of(j, 16 * cb + c, row, head);
            cpos[cb] = cok[cb] ? base_pos + row : -1;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[cb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            m[cb] = kInitMax;   // running maximum of the column (log2 domain)
            lsum[cb] = 0.f;     // this lane's share of the column's weight sum
        }
        cur_j = j;
        wmin = base_pos + min(colw, ncols - 1) / G;
        wmax = colw < ncols ? base_pos + (min(ncols, colw + 32) - 1) / G : -1;
    };
    auto flip = [&](uint4 v) {
        v.x ^= qflip; v.y ^= qflip; v.z ^= qflip; v.w ^= qflip;
        return as_bf16x8(v);
    };
    auto finalize = [&]() {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            // the column's weight sum over its four lanes, then the outputs
            const float ls = column_sum(lsum[cb]);
            if (!cok[cb])
                continue;
            const float inv = 1.f / ls;
            int row, head;
            column_of(cur_j, 16 * cb + c, row, head);
            const int64_t orow_i = (int64_t)(r0 + row) * a.num_qo_heads + head;
            uint16_t *orow = a.out + orow_i * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                // lane holds O^T[16 db + 4 q + r][c]
                const uint32_t w0 = bf16x2_rne(o[cb][db][0] * inv, o[cb][db][1] * inv);
                const uint32_t w1 = bf16x2_rne(o[cb][db][2] * inv, o[cb][db][3] * inv);
                *reinterpret_cast<uint2 *>(orow + 16 * db + 4 * q) = make_uint2(w0, w1);
            }
            if (a.lse != nullptr && q == 0)
                a.lse[orow_i] =
                    (m[cb] + __log2f(ls)) * 0.6931471805599453f;
        }
    };

    // ---- LDS read offsets within a slot, as a lane base and an XOR term (the
    // chunk permutation commutes with the chunk's place: 4 dc + q = 4 dc | q
    // and 2 db + hb = 2 db | hb, and the permutations of K and V keep those
    // low bits apart), so that each offset costs one xor-add
    // K: row 16 tb + c, logical chunk 4 dc + q (also the q rows of chain A's
    // second column tile, one row per column)
    const int kbase = c * RB;
    const int kx = 16 * (q ^ swz_k<D>(c));
    auto koff = [&](int dc) { return (kx ^ (64 * dc)) + kbase; };
    // V (transposed reads): row 4 q + c / 4 (+16), d = 16 db + 4 (c % 4)
    const int vr_ = 4 * q + (c >> 2);
    const int vbase = vr_ * RB + 16 * ((c & 3) >> 1) + 8 * (c & 1);
    const int vx = 16 * swz_v<D>(vr_);   // even chunk permutation: keeps bit 0 (hb)
    auto voff = [&](int db) { return (vx ^ (32 * db)) + vbase; };

    // the first column tile's q rows, straight from global memory
    {
        const int j = chain ? jh : jl;
        set_geometry(j);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            int row, head;
            column_of(j, 16 * cb + c, row, head);
            const uint4 *src = reinterpret_cast<const uint4 *>(
                a.q + ((int64_t)(r0 + row) * a.num_qo_heads + head) * D + 8 * q);
#pragma unroll
            for (int dc = 0; dc < DC; ++dc)
                qb[cb][dc] = flip(src[4 * dc]);
        }
    }

    // ---- copies.  Copy i of a wave moves rows RPC (w4 + 4 i) .. + RPC - 1 of
    // a token tile; lane l holds row + l / CPR, LDS chunk l % CPR, which is
    // logical chunk (l % CPR) ^ swz(row) of the source row.  Token tile s
    // goes to ring slot s % kRing.
    const int pmask = a.page_size - 1;   // page sizes are powers of two
    const bool fresh = a.k_new != nullptr;
    const bool big_pages = a.page_size >= RPC;   // a copy's rows share a page
    const int rr = lane / CPR;   // row within a copy
    // source chunk offsets (elements) of K and V of copy i
    auto kel = [&](int i) { return 8 * ((lane % CPR) ^ swz_k<D>(RPC * (w4 + 4 * i) + rr)); };
    auto vel = [&](int i) { return 8 * ((lane % CPR) ^ swz_v<D>(RPC * (w4 + 4 * i) + rr)); };
    uint32_t kvo[CPW], vvo[CPW]; // the same plus the row, in bytes from the copy's first row
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        kvo[i] = 2u * (uint32_t)(rr * a.row_stride + kel(i));
        vvo[i] = 2u * (uint32_t)(rr * a.row_stride + vel(i));
    }
    // Byte addressing.  New rows come from k_new / v_new (row r0 + tok -
    // base_pos), the others from their page.
    const uint32_t rs_b = 2u * (uint32_t)a.row_stride;   // bytes per token row (all heads)
    const char *knew_t = reinterpret_cast<const char *>(
        fresh ? a.k_new + ((int64_t)r0 - base_pos) * a.row_stride + h * D : a.cache);
    const int64_t vnew_b = fresh ? 2 * (a.v_new - a.k_new) : 0;   // v_new row - k_new row
    const char *cache_hb = reinterpret_cast<const char *>(a.cache + h * D);
    // page and half-page strides in bytes: under 4 GiB (the host checks)
    const uint32_t ps_b = 2u * (uint32_t)a.page_stride, hs_b = 2u * (uint32_t)a.half_stride;
    uint32_t roff[CPW];   // bytes from a tile's first row to copy i's first row
#pragma unroll
    for (int i = 0; i < CPW; ++i)
        roff[i] = (uint32_t)(RPC * (w4 + 4 * i)) * rs_b;
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    const const_i32 *pages_s = (const const_i32 *)(pages);   // scalar loads of the same ids
    typedef int PageIds[CPW];   // page id of each copy's first row (scalar registers)
    auto page_base = [&](int page, int tok0) {   // first element of token tok0's row (head h)
        const int pg = (uint32_t)page < (uint32_t)a.num_pages ? page : 0;   // bad id: no fault
        return (int64_t)pg * a.page_stride + (int64_t)(tok0 & pmask) * a.row_stride + h * D;
    };
    // first byte of copy i's rows in the cache (one page holds them)
    auto cached_base = [&](int page, int t0, int i) {
        const uint32_t pg = (uint32_t)page < (uint32_t)a.num_pages ? (uint32_t)page : 0u;
        return cache_hb + (uint64_t)pg * ps_b +
               (uint32_t)((t0 + RPC * (w4 + 4 * i)) & pmask) * rs_b;
    };
    auto slot_of = [&](int s) { return (s % kRing) * Gm::SLOT; };   // ring slot, bytes
    // A token tile is copied one way for all its rows: kFresh (all new rows,
    // from k_new / v_new), kCached (no new row, every copy's rows in one
    // page), or kEdge (per lane: tiles over the prefix or the entry's end, or
    // pages shorter than a copy).
    enum : int { kCached = 0, kFresh = 1, kEdge = 2 };
    auto tile_mode = [&](int t0) {
        if (t0 + kTileTok > len)
            return (int)kEdge;
        if (fresh && t0 >= base_pos)
            return (int)kFresh;
        if (big_pages && (!fresh || t0 + kTileTok <= base_pos))
            return (int)kCached;
        return (int)kEdge;
    };
    // only a cached tile takes its rows' pages from these ids (the others
    // read none, or look them up per lane)
    auto load_pages = [&](int s, PageIds &pg) {
        const int t0 = tok_tile(s) * kTileTok;
        if (tile_mode(t0) != kCached)
            return;
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            pg[i] = pages_s[min(t0 + RPC * (w4 + 4 * i), len - 1) >> a.page_shift];
    };
    auto issue_kv = [&](int s, const PageIds &pg) {
        const int t0 = tok_tile(s) * kTileTok;
        const uint32_t kdst = ring_lds + slot_of(s) + w4 * 1024;
        const int mode = tile_mode(t0);
        if (mode == kFresh) {
            const char *b = knew_t + (int64_t)t0 * rs_b;
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                copy16_to_lds_s(b + roff[i], kvo[i], kdst + 4096 * i);
                copy16_to_lds_s(b + roff[i] + vnew_b, vvo[i], kdst + Gm::TILE + 4096 * i);
            }
        } else if (mode == kCached) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const char *b = cached_base(pg[i], t0, i);
                copy16_to_lds_s(b, kvo[i], kdst + 4096 * i);
                copy16_to_lds_s(b + hs_b, vvo[i], kdst + Gm::TILE + 4096 * i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                // per lane; past the end the last token again (masked)
                const int tok = min(t0 + RPC * (w4 + 4 * i) + rr, len - 1);
                const uint16_t *kr;
                int64_t vd;
                if (fresh && tok >= base_pos) {
                    kr = reinterpret_cast<const uint16_t *>(knew_t) + (int64_t)tok * a.row_stride;
                    vd = vnew_b / 2;
                } else {
                    kr = a.cache + page_base(pages[tok >> a.page_shift], tok);
                    vd = a.half_stride;
                }
                copy16_to_lds(kr + kel(i), kdst + 4096 * i);
                copy16_to_lds(kr + vd + vel(i), kdst + Gm::TILE + 4096 * i);
            }
        }
    };
    // chain A's second column tile: its q rows through LDS (copied now, read
    // at the switch), rows swizzled like K
    char *qa_lds = smem + 2 * Gm::RING + w4 * (32 * RB);
    const bool a_switch = chain == 0 && nA2 > 0;
    if (a_switch) {
#pragma unroll
        for (int j = 0; j < 32 / RPC; ++j) {
            const int r = RPC * j + rr;
            int row, head;
            column_of(jh, r, row, head);
            copy16_to_lds(a.q + ((int64_t)(r0 + row) * a.num_qo_heads + head) * D +
                              8 * ((lane % CPR) ^ swz_k<D>(r)),
                          (uint32_t)(uintptr_t)qa_lds + j * 1024);
        }
    }
    auto switch_columns = [&]() {
        set_geometry(jh);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int dc = 0; dc < DC; ++dc)
                qb[cb][dc] =
                    flip(*reinterpret_cast<const uint4 *>(qa_lds + 16 * cb * RB + koff(dc)));
    };

    // ---- the work of a token tile, in three parts: its scores (qk, matrix
    // cores), the softmax (vector ALU) and the second product (pv, matrix
    // cores).
    typedef f32x4_t Scores[2][2];   // S^T blocks: tokens 16 tb + MFMA rows, columns of block cb
    typedef bf16x8_t Weights[2];    // P^T operands of the two column blocks
    // (the four accumulators take turns, so no product waits for the one
    // just issued)
    auto qk = [&](int s, Scores &sc) {
        const char *kb = ring + slot_of(s);
        bf16x8_t ka[2][DC];
        // every operand read goes out before the first product, in the order
        // the products take them, so a product waits only for its own reads
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                ka[tb][dc] = as_bf16x8(*reinterpret_cast<const uint4 *>(kb + 16 * tb * RB + koff(dc)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                sc[tb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    sc[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tb][dc], qb[cb][dc],
                                                                         sc[tb][cb], 0, 0, 0);
    };
    // online softmax per column; P^T operands in the token order above.
    // MASK: some token of the tile lies past some column's position.
    using Masked = std::true_type;
    using Plain = std::false_type;
    auto softmax = [&](auto maskc, int t0, const Scores &sc, Weights &phi, Weights &plo) {
        constexpr bool MASK = decltype(maskc)::value;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            bool vis[8];
            float tmax = -__builtin_inff();
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                vis[e] = !MASK || t0 + 16 * (e >> 2) + 4 * q + (e & 3) <= cpos[cb];
                tmax = fmaxf(tmax, vis[e] ? sc[e >> 2][cb][e & 3] : -__builtin_inff());
            }
            // lazy maximum: raised (to the tile's column maximum) only when a
            // score passes it by more than kTau, so weights stay below
            // 2^kTau and most tiles rescale nothing
            const float ts = tmax * c2;
            if (__builtin_amdgcn_ballot_w64(ts > m[cb] + kTau) != 0) {
                const float mn = fmaxf(m[cb], column_max(ts));
                const float alpha = __builtin_amdgcn_exp2f(m[cb] - mn);
                m[cb] = mn;
                lsum[cb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[cb][db] *= alpha;
            }
            const float nm = -m[cb];
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sc[e >> 2][cb][e & 3], c2, nm));
                pv[e] = vis[e] ? p : 0.f;
                lsum[cb] += pv[e];
            }
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                hw[k] = bf16x2_rne(pv[2 * k], pv[2 * k + 1]);
                lw[k] = bf16x2_rne(pv[2 * k] - bf16_lo_up(hw[k]),
                                   pv[2 * k + 1] - bf16_hi_up(hw[k]));
            }
            phi[cb] = __builtin_bit_cast(bf16x8_t, u32x4_t{hw[0], hw[1], hw[2], hw[3]});
            plo[cb] = __builtin_bit_cast(bf16x8_t, u32x4_t{lw[0], lw[1], lw[2], lw[3]});
        }
    };
    // O^T += V^T P^T: lane gets V^T[16 db + c] at tokens 4 q .. 4 q + 3 and
    // 16 + 4 q .. 16 + 4 q + 3.  Two d-blocks at a time: their four high-part
    // products, then the four remainder products (an accumulator's second
    // product three behind its first).
    auto pv = [&](int s, const Weights &phi, const Weights &plo) {
        const char *vb = ring + slot_of(s) + Gm::TILE;
        bf16x8_t va[DB];
        // all operand reads first (as in qk)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t *)(vb + voff(db)));
            const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t *)(vb + voff(db) + 16 * RB));
            va[db] = __builtin_bit_cast(
                bf16x8_t,
                u32x4_t{__builtin_bit_cast(uint2, v0).x, __builtin_bit_cast(uint2, v0).y,
                        __builtin_bit_cast(uint2, v1).x, __builtin_bit_cast(uint2, v1).y});
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; db += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    o[cb][db + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db + u], phi[cb],
                                                                            o[cb][db + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    o[cb][db + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db + u], plo[cb],
                                                                            o[cb][db + u], 0, 0, 0);
        }
    };
    auto visible = [&](int s) { return tok_tile(s) * kTileTok <= wmax; };
    auto masked = [&](int s) { return tok_tile(s) * kTileTok + kTileTok - 1 > wmin; };

    // ---- the walk: one barrier per step.  At step s a wave waits for its
    // chain's tile s (the copies issued after it, one step's, may still be
    // outstanding), then meets the barrier, after which tile s is in LDS for
    // every wave and no wave still reads tile s - 1, whose slot takes the
    // copies of tile s + 2; then it runs qk, softmax and pv of tile s.  The
    // vector and matrix work of the two waves on a SIMD interleave as they
    // come: on gfx950 the matrix products of one wave hide little of the
    // other's vector work, so a fixed alternation between them would buy
    // nothing and cost a second barrier per step.  The append's loads go out
    // before every copy; its stores, at step 1, only make later waits longer.
    // The append: the workgroups of an (entry, KV head) share its new rows,
    // up to four 16-byte chunks per thread; the loads go out before the
    // walk's copies and the stores early in the walk.
    const bool append = a.cache_w != nullptr;
    const int share = (T + 1) / 2;
    const int j0 = (int)((int64_t)nc * kk / share), j1 = (int)((int64_t)nc * (kk + 1) / share);
    const int jobs = append ? (j1 - j0) * 2 * CPR : 0;
    // job: chunk job % CPR of the K (or V) row of new row j0 + job / (2 CPR);
    // past the last job the last job's source is read again (a plain load)
    auto job_src = [&](int job) {
        job = min(job, jobs - 1);
        const int row = j0 + job / (2 * CPR);
        const int is_v = (job / CPR) & 1, ch = job % CPR;
        return reinterpret_cast<const uint4 *>((is_v ? a.v_new : a.k_new) +
                                               (int64_t)(r0 + row) * a.row_stride + h * D) + ch;
    };
    auto job_page = [&](int job) {
        job = min(job, jobs - 1);
        return pages[(base_pos + j0 + job / (2 * CPR)) >> a.page_shift];
    };
    auto job_store = [&](int job, int page, uint4 v) {
        if (job >= jobs || (uint32_t)page >= (uint32_t)a.num_pages)
            return;   // no job, or a bad page id
        const int row = j0 + job / (2 * CPR);
        const int is_v = (job / CPR) & 1, ch = job % CPR;
        const int tok = base_pos + row;
        *reinterpret_cast<uint4 *>(a.cache_w + (int64_t)page * a.page_stride +
                                   (is_v ? a.half_stride : 0) +
                                   (int64_t)(tok & pmask) * a.row_stride + h * D + 8 * ch) = v;
    };
    uint4 av0, av1, av2, av3;
    int ap0 = -1, ap1 = -1, ap2 = -1, ap3 = -1;
    if (jobs > 0) {
        av0 = *job_src(tid);
        av1 = *job_src(tid + kThreads);
        av2 = *job_src(tid + 2 * kThreads);
        av3 = *job_src(tid + 3 * kThreads);
        ap0 = job_page(tid);
        ap1 = job_page(tid + kThreads);
        ap2 = job_page(tid + 2 * kThreads);
        ap3 = job_page(tid + 3 * kThreads);
    }

    PageIds pg0 = {}, pg1 = {}, pg2 = {};   // page ids of steps s, s + 1, s + 2
    if (0 < my_len)
        load_pages(0, pg0);
    if (1 < my_len)
        load_pages(1, pg1);
    if (2 < my_len)
        load_pages(2, pg2);
    if (0 < my_len)
        issue_kv(0, pg0);
    if (1 < my_len)
        issue_kv(1, pg1);
    auto wait_rows = [&](bool later_copies) {
        // no more outstanding than the copies issued after the rows wanted
        if (later_copies)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * CPW));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    };
    // copies of step s + 2, the page ids of step s + 3
    auto issue_step = [&](int s) {
        if (s + 2 < my_len)
            issue_kv(s + 2, pg2);
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            pg0[i] = pg1[i];
            pg1[i] = pg2[i];
        }
        if (s + 3 < my_len)
            load_pages(s + 3, pg2);
    };
    auto softmax_step = [&](int s, const Scores &sc, Weights &phi, Weights &plo) {
        if (!visible(s))
            return;
        const int t0 = tok_tile(s) * kTileTok;
        if (masked(s))
            softmax(Masked{}, t0, sc, phi, plo);
        else
            softmax(Plain{}, t0, sc, phi, plo);
    };
    const int steps = max(lenA, nB);   // steps of the longer chain
    // the append's stores go out at step 1 (by every wave), to run under the
    // rest of the walk: the compiler waits there for their loads, which
    // drains the copies then in flight once
    auto append_stores = [&]() {
        job_store(tid, ap0, av0);
        job_store(tid + kThreads, ap1, av1);
        job_store(tid + 2 * kThreads, ap2, av2);
        job_store(tid + 3 * kThreads, ap3, av3);
        for (int job = tid + 4 * kThreads; job < jobs; job += kThreads)
            job_store(job, job_page(job), *job_src(job));
    };
    for (int s = 0; s < steps; ++s) {
        if (s < my_len)
            wait_rows(s + 1 < my_len);   // tile s
        __syncthreads();
        if (s == 1)
            append_stores();
        if (s < my_len) {
            issue_step(s);
            if (visible(s)) {
                Scores sc;
                Weights phi, plo;
                qk(s, sc);
                softmax_step(s, sc, phi, plo);
                pv(s, phi, plo);
            }
            if (a_switch && s + 1 == nA1) {
                // chain A moves from its own column tile to the pair's other one
                finalize();
                switch_columns();
            }
        }
    }
    __syncthreads();

    if (steps < 2)
        append_stores();

    if (!merge) {
        if (my_len > 0)
            finalize();
        return;
    }
    // chain A's partials through LDS, lane for lane: o, then (m, lsum)
    f32x4_t *part = reinterpret_cast<f32x4_t *>(smem) + w4 * Gm::MQ * 64 + lane;
    if (chain == 0) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                part[(cb * DB + db) * 64] = o[cb][db];
        part[2 * DB * 64] = f32x4_t{m[0], m[1], lsum[0], lsum[1]};
    }
    __syncthreads();
    if (chain == 0)
        return;
    const f32x4_t ml = part[2 * DB * 64];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const float ma = ml[cb], la = ml[2 + cb];
        const float mn = fmaxf(ma, m[cb]);
        const float sa = __builtin_amdgcn_exp2f(ma - mn), sb = __builtin_amdgcn_exp2f(m[cb] - mn);
        m[cb] = mn;
        lsum[cb] = la * sa + lsum[cb] * sb;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            o[cb][db] = part[(cb * DB + db) * 64] * sa + o[cb][db] * sb;
    }
    finalize();
}

// A workgroup per (entry, KV head, pair k): blocks congruent mod 8 share an
// XCD, and each XCD takes a contiguous run of the linear order.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
    const int nb = gridDim.x;
    const int xcd = blockIdx.x & 7;
    const int lin = xcd * (nb >> 3) + min(xcd, nb & 7) + (blockIdx.x >> 3);
    const int pair = lin / a.pair_tiles;
    const int kk = lin - pair * a.pair_tiles;
    const int b = pair / a.num_kv_heads;
    tile_pair<D>(a, b, pair - b * a.num_kv_heads, kk);
}

// Mixed step: only the entries the plan listed (those with several new
// rows), so the decode rows cost no workgroups.  A grid of whole XCD rounds
// walks the items: (entry, KV head) unit u goes to XCD u % 8, its pairs one
// after another on that XCD (they share the unit's keys and values in its
// L2).  A list of another plan (its signature differs) computes nothing.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_list_kernel(PrefillArgs a) {
    const int32_t *list = a.list;
    if (list[0] != a.list_sig)
        return;
    const int count = list[1];
    if (count < 0 || count > a.list_cap)
        return;
    const int64_t units = (int64_t)count * a.num_kv_heads;
    const int x = blockIdx.x & 7;
    for (int64_t j = blockIdx.x >> 3;; j += gridDim.x >> 3) {
        const int64_t grp = j / a.pair_tiles;
        const int64_t u = 8 * grp + x;
        if (u >= units)
            break;   // later items of this workgroup lie further on
        const int e = (int)(u / a.num_kv_heads);
        const int b = list[2 + e];
        if ((unsigned)b < (unsigned)a.batch)
            tile_pair<D>(a, b, (int)(u - (int64_t)e * a.num_kv_heads),
                         (int)(j - grp * a.pair_tiles));
        // the next item reuses the LDS: every copy has landed and every wave
        // has read its last operands
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
    }
}

}  // namespace

bool prefill_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    if (!prefill_supported(a.head_dim) || a.batch > 65535 || a.num_kv_heads > 65535 ||
        a.pair_tiles < 1)
        return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)a.pair_tiles * a.batch * a.num_kv_heads;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidValue;
    PrefillArgs args = a;
    void *params[] = {&args};
    if (a.list != nullptr) {
        // one workgroup per compute unit (the LDS holds one), whole XCD rounds
        int cus = 0;
        const hipError_t err = compute_units(&cus);
        if (err != hipSuccess)
            return err;
        const unsigned grid = cus >= 16 ? (unsigned)(cus & ~7) : 8u;
        const void *k = a.head_dim == 128
                            ? reinterpret_cast<const void *>(&prefill_list_kernel<128>)
                            : reinterpret_cast<const void *>(&prefill_list_kernel<64>);
        return hipLaunchKernel(k, dim3(grid), dim3(kThreads), params, 0, stream);
    }
    const void *k = a.head_dim == 128 ? reinterpret_cast<const void *>(&prefill_kernel<128>)
                                      : reinterpret_cast<const void *>(&prefill_kernel<64>);
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(kThreads), params, 0, stream);
}

}  // namespace pkv
