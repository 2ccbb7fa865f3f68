// pkv_kernels.hip -- gfx950 kernels for paged-KV append and decode attention.
//
// What is computed is fixed by the vox-serve "Adding a Model" page (section 1,
// "The model code": the cache [layers, pages, 2, page_size, kv_heads,
// head_dim], set_kv_cache and run; "How a program runs": per-step page
// tables, padding entries on scratch page 0).  How it is computed here is an
// MI355X design:
//
//  * Decode streams K/V once from HBM and is bandwidth-bound (about g flops
//    per byte for a GQA group of g query heads), so it uses the vector ALUs,
//    not MFMA.  q.k runs on v_dot2_f32_bf16 straight from the bf16 words: no
//    conversion of K, exact products, fp32 accumulation.
//  * A workgroup has one wavefront per KV head of its head group.  Each 8-token
//    tile's K rows and V rows of all those heads are copied from HBM into LDS
//    with direct-to-LDS loads, 1 KiB of one contiguous run per instruction,
//    through a ring of buffers a few tiles deep; every wave then reads its own
//    head's rows.
//  * A token row of a head is spread over 8 (or 16) lanes; row sums are DPP
//    row operations, row groups are combined with the gfx950 cross-row lane
//    swaps (v_permlane16_swap, v_permlane32_swap).
//  * The running maximum is raised only when a score passes it by more than
//    kTau (log2 units); between raises nothing is rescaled.
//
// Work split.  The plan kernel walks the page table once per step (the table
// is the same for every layer) and writes, per decode workgroup, the records
// of its tiles.  Balanced mode (default): the work of all entries is laid end
// to end (tiles, plus a fixed cost per entry for starting and ending it) and
// each of W workgroups (W = what the chip holds at once) takes an equal run
// of it; runs of neighbouring workgroup ids sit on different XCDs, so the
// plan deals consecutive runs to one XCD.  Fixed mode: each entry is cut into
// chunks of a fixed number of tiles, one workgroup each, so how an entry is
// split depends only on its own length and its rows are bit-identical in any
// batch.  An entry covered by several workgroups gets one partial (output,
// lse) per segment; the wave that finishes last merges them by log-sum-exp
// (an agent-scope counter per entry and head decides which), so no second
// launch is needed.
//
// The fused append (k_new != null) treats the tile holding token L-1 of each
// entry specially: that row is read from k_new/v_new and written into the
// cache by the one wave that processes it, which is append followed by decode
// without a second pass over memory.
//
// All cache offsets are 64-bit.  Page ids outside [0, num_pages) are read as
// scratch page 0, and an append with an out-of-range page or slot writes
// nothing: a malformed table can give wrong rows but never a fault.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kTau = 8.0f;        // lazy-rescale threshold, log2 units
constexpr float kMInit = -1.0e30f;  // running maximum before any score: finite, so
                                    // exp2(-inf - kMInit) is 0, never NaN

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Exact bf16 -> fp32 of the low / high half of a 32-bit word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __uint_as_float(w & 0xffff0000u);
}

// fp32 -> bf16 (round to nearest even), two values packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    uint32_t a = __builtin_bit_cast(uint16_t, static_cast<__bf16>(lo));
    uint32_t b = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hi));
    return a | (b << 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the LPR (8 or 16) lanes of an aligned row; every lane gets the total.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp<0x141>(x);   // row_half_mirror: lane i <-> 7 - i within 8
    if constexpr (LPR == 16)
        x += dpp<0x140>(x);   // row_mirror: lane i <-> 15 - i within 16
    return x;
}

// Both halves of a cross-row lane swap of x with itself.
__device__ __forceinline__ void swap16(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Max / sum over the RG row groups of a wave (lanes with equal lane % (64/RG));
// every lane gets the result.
template <int RG>
__device__ __forceinline__ float group_max(float x) {
    float a, b;
    if constexpr (RG == 8)
        x = fmaxf(x, dpp<0x128>(x));   // row_ror:8 = lane ^ 8 within 16
    swap16(x, a, b);
    x = fmaxf(a, b);
    swap32(x, a, b);
    return fmaxf(a, b);
}
template <int RG>
__device__ __forceinline__ float group_sum(float x) {
    float a, b;
    if constexpr (RG == 8)
        x += dpp<0x128>(x);
    swap16(x, a, b);
    x = a + b;
    swap32(x, a, b);
    return a + b;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Partial rows cross workgroups (and XCDs, whose L2s are not coherent with
// each other).  They are written and read through a buffer resource with the
// device-scope cache policy (sc1): stores write through to the coherent
// level and loads read from it, so no L2-wide writeback or invalidate is
// needed around the arrival counter.  The resource's range also bounds every
// access to the partial arrays.
//
// A partial is stored compactly: its normalized outputs in fp16, scaled by a
// power of two 2^-s chosen per (segment, KV head) so that the largest
// magnitude is below 1 (no overflow for any finite input, 11 significant
// bits), and per query head the pair {lse (base 2), s}.
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
constexpr int kPolicyDevice = 16;   // sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const void *base,
                                                               int64_t bytes) {
    const int range = bytes < 0x7fffffff ? (int)bytes : 0x7fffffff;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, range,
                                             0x00020000);
}
__device__ __forceinline__ void store_b128_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                    uint4 v) {
    const v4i_t x = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)off, 0, kPolicyDevice);
}
__device__ __forceinline__ void store_b64_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   uint32_t a, uint32_t b) {
    const v2i_t x = {(int)a, (int)b};
    __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)off, 0, kPolicyDevice);
}
__device__ __forceinline__ void store_b32_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   uint32_t a) {
    __builtin_amdgcn_raw_buffer_store_b32((int)a, r, (int)off, 0, kPolicyDevice);
}
__device__ __forceinline__ void store_b16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   uint16_t a) {
    __builtin_amdgcn_raw_buffer_store_b16((short)a, r, (int)off, 0, kPolicyDevice);
}
__device__ __forceinline__ uint4 load_b128_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v4i_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyDevice);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
__device__ __forceinline__ float2 load_f2_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v2i_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyDevice);
    return make_float2(__int_as_float(v.x), __int_as_float(v.y));
}

// Adds 1 to *p at device scope and returns the old value in `old`, without the
// compiler tracking it: the caller reads `old` only after its own wait for all
// vector memory operations (a compiler-visible atomic whose result is used
// later would make the compiler wait for every outstanding copy right away).
__device__ __forceinline__ void atomic_inc_untracked(int32_t *p, int &old) {
    asm volatile("global_atomic_add %0, %1, %2, off sc0" : "+v"(old) : "v"(p), "v"(1)
                 : "memory");
}

// fp32 -> fp16 (round to nearest even), two values packed low-first, and back.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

__device__ __forceinline__ uint4 load16(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void store16(uint16_t *p, uint4 v) {
    *reinterpret_cast<uint4 *>(p) = v;
}

// ---------------------------------------------------------------------------
// Standalone append: one workgroup per entry copies its K row then its V row,
// 16 bytes a thread.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const int b = blockIdx.x;
    const int end = a.indptr[b + 1];
    if (end - a.indptr[b] < 1)
        return;
    const int page = a.indices[end - 1];
    const int slot = a.last_len[b] - 1;
    if (page < 0 || page >= a.num_pages || slot < 0 || slot >= a.page_size)
        return;
    uint16_t *dst = a.cache + (int64_t)page * a.page_stride + (int64_t)slot * a.row_elems;
    const uint16_t *ks = a.k_new + (int64_t)b * a.row_elems;
    const uint16_t *vs = a.v_new + (int64_t)b * a.row_elems;
    const int words = a.row_elems >> 3;   // 16-byte words per row
    for (int i = threadIdx.x; i < 2 * words; i += blockDim.x) {
        const bool is_v = i >= words;
        const int w = is_v ? i - words : i;
        const uint4 val = reinterpret_cast<const uint4 *>(is_v ? vs : ks)[w];
        reinterpret_cast<uint4 *>(dst + (is_v ? a.half_stride : 0))[w] = val;
    }
}

// ---------------------------------------------------------------------------
// Plan.

// Exclusive scan of one int per thread over the workgroup (<= 16 waves).
__device__ int block_exclusive_scan(int v, int *s_wave, int &total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = (blockDim.x + 63) >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d)
            x += y;
    }
    if (lane == 63)
        s_wave[wave] = x;
    __syncthreads();
    if (threadIdx.x < 64) {
        const int w = lane < nwaves ? s_wave[lane] : 0;
        int sc = w;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(sc, d, 64);
            if (lane >= d)
                sc += y;
        }
        if (lane < nwaves)
            s_wave[lane] = sc - w;     // exclusive prefix of wave totals
        if (lane == nwaves - 1)
            s_wave[16] = sc;           // grand total
    }
    __syncthreads();
    total = s_wave[16];
    return s_wave[wave] + x - v;
}

struct EntryShape {
    int p0;     // first page-table slot
    int n;      // pages listed
    int last;   // rows in the last page, clamped to [1, page_size]
    int tiles;  // tiles the decode covers (0: none, or over the page bound)
};

// The shape of planned entry b: with a row -> entry map (a mixed step), b is
// a row and the shape that of the entry whose single row it is, or empty.
__device__ __forceinline__ EntryShape entry_shape(const PlanArgs &a, const int *rowent, int b) {
    EntryShape e;
    if (rowent != nullptr) {
        b = rowent[b];
        if (b < 0) {
            e.p0 = 0;
            e.n = 0;
            e.last = 1;
            e.tiles = 0;
            return e;
        }
    }
    e.p0 = a.indptr[b];
    e.n = a.indptr[b + 1] - e.p0;
    int last = a.last_len[b];
    e.last = last < 1 ? 1 : (last > a.page_size ? a.page_size : last);
    e.tiles = (e.n < 1 || e.n > a.max_pages)
                  ? 0
                  : (e.n - 1) * a.tiles_per_page + (e.last + kTileTokens - 1) / kTileTokens;
    return e;
}

__device__ __forceinline__ int valid_page(const PlanArgs &a, int page) {
    return (page >= 0 && page < a.num_pages) ? page : 0;
}

// The largest e in [0, hi] with start[e] <= t (start non-decreasing).
__device__ __forceinline__ int entry_of(const int *start, int hi, int64_t t) {
    int lo = 0;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Balanced mode: run index of workgroup id w of W for R <= W runs (R when
// it has none).  Workgroups are dealt to the 8 XCDs round-robin, so ids w,
// w + 8, ... share an XCD; XCD x takes runs [R x / 8, R (x + 1) / 8) on
// consecutive ids, which keeps an entry's pieces (and its q rows and
// partials) within one XCD's L2 as far as possible, and spreads fewer runs
// than workgroups over all XCDs and their CUs.
__device__ __forceinline__ int run_of_block(int w, int W, int R) {
    if (W % 8 != 0)
        return w < R ? w : R;
    const int x = w % 8, i = w / 8;
    const int r0 = (int)((int64_t)R * x / 8), r1 = (int)((int64_t)R * (x + 1) / 8);
    return r0 + i < r1 ? r0 + i : R;
}

// Balanced mode splits cost, not tiles.  Every entry's tiles are laid end to
// end on a cost axis: the entry first takes kEntryCost units for the work of
// starting and ending a segment (q rows, the first tile's rescale, the merge
// of row groups and the stores), then kTileCost units per tile; the axis of
// total length C is cut into W_eff runs [C r / W_eff, C (r+1) / W_eff), and a
// tile belongs to the run holding its start.  Short entries thus count for
// more than their tiles, and a run of several entries gets fewer tiles.

struct CostAxis {
    const int *start;   // [batch + 1] tile prefix sums
    const int *nz;      // [batch + 1] prefix counts of entries with tiles
    int batch;
    int64_t T, C, weff;
    // cost position where entry b begins
    __device__ int64_t entry_pos(int b) const {
        return kTileCost * (int64_t)start[b] + kEntryCost * (int64_t)nz[b];
    }
    // start position of tile i of entry b
    __device__ int64_t tile_pos(int b, int64_t i) const {
        return entry_pos(b) + kEntryCost + kTileCost * i;
    }
    // run holding position p: the largest r with floor(C r / W_eff) <= p
    __device__ int run_of(int64_t p) const { return (int)(((p + 1) * weff - 1) / C); }
    // number of tiles (of all entries) that start before position x
    __device__ int64_t tiles_before(int64_t x) const {
        if (x >= C)
            return T;
        int lo = 0, hi = batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (entry_pos(mid) <= x)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int64_t in = x - entry_pos(lo) - kEntryCost;
        const int64_t i = in <= 0 ? 0 : (in + kTileCost - 1) / kTileCost;
        const int64_t nt = start[lo + 1] - start[lo];
        return start[lo] + (i < nt ? i : nt);
    }
};

// Fixed mode deals whole chunks (runs of chunk_tiles tiles of one entry; an
// entry's last chunk may be shorter) to the W resident workgroups.  Chunks
// are ranked largest first: the F full chunks in entry order, then the P
// shorter last chunks by decreasing size (ties, and every partial chunk of a
// batch above kRankedBatch, in entry order).  Rank r goes to workgroup
// r mod W in round r / W, the rounds alternating direction (a snake), so
// workgroup w holds ranks k W + w for even k and k W + W - 1 - w for odd k:
// with the larger chunks dealt first, the workgroups that drew smaller ones
// draw next, close to a longest-first assignment.  Which workgroup computes a
// chunk never changes its bits: a chunk's partial, and the merge of an
// entry's chunks (in chunk order), depend only on the entry.
struct FixedChunks {
    const int *full;    // [batch + 1] prefix sums of full chunks per entry
    const int *pent;    // [P] entry of the partial chunk of each rank
    const int *psz;     // [P] its tiles
    int batch, ct, W;
    int F, P;
    __device__ int rank_of(int w, int k) const {
        return k * W + ((k & 1) ? W - 1 - w : w);
    }
    // entry b, chunk index c and tiles of the chunk of rank r (< F + P)
    __device__ void chunk(int r, int &b, int &c, int &tiles) const {
        if (r < F) {
            b = entry_of(full, batch - 1, r);
            c = r - full[b];
            tiles = ct;
        } else {
            b = pent[r - F];
            c = full[b + 1] - full[b];
            tiles = psz[r - F];
        }
    }
};

__global__ __launch_bounds__(256) void plan_kernel(PlanArgs a) {
    // balanced: [batch + 1] tile prefix sums, then [batch + 1] prefix counts
    // of entries with tiles
    extern __shared__ int s_start[];
    __shared__ int s_wave[17];
    const bool fixed = a.chunk_tiles > 0;
    int *s_nz = s_start + a.batch + 1;
    // mixed step: the row -> entry map after the arrays below
    int *s_rowent = nullptr;
    if (a.qo_indptr != nullptr) {
        // past the arrays plan_lds_bytes sizes for the plain plan
        s_rowent = s_start + (fixed ? 3 * a.batch + 1 + (a.batch <= kRankedBatch ? a.batch : 0)
                                    : 2 * (a.batch + 1));
        for (int r = threadIdx.x; r < a.batch; r += blockDim.x)
            s_rowent[r] = -1;
        __syncthreads();
        for (int b = threadIdx.x; b < a.num_entries; b += blockDim.x) {
            const int r0 = a.qo_indptr[b];
            if (a.qo_indptr[b + 1] - r0 == 1 && (unsigned)r0 < (unsigned)a.batch)
                s_rowent[r0] = b;
        }
        __syncthreads();
        if (blockIdx.x == 0) {
            // the prefill's list: entries with several new rows, in order
            const int per = (a.num_entries + blockDim.x - 1) / blockDim.x;
            const int e0 = min(a.num_entries, (int)threadIdx.x * per);
            const int e1 = min(a.num_entries, e0 + per);
            int local = 0;
            for (int b = e0; b < e1; ++b)
                local += a.qo_indptr[b + 1] - a.qo_indptr[b] > 1;
            int total = 0;
            int at = block_exclusive_scan(local, s_wave, total);
            for (int b = e0; b < e1; ++b)
                if (a.qo_indptr[b + 1] - a.qo_indptr[b] > 1) {
                    if (at < a.list_cap)
                        a.list[2 + at] = b;
                    ++at;
                }
            if (threadIdx.x == 0) {
                a.list[0] = a.plan_sig;
                a.list[1] = min(total, a.list_cap);
            }
            __syncthreads();   // s_wave is reused
        }
    }
    int64_t T = 0;
    const int W = a.num_blocks;
    CostAxis ax{s_start, s_nz, a.batch, 0, 0, 1};
    if (!fixed) {
        const int nthreads = blockDim.x;
        const int per = (a.batch + nthreads - 1) / nthreads;
        const int e0 = min(a.batch, (int)threadIdx.x * per);
        const int e1 = min(a.batch, e0 + per);
        int local = 0, localz = 0;
        for (int e = e0; e < e1; ++e) {
            const int t = entry_shape(a, s_rowent, e).tiles;
            s_start[e] = t;
            local += t;
            localz += t > 0;
        }
        int total = 0, totalz = 0;
        int run = block_exclusive_scan(local, s_wave, total);
        __syncthreads();   // s_wave is reused
        int runz = block_exclusive_scan(localz, s_wave, totalz);
        for (int e = e0; e < e1; ++e) {
            const int t = s_start[e];
            s_start[e] = run;
            s_nz[e] = runz;
            run += t;
            runz += t > 0;
        }
        if (threadIdx.x == 0) {
            s_start[a.batch] = total;
            s_nz[a.batch] = totalz;
        }
        __syncthreads();
        T = total;
        ax.T = T;
        ax.C = kTileCost * (int64_t)total + kEntryCost * (int64_t)totalz;
        // runs no shorter than kMinRunTiles tiles: a shorter run costs more
        // in its start, its partial and the merge than its tiles take (and
        // no run inside an entry's tiles is empty)
        const int64_t cap = ax.C / (kTileCost * kMinRunTiles);
        ax.weff = cap < 1 ? 1 : (cap < W ? cap : W);
    }
    FixedChunks fc{s_start, s_nz, s_nz + a.batch, a.batch, a.chunk_tiles, W, 0, 0};
    if (fixed) {
        // [batch + 1] full-chunk prefix sums, then [batch] entries and
        // [batch] sizes of the partial chunks by rank; for ranking, the
        // partial size of every entry (or 0) in a further [batch] array
        int *s_pent = s_nz, *s_psz = s_nz + a.batch, *s_pse = s_nz + 2 * a.batch;
        const int ranked = a.batch <= kRankedBatch;
        const int nthreads = blockDim.x;
        const int per = (a.batch + nthreads - 1) / nthreads;
        const int e0 = min(a.batch, (int)threadIdx.x * per);
        const int e1 = min(a.batch, e0 + per);
        int local = 0, localp = 0;
        for (int e = e0; e < e1; ++e) {
            const int t = entry_shape(a, s_rowent, e).tiles;
            const int fl = t / a.chunk_tiles, ps = t - fl * a.chunk_tiles;
            s_start[e] = fl;
            if (ranked)
                s_pse[e] = ps;
            local += fl;
            localp += ps > 0;
        }
        int totf = 0, totp = 0;
        int run = block_exclusive_scan(local, s_wave, totf);
        __syncthreads();   // s_wave is reused
        int runp = block_exclusive_scan(localp, s_wave, totp);
        for (int e = e0; e < e1; ++e) {
            const int fl = s_start[e];
            s_start[e] = run;
            run += fl;
        }
        if (threadIdx.x == 0)
            s_start[a.batch] = totf;
        __syncthreads();
        for (int e = e0; e < e1; ++e) {
            const int t = entry_shape(a, s_rowent, e).tiles;
            const int ps = t - (s_start[e + 1] - s_start[e]) * a.chunk_tiles;
            if (ps <= 0)
                continue;
            int q = runp++;   // entry order
            if (ranked) {
                // larger partial chunks first, ties in entry order
                q = 0;
                for (int f = 0; f < a.batch; ++f) {
                    const int pf = s_pse[f];
                    q += pf > ps || (pf == ps && f < e);
                }
            }
            s_pent[q] = e;
            s_psz[q] = ps;
        }
        __syncthreads();
        fc.F = totf;
        fc.P = totp;
    }
    const int64_t weff = fixed ? W : ax.weff;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    int4 *blocks = reinterpret_cast<int4 *>(a.blocks);
    int4 *ent = reinterpret_cast<int4 *>(a.ent);

    for (int64_t i = tid; i < (int64_t)a.batch * a.num_kv_heads; i += nth)
        a.cnt[i] = 0;

    for (int64_t bb = tid; bb < a.batch; bb += nth) {
        const int b = (int)bb;
        const EntryShape e = entry_shape(a, s_rowent, b);
        int4 d = make_int4(0, 0, 0, 0);
        if (e.n > a.max_pages) {
            // over the bound: no tiles; the decode writes NaN rows and, when
            // fused, still appends the new row to its slot
            d = make_int4(0, -1, valid_page(a, a.indices[e.p0 + e.n - 1]), e.last - 1);
        } else if (e.tiles > 0) {
            if (fixed) {
                d.x = b * a.max_chunks;
                d.y = (e.tiles + a.chunk_tiles - 1) / a.chunk_tiles;
            } else {
                const int first = ax.run_of(ax.tile_pos(b, 0));
                d.x = first + b;
                d.y = ax.run_of(ax.tile_pos(b, e.tiles - 1)) - first + 1;
            }
        }
        ent[b] = d;
    }

    const int64_t items = (int64_t)W * a.block_stride;
    for (int64_t i = tid; i < items; i += nth) {
        const int w = (int)(i / a.block_stride);
        const int jj = (int)(i - (int64_t)w * a.block_stride);
        int b = 0, run = 0, ntiles = 0, nseg = 1, slot = 0;
        int64_t g0 = 0, g1 = 0, s0 = 0;
        EntryShape e{};
        int kc = 0, ct0 = 0, ctiles = 0;   // fixed: the chunk holding record jj - 1
        if (fixed) {
            // walk this workgroup's chunks (ranks in dealing order) to the one
            // holding record jj - 1 (the header, jj 0, sums them all)
            run = w;
            const int T = fc.F + fc.P;
            for (int k = 0;; ++k) {
                const int r = fc.rank_of(w, k);
                if (r >= T)
                    break;
                int cb, cc, csz;
                fc.chunk(r, cb, cc, csz);
                if (jj > 0 && jj - 1 < ntiles + csz) {
                    b = cb;
                    kc = cc;
                    ct0 = ntiles;
                    ctiles = csz;
                    ntiles += csz;
                    break;
                }
                ntiles += csz;
            }
            if (jj > 0 && ctiles == 0)
                continue;   // capacity this block does not use; never read
        } else {
            run = run_of_block(w, W, (int)weff);
            if (run < weff) {
                g0 = ax.tiles_before(ax.C * run / weff);
                g1 = ax.tiles_before(ax.C * (run + 1) / weff);
                ntiles = (int)(g1 - g0);
            }
        }
        if (jj == 0) {
            blocks[i] = make_int4(ntiles, run, a.plan_sig, 0);
            continue;
        }
        const int k = jj - 1;
        if (k >= ntiles)
            continue;   // capacity this block does not use; never read
        int lt;
        bool seg_first, seg_last;
        if (fixed) {
            const int t = k - ct0;   // tile within the chunk
            e = entry_shape(a, s_rowent, b);
            lt = kc * a.chunk_tiles + t;
            seg_first = t == 0;
            seg_last = t == ctiles - 1;
            nseg = (e.tiles + a.chunk_tiles - 1) / a.chunk_tiles;
            slot = b * a.max_chunks + kc;
        } else {
            const int64_t gk = g0 + k;
            b = entry_of(s_start, a.batch - 1, gk);
            e = entry_shape(a, s_rowent, b);
            s0 = s_start[b];
            lt = (int)(gk - s0);
            seg_first = gk == (g0 > s0 ? g0 : s0);
            const int64_t s1 = s0 + e.tiles;
            seg_last = gk == (g1 < s1 ? g1 : s1) - 1;
            nseg = ax.run_of(ax.tile_pos(b, e.tiles - 1)) - ax.run_of(ax.tile_pos(b, 0)) + 1;
            slot = run + b;
        }
        const int pl = lt / a.tiles_per_page;
        const int sub = lt - pl * a.tiles_per_page;
        const int page = valid_page(a, a.indices[e.p0 + pl]);
        const bool last_page = pl == e.n - 1;
        const int rows = last_page ? e.last : a.page_size;
        const int slot0 = sub * kTileTokens;
        const int ntok = min(kTileTokens, rows - slot0);
        int info = (ntok - 1) | (slot0 << kInfoSlotShift);
        if (seg_first)
            info |= kInfoSegFirst;
        if (seg_last)
            info |= kInfoSegLast;
        if (nseg == 1)
            info |= kInfoSegWhole;
        if (last_page && sub == (e.last - 1) / kTileTokens)
            info |= kInfoHasNew | (((e.last - 1) & (kTileTokens - 1)) << kInfoNewRowShift);
        blocks[i] = make_int4(page, info, b, slot);
    }
}

// ---------------------------------------------------------------------------
// Decode.
//
// Tiles are staged through LDS.  A workgroup has one wave per KV head of its
// head group, and all its waves walk the same tiles.  For each 8-token tile a
// wave copies its own head's K rows and V rows from HBM into its own region
// of an LDS buffer with direct-to-LDS loads (global_load_lds_dwordx4, 1 KiB
// per instruction: 4 rows of 256 B at D = 128), so no registers hold data in
// flight; together the waves read every 16 KiB run of a tile's K (and V)
// rows at about the same time.  A ring of NBUF buffers keeps NBUF tiles in
// flight per wave while it waits: the buffer a wave has just computed is
// refilled at once with the tile NBUF ahead.  No LDS data is shared between
// waves, so there is no barrier: each wave waits for its own copies only and
// issues its next copies before anything waits for a
// slower wave (a barrier per tile ahead of the copies made every wave's next
// copies wait for the slowest wave's compute, which cost about a tenth of the
// streaming rate; the waves now meet only every kSyncTiles tiles, after
// their copies are out).
// The loads are non-temporal: the stream is read once, and it leaves the
// L2 to what is reused.  The q rows of a segment's entry travel the same
// way, in the wave's slot of the tile where the segment starts.
//
// The copies are written as inline assembly, so the compiler does not track
// them; the kernel waits for them itself.  Vector memory operations of a wave
// complete in issue order, so a tile has landed once no more are outstanding
// than were issued after its copies: the copies of later tiles and their q
// rows, and the output, partial and append stores of the tiles computed
// since.  The kernel counts all of them (stores as a lower bound: a count too
// low only waits longer) and waits for exactly that many.
//
// Lane layout in compute.  A row of the tile (one token of one head, D
// elements) is spread over LPR lanes, 8 for G <= 4 query heads per KV head
// and 16 for more (D = 128), so the wave holds RG = 64 / LPR rows at a time
// and each lane RPL = 8 / RG rows of a tile.  Lane = r * LPR + j holds rows
// r + RG i and, of each, the 8-element chunks j + LPR c (c < NC =
// D / (8 LPR)) of K and of V: the LPR lanes of a row read 16 * LPR
// contiguous bytes, so the LDS reads are conflict-free.  A row's score is
// summed over its lanes in DPP steps.  The lane accumulates the G query
// heads' outputs of its elements over its rows.  The running maximum of a
// query head is the same in all row groups (when a raise is due it is taken
// over the whole tile), so at the end of a segment the row groups' sums are
// simply added, by a reduce-scatter that leaves each lane a distinct share of
// the G x D outputs to write.  Eight lanes per row halve the DPP steps and
// the exponentials of sixteen; sixteen keep the accumulators of G > 4 heads
// within the registers of two waves per SIMD.

// s_waitcnt immediate for "at most n vector memory operations outstanding"
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at
// their maximum, i.e. not waited for).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kMaxVmWait = 24;   // largest wait count the decode loop uses
// Two waves of a workgroup share each SIMD, and the older one wins the issue
// arbitration: left alone, the younger waves fall about an eighth behind and
// the workgroup ends with its slowest wave.  A barrier every kSyncTiles tiles,
// placed after the wave has issued its next copies (so no copy waits for it),
// keeps the waves within a few tiles of each other.
constexpr int kSyncTiles = 4;

// s_waitcnt vmcnt(min(n, N)) for a wave-uniform n >= 0 (the immediate must be
// a constant: a chain of scalar compares picks it).
template <int N>
__device__ __forceinline__ void wait_vm_at_most(int n) {
    if constexpr (N == 0) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
        if (n >= N)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
        else
            wait_vm_at_most<N - 1>(n);
    }
}

// One direct-to-LDS copy: 16 bytes from each lane's global address to LDS at
// lds + 16 * lane (lds is wave-uniform and goes through M0).
__device__ __forceinline__ void copy_to_lds(const void *src, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds) : "memory");
}
// 4 bytes per lane from src into LDS at byte address lds + 4 * lane.
__device__ __forceinline__ void copy_dword_to_lds(const void *src, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
// The same from a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void copy_to_lds(const void *base, uint32_t off, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "{m0}"(lds)
                 : "memory");
}

// v[i] of a wave-uniform array for a lane-varying i < N.  The candidates go
// through scalar registers first: a selection among plain loads of v would be
// folded into one load from a computed address, which would force v (and the
// caller's array) out of registers into scratch memory.
template <int N>
__device__ __forceinline__ float pick_uniform(const float (&v)[N], int i) {
    float r = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v[0])));
#pragma unroll
    for (int t = 1; t < N; ++t) {
        const float c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v[t])));
        r = i == t ? c : r;
    }
    return r;
}

// x of lane ^ DIST (DIST = 8, 16 or 32) for every lane.
template <int DIST>
__device__ __forceinline__ float partner_lane(float x, int lane) {
    if constexpr (DIST == 8) {
        return dpp<0x128>(x);   // row_ror:8 = lane ^ 8 within 16
    } else if constexpr (DIST == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        return __uint_as_float((lane & 32) ? r[0] : r[1]);
    }
}

// Stores n (8, 4, 2 or 1) consecutive outputs as bf16.
template <int N>
__device__ __forceinline__ void store_bf16(uint16_t *p, const float *v, float s) {
    if constexpr (N == 8) {
        store16(p, make_uint4(pack_bf16x2(v[0] * s, v[1] * s), pack_bf16x2(v[2] * s, v[3] * s),
                              pack_bf16x2(v[4] * s, v[5] * s), pack_bf16x2(v[6] * s, v[7] * s)));
    } else if constexpr (N == 4) {
        *reinterpret_cast<uint2 *>(p) =
            make_uint2(pack_bf16x2(v[0] * s, v[1] * s), pack_bf16x2(v[2] * s, v[3] * s));
    } else if constexpr (N == 2) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(v[0] * s, v[1] * s);
    } else {
        *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[0] * s));
    }
}

// Stores n (8, 4, 2 or 1) consecutive partial outputs v[i] * s in fp16 at byte
// offset off.
template <int N>
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                              const float *v, float s) {
    if constexpr (N == 8) {
        store_b128_coherent(r, off, make_uint4(pack_f16x2(v[0] * s, v[1] * s),
                                               pack_f16x2(v[2] * s, v[3] * s),
                                               pack_f16x2(v[4] * s, v[5] * s),
                                               pack_f16x2(v[6] * s, v[7] * s)));
    } else if constexpr (N == 4) {
        store_b64_coherent(r, off, pack_f16x2(v[0] * s, v[1] * s), pack_f16x2(v[2] * s, v[3] * s));
    } else if constexpr (N == 2) {
        store_b32_coherent(r, off, pack_f16x2(v[0] * s, v[1] * s));
    } else {
        store_b16_coherent(r, off, __builtin_bit_cast(uint16_t, (_Float16)(v[0] * s)));
    }
}

// Maximum over all 64 lanes of a wave; every lane gets it.
__device__ __forceinline__ float wave_max(float x, int lane) {
    x = fmaxf(x, dpp<0xB1>(x));    // lane ^ 1
    x = fmaxf(x, dpp<0x4E>(x));    // lane ^ 2
    x = fmaxf(x, dpp<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));   // row_mirror
    x = fmaxf(x, partner_lane<16>(x, lane));
    return fmaxf(x, partner_lane<32>(x, lane));
}

// Fused q/k RMSNorm + rotary embedding of head rows held as 8 lanes x two
// 8-element chunks (D = 128, 8 lanes per row: lane j holds elements 8 j .. 8 j
// + 7 and 64 + 8 j .. 64 + 8 j + 7 as packed bf16 pairs, so each element's
// rotate-half partner, D/2 away, is in the same lane).  y = x / sqrt(mean(x^2)
// + eps) * w, then pair i = 8 j + t turns by pos * turns[i] (in turns, reduced
// in fp64, sine and cosine in fp32); fp32 throughout, rounded to bf16 once.
// Lane i computes the angle of pair i only and the lanes share the 64 cosines
// and sines through LDS (the eight row groups need the same ones).
// The weights and the rates come from LDS: a vector memory load in the tile
// loop would count in vmcnt behind the tile copies in flight, and waiting for
// it would drain them.
//
// Per-wave LDS block of the fused step: q weight [128] bf16, k weight [128]
// bf16, the cosines [64] and sines [64] (fp32) of the current segment's
// angles, then per staging buffer 16 bytes for the position
// (or the (t, h, w) positions) of the entry whose segment starts in that
// buffer's tile: they travel with the tile's copies, so the rotation at the
// segment start waits for no load of its own.
constexpr int kNormRopeLds = 1024 + 16 * kMaxStageBuffers;

// sin and cos of 2 pi x for |x| <= 1/2 (x in turns): the nearest quarter turn
// q comes off exactly, the rest r (|r| <= 1/8 turn, |2 pi r| <= pi/4) goes
// through the Taylor series of sin to degree 9 and of cos to degree 10
// (truncation below 2e-9), then the result turns by q quarter turns.
__device__ __forceinline__ void sincos_turns(float x, float &s, float &c) {
    const float q = rintf(4.f * x);
    const float t = fmaf(q, -0.25f, x) * 6.2831853071795865f;
    const float t2 = t * t;
    float ps = fmaf(t2, 2.7557319e-6f, -1.9841270e-4f);
    ps = fmaf(t2, ps, 8.3333333e-3f);
    ps = fmaf(t2, ps, -1.6666667e-1f);
    const float sv = fmaf(t * t2, ps, t);
    float pc = fmaf(t2, -2.7557319e-7f, 2.4801587e-5f);
    pc = fmaf(t2, pc, -1.3888889e-3f);
    pc = fmaf(t2, pc, 4.1666667e-2f);
    pc = fmaf(t2, pc, -0.5f);
    const float cv = fmaf(t2, pc, 1.0f);
    const int qi = (int)q & 3;   // quarter turns, modulo a whole turn
    const float s1 = (qi & 1) ? cv : sv;
    const float c1 = (qi & 1) ? sv : cv;
    s = (qi & 2) ? -s1 : s1;                    // q = 2, 3: sin negated
    c = (qi == 1 || qi == 2) ? -c1 : c1;        // q = 1, 2: cos negated
}

// One row: RMSNorm with weight row wsel (0: q, 1: k) and the rotation by the
// lane's angles.  Every lane of the wave runs it (the sum of squares takes DPP
// steps within each 8-lane row group).
__device__ __forceinline__ void norm_rope_row(uint32_t (&x)[2][4], const char *nrl, int wsel,
                                              int j, float eps, const float (&cs)[8],
                                              const float (&sn)[8]) {
    float f[2][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[c][2 * k] = bf16_lo(x[c][k]);
            f[c][2 * k + 1] = bf16_hi(x[c][k]);
            ss += f[c][2 * k] * f[c][2 * k] + f[c][2 * k + 1] * f[c][2 * k + 1];
        }
    ss = row_sum<8>(ss);
    const float inv = 1.0f / sqrtf(ss / 128.0f + eps);
    const uint4 *wrow = reinterpret_cast<const uint4 *>(nrl + 256 * wsel);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint4 wv = wrow[j + 8 * c];
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[c][2 * k] = f[c][2 * k] * inv * bf16_lo(ww[k]);
            f[c][2 * k + 1] = f[c][2 * k + 1] * inv * bf16_hi(ww[k]);
        }
    }
    float z[2][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        z[0][t] = f[0][t] * cs[t] - f[1][t] * sn[t];
        z[1][t] = f[1][t] * cs[t] + f[0][t] * sn[t];
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            x[c][k] = pack_bf16x2(z[c][2 * k], z[c][2 * k + 1]);
}

template <int D, int G, int NBUF, bool NR = false>
__global__ __launch_bounds__(kMaxWavesPerGroup * 64) void run_kernel(
    RunArgs a, const int4 *__restrict__ blocks, const int4 *__restrict__ ent,
    const int32_t *__restrict__ positions) {
    constexpr int LPR = (D == 128 && G > 4) ? 16 : 8;   // lanes per row
    constexpr int RG = 64 / LPR;               // row groups: rows the wave holds at once
    constexpr int RPL = kTileTokens / RG;      // rows per lane per tile
    constexpr int NC = D / (8 * LPR);          // 8-element chunks per lane and row
    constexpr int V = G * NC * 8 / RG;         // outputs per lane after the reduce-scatter
    constexpr int HPR = (G + RG - 1) / RG;     // heads per row group in merges and lse
    constexpr int IPW = D / 64;                // copies per wave per tile half (K or V)
    constexpr int IPT = 2 * IPW;               // copies per wave per tile
    constexpr int QB = G * D * 2;              // q bytes of one KV head's query heads
    constexpr int QI = (QB + 1023) / 1024;     // copies for them
    static_assert(NC >= 1 && RPL >= 1 && V >= 1, "unsupported head_dim");
    static_assert(!NR || (D == 128 && LPR == 8), "the fused norm/rotary needs 8 lanes per row");
    // Vector memory stores a segment end issues (outputs and lse): they count
    // in vmcnt like the copies, so the waits below include them.
    // (fp16 partial outputs take as many stores as bf16 outputs)
    constexpr int kOutStores = V % 8 == 0 ? V / 8 : (8 % V == 0 ? 1 : V);
    constexpr int kPartStores = kOutStores;
    extern __shared__ uint4 smem[];
    const int lane = threadIdx.x & 63;
    const int rg = lane / LPR;                 // row group of this lane
    const int j = lane % LPR;
    const int nw = blockDim.x >> 6;            // waves = KV heads of the group
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h0 = blockIdx.y * nw;
    const int h = h0 + w;
    const bool fused = a.k_new != nullptr;
    const int hq0 = h * G;
    const int col = h * D + j * 8;             // element of this lane's chunk 0 in a token row

    // LDS buffer b: K rows [8][nw][D], V rows, then per wave QI KiB of q
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t part_bytes = (uint32_t)(kTileTokens * nw * D * 2);
    const uint32_t buf_bytes = 2 * part_bytes + (uint32_t)(nw * QI * 1024);
    constexpr int RPI = 512 / D;               // rows of one head per 1 KiB copy
    // LDS reads of 16 lanes meet in one pass: with 8 lanes per 256-byte row
    // those are two rows, on the same banks, so odd rows hold their two
    // 128-byte halves swapped (the copies place them so: every lane picks its
    // own source)
    constexpr bool SWZ = D == 128 && LPR == 8;
    static_assert(!SWZ || RPL == 1, "the swap is keyed to a lane's one row");
    constexpr int HB = kTileTokens * D * 2;    // bytes of a wave's K (or V) rows of a tile
    const int64_t half_bytes = (int64_t)a.half_stride * 2;
    const int64_t row_bytes = (int64_t)a.row_stride * 2;

    // The fused step's weights and rates, in this wave's own LDS block: the
    // weights by two copies issued ahead of every tile copy (so a tile that
    // has landed implies they have), the rate of pair `lane`, theta^(-lane/64)
    // / (2 pi), computed here in fp64.
    const char *nrl = reinterpret_cast<const char *>(smem) + NBUF * buf_bytes +
                      w * kNormRopeLds;
    // pair `lane`'s rate in turns per position, theta^(-lane/64) / (2 pi)
    double pair_rate = 0.0;
    if constexpr (NR) {
        const uint32_t nb = lds0 + NBUF * buf_bytes + (uint32_t)(w * kNormRopeLds);
        copy_dword_to_lds(a.q_w + 2 * lane, nb);
        copy_dword_to_lds(a.k_w + 2 * lane, nb + 256);
        pair_rate = exp2(-(double)lane * (a.log2_theta / 64.0)) * 0.15915494309189535;
    }
    // The lane's eight rotary angles (pairs 8 j .. 8 j + 7) for positions
    // p[0..2]: one position per entry (p[0]), or for multimodal RoPE the
    // (t, h, w) component each pair follows.  Lane i turns pair i (the
    // component it follows is picked once here, through scalar registers: a
    // lane-varying index into the argument array would become a memory load)
    // and the lanes exchange the results through the wave's LDS block.
    uint32_t pair_axis = 0;
    if constexpr (NR) {
        if (a.pos_stride != 1) {
            const uint32_t w0 = __builtin_amdgcn_readfirstlane(a.axis_bits[0]);
            const uint32_t w1 = __builtin_amdgcn_readfirstlane(a.axis_bits[1]);
            const uint32_t w2 = __builtin_amdgcn_readfirstlane(a.axis_bits[2]);
            const uint32_t w3 = __builtin_amdgcn_readfirstlane(a.axis_bits[3]);
            const int q4 = lane >> 4;   // word of pairs 16 q4 .. 16 q4 + 15
            const uint32_t word = q4 == 0 ? w0 : (q4 == 1 ? w1 : (q4 == 2 ? w2 : w3));
            pair_axis = (word >> (2 * (lane & 15))) & 3u;
        }
    }
    auto angles_at = [&](const int32_t *p, float (&cs)[8], float (&sn)[8]) {
        const double p0 = (double)p[0];
        double pp = p0;
        if (a.pos_stride != 1) {
            const double p1 = (double)p[1], p2 = (double)p[2];
            pp = pair_axis == 0 ? p0 : (pair_axis == 1 ? p1 : p2);
        }
        const double tn = pp * pair_rate;
        float sv, cv;
        sincos_turns((float)(tn - rint(tn)), sv, cv);
        float *tab = reinterpret_cast<float *>(const_cast<char *>(nrl) + 512);
        tab[lane] = cv;
        tab[64 + lane] = sv;
        const float4 c0 = *reinterpret_cast<const float4 *>(tab + 8 * j);
        const float4 c1 = *reinterpret_cast<const float4 *>(tab + 8 * j + 4);
        const float4 s0 = *reinterpret_cast<const float4 *>(tab + 64 + 8 * j);
        const float4 s1 = *reinterpret_cast<const float4 *>(tab + 64 + 8 * j + 4);
        cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w;
        cs[4] = c1.x; cs[5] = c1.y; cs[6] = c1.z; cs[7] = c1.w;
        sn[0] = s0.x; sn[1] = s0.y; sn[2] = s0.z; sn[3] = s0.w;
        sn[4] = s1.x; sn[5] = s1.y; sn[6] = s1.z; sn[7] = s1.w;
    };
    const __amdgpu_buffer_rsrc_t ro = partial_rsrc(a.part_o, a.part_o_bytes);
    const __amdgpu_buffer_rsrc_t rl = partial_rsrc(a.part_lse, a.part_lse_bytes);
    const int4 *blk = blocks + (int64_t)blockIdx.x * a.block_stride;
    // the header and the first NBUF records load together (the block region
    // is padded, so they are in bounds even past a short block's records)
    const int4 hdr = blk[0];
    int4 rec0[NBUF];
#pragma unroll
    for (int t = 0; t < NBUF; ++t)
        rec0[t] = blk[1 + t];
    // The plan must be the one made for this launch's arguments: the
    // signature in the block header is compared before any record is used.
    // A workspace holding another plan (or none) gives NaN rows and writes no
    // cache byte.
    const bool plan_ok = hdr.z == a.plan_sig;
    const int n = plan_ok ? hdr.x : 0;

    uint32_t qv[G][NC][4];    // q of the entry being computed
    float m[G], l[G], acc[G][NC][8];
    int pend0 = -1, pend1 = -1;   // entries of this wave's first and last partials
    int nsplit = 0;               // partials this wave wrote (split segment ends)
    // The first partial of a block usually ends before the block's last tile;
    // it signals its arrival at loop iteration sig_at, when its stores are
    // known to be complete, and old0 keeps what its counter held then.
    int sig_at = -1, old0 = 0;
    bool signaled0 = false;

    // Writes this lane's share of a finished segment: the outputs (whole
    // entry) or the partial of slot `slot` (fp16 outputs scaled by 2^-s, and
    // per query head {base-2 lse, s}).  u[t] is the total of value r * V + t
    // of the lane's flattened [G][NC][8] accumulators; lt[g] is head g's sum
    // of weights.
    auto write_rows = [&](int b, int slot, bool whole, const float (&u)[V],
                          const float (&lt)[G]) {
        float inv[G];
#pragma unroll
        for (int g = 0; g < G; ++g)
            inv[g] = 1.f / lt[g];
        const int64_t orow = (int64_t)b * a.num_qo_heads + hq0;    // output row of head 0
        const uint32_t prow = (uint32_t)slot * a.num_qo_heads + hq0;
        float nv[V];   // normalized outputs
#pragma unroll
        for (int t = 0; t < V; ++t)
            nv[t] = u[t] * pick_uniform<G>(inv, ((rg * V + t) >> 3) / NC);
        float sc = 1.f, sexp = 0.f;
        if (!whole) {
            float amax = 0.f;
#pragma unroll
            for (int t = 0; t < V; ++t)
                amax = fmaxf(amax, fabsf(nv[t]));
            const int e = __builtin_amdgcn_frexp_expf(wave_max(amax, lane));   // amax < 2^e
            sc = __builtin_amdgcn_ldexpf(1.f, -e);
            sexp = (float)e;
        }
        // one run of N values starting at flattened value f
        auto put = [&](auto nvc, int f, const float *v) {
            constexpr int N = decltype(nvc)::value;
            const int k = f >> 3;
            const int g = k / NC;
            const int e = ((j + LPR * (k % NC)) << 3) + (f & 7);   // element within the head
            if (whole)
                store_bf16<N>(a.out + (orow + g) * D + e, v, 1.f);
            else
                store_partial<N>(ro, ((prow + g) * D + e) * 2, v, sc);
        };
        if constexpr (V % 8 == 0) {
#pragma unroll
            for (int q = 0; q < V; q += 8)
                put(std::integral_constant<int, 8>{}, rg * V + q, nv + q);
        } else if constexpr (8 % V == 0) {
            put(std::integral_constant<int, V>{}, rg * V, nv);
        } else {
#pragma unroll
            for (int t = 0; t < V; ++t)
                put(std::integral_constant<int, 1>{}, rg * V + t, nv + t);
        }
        if (j == 0) {
#pragma unroll
            for (int t = 0; t < HPR; ++t) {
                const int g = rg + RG * t;
                if (g >= G)
                    break;
                const float lse2 = pick_uniform<G>(m, g) + log2_fast(pick_uniform<G>(lt, g));
                if (whole) {
                    if (a.lse != nullptr)
                        a.lse[orow + g] = lse2 * kLn2;
                } else {
                    store_b64_coherent(rl, (prow + g) * 8, __float_as_uint(lse2),
                                       __float_as_uint(sexp));
                }
            }
        }
    };

    if (n > 0) {
        auto rec_of = [&](int i) { return blk[1 + min(i, n - 1)]; };

        // Per-lane byte offsets of this wave's copies: copy i (of IPW per
        // half) moves rows RPI i .. RPI i + RPI - 1 of head w, lane = row
        // within the copy * D / 8 + 16-byte unit of the row, into LDS rows of
        // D * 2 bytes.  Rows past the tile's last token re-read its first row
        // (off0).
        int crow[IPW];
        uint32_t coff[IPW], coff0[IPW];
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            crow[i] = RPI * i + lane / (D / 8);
            const int unit = (lane % (D / 8)) ^ (SWZ ? ((crow[i] & 1) << 3) : 0);
            coff0[i] = (uint32_t)(w * D * 2 + unit * 16);
            coff[i] = (uint32_t)(crow[i] * row_bytes) + coff0[i];
        }
        const char *cache_b = reinterpret_cast<const char *>(a.cache) + (int64_t)h0 * D * 2;
        const int64_t page_bytes = a.page_stride * 2;

        // The records of the tiles in the ring: record of buffer b in lane b
        // of four registers.
        int ring_x = 0, ring_y = 0, ring_z = 0, ring_w = 0;
        // Vector memory operations issued so far (modulo 2^32), and in lane b
        // of ring_ops their number right after the copies of buffer b's tile:
        // a tile has landed once at most ops - ring_ops[b] are outstanding.
        uint32_t ops = 0;
        float seg_cs[8], seg_sn[8];   // fused norm/rotary: the segment's angles
        int ring_ops = 0;

        // This wave's share of the copies of tile `rec` into LDS buffer `buf`:
        // the q rows first (when a segment starts there), then IPW 1-KiB runs
        // of K rows and as many of V rows; the fused append's new row comes
        // from k_new / v_new.
        auto issue = [&](const int4 rec, int buf) {
            const int info = rec.y;
            // (with the fused norm/rotary, a segment start also copies the
            // entry's positions: one more operation)
            ops += ((info & kInfoSegFirst) ? QI + (NR ? 1 : 0) : 0) + IPT;
            if (lane == buf) {
                ring_x = rec.x;
                ring_y = rec.y;
                ring_z = rec.z;
                ring_w = rec.w;
                ring_ops = (int)ops;
            }
            const int ntok = (info & kInfoNtokMask) + 1;
            const int slot0 = (info >> kInfoSlotShift) & kInfoSlotMask;
            const uint32_t bb = lds0 + (uint32_t)buf * buf_bytes;
            if (info & kInfoSegFirst) {
                if constexpr (NR) {
                    // the entry's position(s) into this buffer's 16 bytes of
                    // the wave's norm/rotary block
                    if (lane < a.pos_stride)
                        copy_dword_to_lds(positions + (int64_t)rec.z * a.pos_stride + lane,
                                          lds0 + NBUF * buf_bytes +
                                              (uint32_t)(w * kNormRopeLds + 1024 + buf * 16));
                }
                const char *qs = reinterpret_cast<const char *>(a.q) +
                                 ((int64_t)rec.z * a.num_qo_heads + hq0) * D * 2;
#pragma unroll
                for (int i = 0; i < QI; ++i) {
                    const int off = min((i * 64 + lane) * 16, QB - 16);
                    copy_to_lds(qs + off, bb + 2 * part_bytes + (uint32_t)(w * QI + i) * 1024);
                }
            }
            const int page = (unsigned)rec.x < (unsigned)a.num_pages ? rec.x : 0;
            const char *kb = cache_b + (int64_t)page * page_bytes + (int64_t)slot0 * row_bytes;
            const char *vb = kb + half_bytes;
            if (fused && (info & kInfoHasNew)) {
                const int nr = (info >> kInfoNewRowShift) & (kTileTokens - 1);
                const int64_t nsrc = ((int64_t)rec.z * a.num_kv_heads + h0) * D * 2;
#pragma unroll
                for (int i = 0; i < IPW; ++i) {
                    const uint32_t o = crow[i] < ntok ? coff[i] : coff0[i];
                    const bool is_new = crow[i] == nr;
                    const char *ks = is_new ? reinterpret_cast<const char *>(a.k_new) + nsrc +
                                                  coff0[i]
                                            : kb + o;
                    const char *vs = is_new ? reinterpret_cast<const char *>(a.v_new) + nsrc +
                                                  coff0[i]
                                            : vb + o;
                    copy_to_lds(ks, bb + (uint32_t)(w * HB + i * 1024));
                    copy_to_lds(vs, bb + part_bytes + (uint32_t)(w * HB + i * 1024));
                }
            } else if (ntok == kTileTokens) {
#pragma unroll
                for (int i = 0; i < IPW; ++i) {
                    copy_to_lds(kb, coff[i], bb + (uint32_t)(w * HB + i * 1024));
                    copy_to_lds(vb, coff[i], bb + part_bytes + (uint32_t)(w * HB + i * 1024));
                }
            } else {
#pragma unroll
                for (int i = 0; i < IPW; ++i) {
                    const uint32_t o = crow[i] < ntok ? coff[i] : coff0[i];
                    copy_to_lds(kb, o, bb + (uint32_t)(w * HB + i * 1024));
                    copy_to_lds(vb, o, bb + part_bytes + (uint32_t)(w * HB + i * 1024));
                }
            }
        };

        // LDS in 16-byte units: this lane's chunk 0 of its first K row (head
        // w's region, row rg, unit j), the step to its next row, its q chunk 0
        const int kunit = (w * kTileTokens + rg) * (D / 8) + j;   // SWZ: chunk at j + 8 (c ^ rg&1)
        const int rstep = RG * (D / 8);
        const int part_units = (int)(part_bytes / 16);
        const int buf_units = (int)(buf_bytes / 16);
        const int qunit = (2 * part_bytes + w * QI * 1024) / 16 + j;

        auto compute_tile = [&](int k) {
            const int buf = k % NBUF;
            const int4 rec = make_int4(__builtin_amdgcn_readlane(ring_x, buf),
                                       __builtin_amdgcn_readlane(ring_y, buf),
                                       __builtin_amdgcn_readlane(ring_z, buf),
                                       __builtin_amdgcn_readlane(ring_w, buf));
            const int info = rec.y;
            const uint4 *sb = smem + buf * buf_units;
            if (info & kInfoSegFirst) {
                if constexpr (NR) {
                    // row group rg normalizes and rotates query head rg in
                    // place (the other groups compute a copy and keep it);
                    // the loads below then give every group all G heads
                    angles_at(reinterpret_cast<const int32_t *>(nrl + 1024 + buf * 16), seg_cs,
                              seg_sn);
                    uint4 *qrow = smem + buf * buf_units + qunit + (rg < G ? rg : 0) * (D / 8);
                    const uint4 v0 = qrow[0], v1 = qrow[8];
                    uint32_t x[2][4] = {{v0.x, v0.y, v0.z, v0.w}, {v1.x, v1.y, v1.z, v1.w}};
                    norm_rope_row(x, nrl, 0, j, a.eps, seg_cs, seg_sn);
                    if (rg < G) {
                        qrow[0] = make_uint4(x[0][0], x[0][1], x[0][2], x[0][3]);
                        qrow[8] = make_uint4(x[1][0], x[1][1], x[1][2], x[1][3]);
                    }
                    asm volatile("" ::: "memory");
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const uint4 v = sb[qunit + g * (D / 8) + LPR * c];
                        qv[g][c][0] = v.x;
                        qv[g][c][1] = v.y;
                        qv[g][c][2] = v.z;
                        qv[g][c][3] = v.w;
                    }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    m[g] = kMInit;
                    l[g] = 0.f;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[g][c][e] = 0.f;
                }
            }
            const int ntok = (info & kInfoNtokMask) + 1;
            const int nr = (info >> kInfoNewRowShift) & (kTileTokens - 1);
            uint4 kx[RPL][NC], vx[RPL][NC];
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int cu = SWZ ? 8 * (c ^ (rg & 1)) : LPR * c;
                    kx[i][c] = sb[kunit + i * rstep + cu];
                    vx[i][c] = sb[part_units + kunit + i * rstep + cu];
                }
            if constexpr (NR) {
                if (info & kInfoHasNew) {
                    // the new row arrives raw from k_new: normalize and rotate
                    // it here, in the row group holding it (every lane runs
                    // the arithmetic; the others keep their rows), so the
                    // dot product and the cache store below both see the
                    // transformed row
                    uint32_t kk[2][4] = {{kx[0][0].x, kx[0][0].y, kx[0][0].z, kx[0][0].w},
                                         {kx[0][1].x, kx[0][1].y, kx[0][1].z, kx[0][1].w}};
                    // the segment's angles (the new row belongs to it)
                    norm_rope_row(kk, nrl, 1, j, a.eps, seg_cs, seg_sn);
                    if (rg == nr) {
                        kx[0][0] = make_uint4(kk[0][0], kk[0][1], kk[0][2], kk[0][3]);
                        kx[0][1] = make_uint4(kk[1][0], kk[1][1], kk[1][2], kk[1][3]);
                    }
                }
            }
            // q.k: RPL x G independent dot products over the lane's chunks,
            // then their row sums step by step across all of them
            float d[RPL][G];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        d[i][g] = dot2_bf16(qv[g][c][0], kx[i][c].x, c == 0 ? 0.f : d[i][g]);
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        d[i][g] = dot2_bf16(qv[g][c][1], kx[i][c].y, d[i][g]);
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        d[i][g] = dot2_bf16(qv[g][c][2], kx[i][c].z, d[i][g]);
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        d[i][g] = dot2_bf16(qv[g][c][3], kx[i][c].w, d[i][g]);
            }
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    d[i][g] += dpp<0xB1>(d[i][g]);    // quad_perm [1,0,3,2]: lane ^ 1
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    d[i][g] += dpp<0x4E>(d[i][g]);    // quad_perm [2,3,0,1]: lane ^ 2
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    d[i][g] += dpp<0x141>(d[i][g]);   // row_half_mirror: 7 - lane within 8
            if constexpr (LPR == 16) {
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        d[i][g] += dpp<0x140>(d[i][g]);   // row_mirror: 15 - lane within 16
            }
            if (ntok < kTileTokens) {
                // rows past the tile's last token (they re-read its first row,
                // which for a fused append is the stale slot of the new row):
                // weight 0 and value 0, so nothing they hold reaches the sums
#pragma unroll
                for (int i = 0; i < RPL; ++i)
                    if (rg + RG * i >= ntok) {
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            d[i][g] = -INFINITY;
#pragma unroll
                        for (int c = 0; c < NC; ++c)
                            vx[i][c] = make_uint4(0u, 0u, 0u, 0u);
                    }
            }
            // Lazy maximum (log2 units, scores d * scale_log2): raised only
            // when some row's score passes it by more than kTau, then to the
            // maximum over the tile's rows, in every row group alike.
            const float c2 = a.scale_log2;
            bool raise = false;
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    raise |= fmaf(d[i][g], c2, -m[g]) > kTau;
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float dm = d[0][g];
#pragma unroll
                    for (int i = 1; i < RPL; ++i)
                        dm = fmaxf(dm, d[i][g]);
                    const float sm = group_max<RG>(dm) * c2;
                    if (sm - m[g] > kTau) {
                        const float alpha = exp2_fast(m[g] - sm);
                        m[g] = sm;
                        l[g] *= alpha;
#pragma unroll
                        for (int c = 0; c < NC; ++c)
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[g][c][e] *= alpha;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                float p[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    p[g] = exp2_fast(fmaf(d[i][g], c2, -m[g]));   // 0 for masked rows
                    l[g] += p[g];
                }
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const uint4 v = vx[i][c];
                    const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y),
                                         bf16_hi(v.y), bf16_lo(v.z), bf16_hi(v.z),
                                         bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[g][c][e] = fmaf(p[g], vf[e], acc[g][c][e]);
                }
            }
            if (fused && (info & kInfoHasNew)) {
                // append: the lanes holding the new row store it into its slot
                const int slot0 = (info >> kInfoSlotShift) & kInfoSlotMask;
                // a page or slot outside the pool (only a corrupted plan has
                // one) writes nothing
                const bool in_pool = (unsigned)rec.x < (unsigned)a.num_pages &&
                                     slot0 + nr < a.page_size;
                uint16_t *dst = a.cache_w + (int64_t)rec.x * a.page_stride +
                                (int64_t)(slot0 + nr) * a.row_stride + col;
#pragma unroll
                for (int i = 0; i < RPL; ++i)
                    if (rg + RG * i == nr && in_pool) {
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            store16(dst + 8 * LPR * c, kx[i][c]);
                            store16(dst + 8 * LPR * c + a.half_stride, vx[i][c]);
                        }
                    }
                // one row of the tile holds the new token; in_pool is the same
                // in every lane, so the stores were issued exactly when it holds
                if (in_pool)
                    ops += 2 * NC;
            }
            if (info & kInfoSegLast) {
                // Add the row groups: the weight sums in every lane, the
                // accumulators by halving steps across lanes 32, 16 and (for
                // 8 row groups) 8 apart: at each step a lane keeps the lower
                // half of its values when its lane bit is 0 and the upper half
                // when it is 1, and adds the partner's same half.  Lane (r, j)
                // ends with the totals of values r * V .. r * V + V - 1.
                float lt[G];
#pragma unroll
                for (int g = 0; g < G; ++g)
                    lt[g] = group_sum<RG>(l[g]);
                constexpr int T = G * NC * 8;
                float x4[T / 2];
#pragma unroll
                for (int i = 0; i < T / 2; ++i) {
                    constexpr int S = 8 * NC;
                    const int i2 = i + T / 2;
                    // permlane32_swap(a, b): lanes 0-31 get a of lanes 32-63 in
                    // b's place, lanes 32-63 get b of lanes 0-31 in a's place
                    const auto r = __builtin_amdgcn_permlane32_swap(
                        __float_as_uint(acc[i / S][(i % S) / 8][i % 8]),
                        __float_as_uint(acc[i2 / S][(i2 % S) / 8][i2 % 8]), false, false);
                    x4[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                }
                float x2[T / 4];
#pragma unroll
                for (int i = 0; i < T / 4; ++i) {
                    const auto r = __builtin_amdgcn_permlane16_swap(
                        __float_as_uint(x4[i]), __float_as_uint(x4[i + T / 4]), false, false);
                    x2[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                }
                float u[V];
                if constexpr (RG == 8) {
                    const bool odd = (rg & 1) != 0;
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        const float keep = odd ? x2[i + V] : x2[i];
                        const float send = odd ? x2[i] : x2[i + V];
                        u[i] = keep + dpp<0x128>(send);   // row_ror:8 = lane ^ 8 within 16
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < V; ++i)
                        u[i] = x2[i];
                }
                const bool whole = (info & kInfoSegWhole) != 0;
                write_rows(rec.z, rec.w, whole, u, lt);
                ops += whole ? kOutStores + (a.lse != nullptr ? HPR : 0) : kPartStores + HPR;
                if (!whole) {
                    ++nsplit;
                    // the first split end is pend0, later ones pend1; the
                    // first signals when the copies of tile k + NBUF, issued
                    // after these stores, have landed.  Written as value
                    // selects: branches can let the compiler merge the stores
                    // into one through a selected address, which puts these
                    // variables in scratch memory.
                    const bool first = pend0 < 0;
                    pend1 = first ? pend1 : rec.z;
                    sig_at = first && k + NBUF < n ? k + NBUF : sig_at;
                    pend0 = first ? rec.z : pend0;
                }
            }
        };

        // Tiles 0 .. NBUF-1 in flight before the loop; every iteration waits
        // for its tile, computes it and refills the buffer it has just
        // finished with the tile NBUF ahead (none past the end: the waits
        // count only what was issued, so they stay exact), so NBUF tiles are
        // in flight while a wave waits.
#pragma unroll
        for (int t = 0; t < NBUF; ++t) {
            if (t < n)
                issue(rec0[t], t);
        }
        int4 rn = rec_of(NBUF);
        for (int k = 0; k < n; ++k) {
            // tile k has landed: at most the operations issued after its
            // copies (NBUF - 1 tiles, their q rows, the stores since) remain
            const int after = (int)(ops - (uint32_t)__builtin_amdgcn_readlane(ring_ops, k % NBUF));
            if (after == IPT * (NBUF - 1))
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPT * (NBUF - 1)));
            else
                wait_vm_at_most<kMaxVmWait>(after);
            if (k == sig_at) {
                // the first partial's stores are complete (tile k landed)
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                if (lane == 0)
                    atomic_inc_untracked(a.cnt + (int64_t)pend0 * a.num_kv_heads + h, old0);
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                signaled0 = true;
                ops += 1;
            }
            compute_tile(k);
            const bool more = k + NBUF < n;   // uniform: the waves share the block
            if (more)
                issue(rn, k % NBUF);
            rn = rec_of(k + NBUF + 1);
            // keep the waves together while they still issue copies: see
            // kSyncTiles (past the last copies a barrier would only hold the
            // faster waves' stores and arrival counts back)
            if (more && k % kSyncTiles == kSyncTiles - 1)
                __builtin_amdgcn_s_barrier();
        }
        // the last stores complete before the wave moves on
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }

    // Split entries: count this wave's remaining partials in; the last of an
    // entry's segments to arrive merges them all and resets the counter.
    if (pend0 >= 0) {
        // the entries' descriptors load while the stores complete
        const int4 ent0 = ent[pend0];
        const int4 ent1 = ent[pend1 >= 0 ? pend1 : pend0];
        // this wave's partial stores are complete (written through) before
        // its arrivals are counted; the compiler may not move them past here
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        int32_t *cnt0 = a.cnt + (int64_t)pend0 * a.num_kv_heads + h;
        int32_t *cnt1 = a.cnt + (int64_t)(pend1 >= 0 ? pend1 : pend0) * a.num_kv_heads + h;
        int old = 0;
        if ((lane == 0 && !signaled0) || (lane == 1 && pend1 >= 0))
            old = __hip_atomic_fetch_add(lane == 0 ? cnt0 : cnt1, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        const int arr0 = __builtin_amdgcn_readlane(signaled0 ? old0 : old, 0);
        const int arr1 = __builtin_amdgcn_readlane(old, 1);
        // Merge: lane handles UPL units of 8 consecutive outputs of the KV
        // head's G x D; all of a round's SR segments are loaded at once.
        constexpr int DU = D / 8;                   // units per query head
        constexpr int NU = G * DU;
        constexpr int UPL = (NU + 63) / 64;
        constexpr int SR = 24 / UPL;
        // The entries this wave arrived last for are merged one after the
        // other: pend0, pend1 (each merge in line), then, in a block that
        // ended more than two split segments (fixed runs dealt several to a
        // workgroup), the ones between, found from the block's records one
        // lane per record, 64 at a time, their arrivals counted together.
        auto merge_entry = [&](const int b, const int4 e, int32_t *cp) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const int ns = e.y;
            uint32_t lo[UPL], oo[UPL];   // byte offsets in slot e.x: lse pair, outputs
            float mm[UPL], zs[UPL], o[UPL][8];
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const int unit = min(lane + 64 * i, NU - 1);
                const uint32_t row = (uint32_t)e.x * a.num_qo_heads + hq0 + unit / DU;
                lo[i] = row * 8;
                oo[i] = (row * D + (unit % DU) * 8) * 2;
                mm[i] = kMInit;
                zs[i] = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    o[i][q] = 0.f;
            }
            const uint32_t sl = (uint32_t)a.num_qo_heads * 8;       // slot stride, lse pairs
            const uint32_t so = (uint32_t)a.num_qo_heads * D * 2;   // slot stride, outputs
            for (int s0 = 0; s0 < ns; s0 += SR) {
                float2 lv[SR][UPL];
                uint4 ov[SR][UPL];
                // only the segments that exist: device-scope loads of the
                // same address are not merged, each one costs a full access
#pragma unroll
                for (int u = 0; u < SR; ++u) {
                    const uint32_t s = (uint32_t)(s0 + u);
#pragma unroll
                    for (int i = 0; i < UPL; ++i) {
                        if (s0 + u < ns) {
                            lv[u][i] = load_f2_coherent(rl, lo[i] + s * sl);
                            ov[u][i] = load_b128_coherent(ro, oo[i] + s * so);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < SR; ++u) {
                    if (s0 + u >= ns)   // wave-uniform: absent segments cost nothing
                        continue;
#pragma unroll
                    for (int i = 0; i < UPL; ++i) {
                        // weight of the segment: 2^(lse - m); its stored
                        // outputs carry a further factor 2^-s
                        const float l2 = lv[u][i].x;
                        const float mn = fmaxf(mm[i], l2);
                        const float al = exp2_fast(mm[i] - mn);
                        const float wz = exp2_fast(l2 - mn);
                        const float wo = exp2_fast(l2 + lv[u][i].y - mn);
                        zs[i] = fmaf(zs[i], al, wz);
                        const uint4 v = ov[u][i];
                        const float x[8] = {f16_lo(v.x), f16_hi(v.x), f16_lo(v.y), f16_hi(v.y),
                                            f16_lo(v.z), f16_hi(v.z), f16_lo(v.w), f16_hi(v.w)};
#pragma unroll
                        for (int q = 0; q < 8; ++q)
                            o[i][q] = fmaf(wo, x[q], o[i][q] * al);
                        mm[i] = mn;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const int unit = lane + 64 * i;
                if (unit < NU) {
                    const int hq = hq0 + unit / DU;
                    const float inv = 1.f / zs[i];
                    store_bf16<8>(a.out + ((int64_t)b * a.num_qo_heads + hq) * D + (unit % DU) * 8,
                                  o[i], inv);
                    if (a.lse != nullptr && unit % DU == 0)
                        a.lse[(int64_t)b * a.num_qo_heads + hq] = (mm[i] + log2_fast(zs[i])) * kLn2;
                }
            }
            if (lane == 0)
                __hip_atomic_store(cp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        if (arr0 == ent0.y - 1)
            merge_entry(pend0, ent0, cnt0);
        if (pend1 >= 0 && arr1 == ent1.y - 1)
            merge_entry(pend1, ent1, cnt1);
        if (nsplit > 2) {
            int idx_base = 0;   // split ends before the current round
            for (int k0 = 0; k0 < n; k0 += 64) {
                const int k = k0 + lane;
                const int4 rec = k < n ? blk[1 + k] : make_int4(0, 0, 0, 0);
                const bool split_end =
                    k < n && (rec.y & kInfoSegLast) != 0 && (rec.y & kInfoSegWhole) == 0;
                const uint64_t m = __builtin_amdgcn_ballot_w64(split_end);
                const int idx = idx_base + __builtin_popcountll(m & ((1ull << lane) - 1ull));
                idx_base += __builtin_popcountll(m);
                const bool mine = split_end && idx >= 1 && idx <= nsplit - 2;
                int oldm = -1;
                int4 rem = make_int4(0, 0, 0, 0);
                if (mine) {
                    rem = ent[rec.z];
                    oldm = __hip_atomic_fetch_add(a.cnt + (int64_t)rec.z * a.num_kv_heads + h, 1,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                uint64_t todo = __builtin_amdgcn_ballot_w64(mine && oldm == rem.y - 1);
                while (todo != 0) {
                    const int l = __builtin_ctzll(todo);
                    todo &= todo - 1;
                    const int b = __builtin_amdgcn_readlane(rec.z, l);
                    const int4 e = make_int4(__builtin_amdgcn_readlane(rem.x, l),
                                             __builtin_amdgcn_readlane(rem.y, l), 0, 0);
                    merge_entry(b, e, a.cnt + (int64_t)b * a.num_kv_heads + h);
                }
                if (idx_base >= nsplit - 1)
                    break;   // every split end between has been seen
            }
        }
    }

    // Entries over the page bound: NaN rows (the broken precondition shows
    // instead of a truncated result) and, when fused, the append all the same.
    for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
        const int4 e = plan_ok ? ent[b] : make_int4(0, -1, -1, -1);
        if (e.y >= 0)
            continue;
#pragma unroll
        for (int t = 0; t < HPR; ++t) {
            const int g = rg + RG * t;
            if (g >= G)
                break;
            const int hq = hq0 + g;
            uint16_t *orow = a.out + ((int64_t)b * a.num_qo_heads + hq) * D + j * 8;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                store16(orow + 8 * LPR * c,
                        make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u));
            if (a.lse != nullptr && j == 0)
                a.lse[(int64_t)b * a.num_qo_heads + hq] = __builtin_nanf("");
        }
        // with a plan of other arguments, no append; otherwise the target must
        // lie in the pool
        if (fused && plan_ok && (unsigned)e.z < (unsigned)a.num_pages &&
            (unsigned)e.w < (unsigned)a.page_size) {
            const int64_t src = ((int64_t)b * a.num_kv_heads + h) * D + j * 8;
            uint16_t *dst = a.cache_w + (int64_t)e.z * a.page_stride +
                            (int64_t)e.w * a.row_stride + col;
            uint4 kr[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                kr[c] = load16(a.k_new + src + 8 * LPR * c);
            if constexpr (NR) {
                // every row group transforms the row (the sums run on whole
                // 8-lane groups); the first stores it.  The staged weights
                // have landed once nothing is outstanding.
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                uint32_t kk[2][4] = {{kr[0].x, kr[0].y, kr[0].z, kr[0].w},
                                     {kr[1].x, kr[1].y, kr[1].z, kr[1].w}};
                float cs[8], sn[8];
                angles_at(positions + (int64_t)b * a.pos_stride, cs, sn);
                norm_rope_row(kk, nrl, 1, j, a.eps, cs, sn);
                kr[0] = make_uint4(kk[0][0], kk[0][1], kk[0][2], kk[0][3]);
                kr[1] = make_uint4(kk[1][0], kk[1][1], kk[1][2], kk[1][3]);
            }
            if (rg == 0) {
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    store16(dst + 8 * LPR * c, kr[c]);
                    store16(dst + 8 * LPR * c + a.half_stride,
                            load16(a.v_new + src + 8 * LPR * c));
                }
            }
        }
    }
}

// Launch through hipLaunchKernel so the returned status belongs to this
// launch alone (hipGetLastError could report an older, unrelated error).
hipError_t launch_raw(const void *kernel, dim3 grid, dim3 block, size_t lds, void **params,
                      hipStream_t stream) {
    return hipLaunchKernel(kernel, grid, block, params, lds, stream);
}

template <int D, int NBUF>
const void *run_kernel_dn(int group) {
    switch (group) {
    case 1: return reinterpret_cast<const void *>(&run_kernel<D, 1, NBUF>);
    case 2: return reinterpret_cast<const void *>(&run_kernel<D, 2, NBUF>);
    case 3: return reinterpret_cast<const void *>(&run_kernel<D, 3, NBUF>);
    case 4: return reinterpret_cast<const void *>(&run_kernel<D, 4, NBUF>);
    case 5: return reinterpret_cast<const void *>(&run_kernel<D, 5, NBUF>);
    case 6: return reinterpret_cast<const void *>(&run_kernel<D, 6, NBUF>);
    case 7: return reinterpret_cast<const void *>(&run_kernel<D, 7, NBUF>);
    case 8: return reinterpret_cast<const void *>(&run_kernel<D, 8, NBUF>);
    default: return nullptr;
    }
}

template <int D>
const void *run_kernel_d(int group, int nbuf) {
    static_assert(kMaxStageBuffers == 2, "only the two-buffer ring is instantiated");
    return nbuf == 2 ? run_kernel_dn<D, 2>(group) : nullptr;
}

// The decode with the fused q/k norm + rotary embedding: head_dim 128, groups
// up to 4, two staging buffers.
const void *run_kernel_nr_ptr(int head_dim, int group, int nbuf) {
    if (head_dim != 128 || nbuf != 2)
        return nullptr;
    switch (group) {
    case 1: return reinterpret_cast<const void *>(&run_kernel<128, 1, 2, true>);
    case 2: return reinterpret_cast<const void *>(&run_kernel<128, 2, 2, true>);
    case 3: return reinterpret_cast<const void *>(&run_kernel<128, 3, 2, true>);
    case 4: return reinterpret_cast<const void *>(&run_kernel<128, 4, 2, true>);
    default: return nullptr;
    }
}

const void *run_kernel_ptr(int head_dim, int group, int nbuf) {
    if (head_dim == 64)
        return run_kernel_d<64>(group, nbuf);
    if (head_dim == 128)
        return run_kernel_d<128>(group, nbuf);
    return nullptr;
}

// LDS bytes of one staging buffer: K and V rows of a tile for nw heads, and
// the q rows of their query heads.
size_t stage_buffer_bytes(int nw, int head_dim, int group) {
    const size_t qi = ((size_t)group * head_dim * 2 + 1023) / 1024;
    return (size_t)2 * kTileTokens * nw * head_dim * 2 + (size_t)nw * qi * 1024;
}

// Per-device facts the launches need, queried once per device and kept for
// the life of the process: the LDS a workgroup may use, the compute units,
// and for each decode kernel the dynamic LDS it has been allowed and how many
// of its workgroups one compute unit holds.  Guarded by a mutex, so the
// calls stay thread-safe.
constexpr int kMaxDevices = 64;
struct DeviceFacts {
    bool known = false;
    int max_lds = 0;
    int cus = 0;
};
struct KernelFacts {
    int dev;
    const void *kernel;
    size_t lds;       // dynamic LDS the kernel has been allowed on dev
    int threads;
    int per_cu;       // workgroups of `threads` threads with `lds` bytes per CU
};
std::mutex g_facts_mu;
DeviceFacts g_dev_facts[kMaxDevices];
constexpr int kMaxKernelFacts = 256;
KernelFacts g_kernel_facts[kMaxKernelFacts];
int g_num_kernel_facts = 0;

hipError_t device_facts(int *dev, DeviceFacts *out) {
    hipError_t err = hipGetDevice(dev);
    if (err != hipSuccess)
        return err;
    if (*dev < 0 || *dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_facts_mu);
    DeviceFacts &f = g_dev_facts[*dev];
    if (!f.known) {
        int lds = 0, cus = 0;
        err = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, *dev);
        if (err == hipSuccess)
            err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, *dev);
        if (err != hipSuccess)
            return err;
        f.max_lds = lds;
        f.cus = cus;
        f.known = true;
    }
    *out = f;
    return hipSuccess;
}

// Allows `kernel` `lds` bytes of dynamic LDS on device dev (once; again only
// when a call needs more) and returns how many of its workgroups of
// `threads` threads a compute unit holds with that much LDS.
hipError_t kernel_facts(int dev, const void *kernel, size_t lds, int threads, int *per_cu) {
    std::lock_guard<std::mutex> lock(g_facts_mu);
    KernelFacts *f = nullptr;
    for (int i = 0; i < g_num_kernel_facts; ++i)
        if (g_kernel_facts[i].dev == dev && g_kernel_facts[i].kernel == kernel) {
            f = &g_kernel_facts[i];
            break;
        }
    if (f != nullptr && f->lds >= lds && f->threads == threads) {
        if (per_cu != nullptr)
            *per_cu = f->per_cu;
        return hipSuccess;
    }
    const size_t allow = f != nullptr && f->lds > lds ? f->lds : lds;
    hipError_t err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)allow);
    int pc = 0;
    if (err == hipSuccess)
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, kernel, threads, lds);
    if (err != hipSuccess)
        return err;
    if (f == nullptr) {
        if (g_num_kernel_facts == kMaxKernelFacts) {
            // full (far more kernels than exist): answer without keeping it
            if (per_cu != nullptr)
                *per_cu = pc;
            return hipSuccess;
        }
        f = &g_kernel_facts[g_num_kernel_facts++];
        f->dev = dev;
        f->kernel = kernel;
    }
    f->lds = allow;
    f->threads = threads;
    f->per_cu = pc;
    if (per_cu != nullptr)
        *per_cu = pc;
    return hipSuccess;
}

// Staging depth (buffers) and LDS bytes of the decode kernel on the current
// device: as deep as LDS allows, up to kMaxStageBuffers.
hipError_t stage_shape(int head_dim, int group, int num_kv_heads, int *dev, int *cus,
                       int *nbuf, size_t *lds) {
    DeviceFacts f;
    hipError_t err = device_facts(dev, &f);
    if (err != hipSuccess)
        return err;
    const size_t buf = stage_buffer_bytes(group_waves(num_kv_heads), head_dim, group);
    int n = (int)((size_t)f.max_lds / buf);
    n = n > kMaxStageBuffers ? kMaxStageBuffers : n;
    if (n < 2)
        return hipErrorInvalidValue;
    *nbuf = n;
    *lds = buf * (size_t)n;
    *cus = f.cus;
    return hipSuccess;
}

// Device memory of pkv_decode_static: the plan and partial rows of one call
// live in this file-scope array instead of a caller's workspace.  Each GPU
// the library runs on holds its own copy for the life of the process.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch_ptr.
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t static_scratch(void **ptr) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t compute_units(int *cus) {
    int dev = 0;
    DeviceFacts f;
    const hipError_t err = device_facts(&dev, &f);
    if (err == hipSuccess)
        *cus = f.cus;
    return err;
}

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream) {
    AppendArgs args = a;
    void *params[] = {&args};
    return launch_raw(reinterpret_cast<const void *>(&append_kernel), dim3((unsigned)batch),
                      dim3(256), 0, params, stream);
}

bool run_supported(int head_dim, int group) {
    return run_kernel_ptr(head_dim, group, 2) != nullptr;
}

bool run_norm_rope_supported(int head_dim, int group) {
    return run_kernel_nr_ptr(head_dim, group, kMaxStageBuffers) != nullptr;
}

hipError_t balanced_blocks(int head_dim, int group, int num_kv_heads, int *blocks) {
    int dev = 0, cus = 0, nbuf = 0, per_cu = 0;
    size_t lds = 0;
    hipError_t err = stage_shape(head_dim, group, num_kv_heads, &dev, &cus, &nbuf, &lds);
    if (err != hipSuccess)
        return err;
    const void *k = run_kernel_ptr(head_dim, group, nbuf);
    if (k == nullptr)
        return hipErrorInvalidValue;
    const int waves = group_waves(num_kv_heads);
    err = kernel_facts(dev, k, lds, 64 * waves, &per_cu);
    if (err != hipSuccess)
        return err;
    const int head_groups = num_kv_heads / waves;
    if (per_cu < 1)
        per_cu = 1;
    if (cus > kMaxComputeUnits)
        cus = kMaxComputeUnits;
    // workgroups resident at once, shared by the head groups
    int64_t w = ((int64_t)cus * per_cu + head_groups - 1) / head_groups;
    const int64_t bound = balanced_blocks_bound(num_kv_heads);
    *blocks = (int)(w < bound ? w : bound);
    return hipSuccess;
}

hipError_t launch_plan(const PlanArgs &a, hipStream_t stream) {
    PlanArgs args = a;
    void *params[] = {&args};
    const int64_t items = (int64_t)a.num_blocks * a.block_stride;
    const int64_t other = (int64_t)a.batch * a.num_kv_heads;
    const int64_t work = items > other ? items : other;
    int64_t grid = (work + 255) / 256;
    grid = grid < 1 ? 1 : (grid > 1024 ? 1024 : grid);
    const size_t lds = plan_lds_bytes(a.batch, a.chunk_tiles > 0, a.qo_indptr != nullptr);
    int dev = 0;
    DeviceFacts f;
    hipError_t err = device_facts(&dev, &f);
    if (err == hipSuccess && lds > (size_t)f.max_lds)
        err = hipErrorInvalidValue;
    if (err == hipSuccess)
        err = kernel_facts(dev, reinterpret_cast<const void *>(&plan_kernel), lds, 256, nullptr);
    if (err != hipSuccess)
        return err;
    return launch_raw(reinterpret_cast<const void *>(&plan_kernel), dim3((unsigned)grid),
                      dim3(256), lds, params, stream);
}

hipError_t launch_run(const RunArgs &a, const int32_t *blocks, const int32_t *ent,
                      int num_blocks, int head_dim, int group, hipStream_t stream) {
    int dev = 0, cus = 0, nbuf = 0;
    size_t lds = 0;
    hipError_t err = stage_shape(head_dim, group, a.num_kv_heads, &dev, &cus, &nbuf, &lds);
    if (err != hipSuccess)
        return err;
    const void *k = a.q_w != nullptr ? run_kernel_nr_ptr(head_dim, group, nbuf)
                                     : run_kernel_ptr(head_dim, group, nbuf);
    if (k == nullptr)
        return hipErrorInvalidValue;
    if (a.q_w != nullptr)
        lds += (size_t)group_waves(a.num_kv_heads) * kNormRopeLds;
    err = kernel_facts(dev, k, lds, 64 * group_waves(a.num_kv_heads), nullptr);
    if (err != hipSuccess)
        return err;
    RunArgs args = a;
    const int4 *bp = reinterpret_cast<const int4 *>(blocks);
    const int4 *ep = reinterpret_cast<const int4 *>(ent);
    const int32_t *pp = a.positions;
    void *params[] = {&args, &bp, &ep, &pp};
    const int waves = group_waves(a.num_kv_heads);
    const unsigned head_groups = (unsigned)(a.num_kv_heads / waves);
    return launch_raw(k, dim3((unsigned)num_blocks, head_groups), dim3(64 * waves), lds, params,
                      stream);
}

}  // namespace pkv
