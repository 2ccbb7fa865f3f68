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
//  * A workgroup has one wavefront per KV head.  In a wave, eight lanes cover
//    one token row of its head (D/8 contiguous elements each) and the eight
//    8-lane row groups cover 8 consecutive tokens: an 8-token "tile".  One
//    16-byte load per lane reads 8 rows x 128 bytes, and the workgroup as a
//    whole reads each tile's K rows and V rows of all heads, 16 KiB apiece
//    for 8 heads of 128, as contiguous runs.
//  * Partial dot products of a row are summed with three DPP steps
//    (quad_perm, quad_perm, row_half_mirror): no LDS traffic.
//  * Each row group keeps its own online-softmax state in the exp2 domain.
//    The running maximum is raised only when a new score passes it by more
//    than kTau (log2 units); between raises nothing is rescaled and exp2
//    arguments stay <= kTau.  Row groups are merged once per segment.
//  * Loads run two tiles ahead in registers (three rotating buffers), from
//    an LDS table of the tiles' page ids built once per piece of work; see
//    decode_kernel.
//
// Work split.  Balanced mode (default): the tiles of all entries are laid end
// to end and each of W workgroups takes an equal run of them (W = what the
// chip holds at once), so every compute unit streams the same number of
// bytes.  A run may cover several entries and an entry may span several runs;
// each (run, entry) segment writes either the final row (entry entirely in
// the run) or a partial (output, lse) into slot run + entry, and the merge
// kernel combines an entry's partials by log-sum-exp.  The split then depends
// on the whole batch.  Fixed mode (chunk_tiles > 0): each entry is cut into
// chunks of a fixed number of tiles, one workgroup each, so how an entry is
// split depends only on its own length and its rows are bit-identical in any
// batch.
//
// The fused append (k_new != null) treats the tile holding token L-1 of each
// entry specially: that row is read from k_new/v_new and written into the
// cache by the one workgroup that processes it, which is append followed by
// decode without a second pass over memory.
//
// All cache offsets are 64-bit.  Page ids outside [0, num_pages) are read as
// scratch page 0, and an append with an out-of-range page or slot writes
// nothing: a malformed table can give wrong rows but never a fault.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kTau = 8.0f;   // lazy-rescale threshold, log2 units

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

// Sum over the 8 lanes of an aligned row group; every lane gets the total.
__device__ __forceinline__ float sum_row8(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp<0x141>(x);   // row_half_mirror: lane i <-> 7 - i within 8
    return x;
}

// Reductions across the 8 row groups of a wave (lanes with equal lane % 8).
__device__ __forceinline__ float max_across_rows(float x) {
    x = fmaxf(x, dpp<0x128>(x));        // row_ror:8 within 16 lanes = lane ^ 8
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}
__device__ __forceinline__ float sum_across_rows(float x) {
    x += dpp<0x128>(x);
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint4 load16(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// Tiles (8 tokens) of entry b; 0 for a malformed entry with no page.
__device__ __forceinline__ int entry_tiles(const DecodeArgs &a, int b) {
    const int n = a.indptr[b + 1] - a.indptr[b];
    if (n < 1)
        return 0;
    int last = a.last_len[b];
    last = last < 1 ? 1 : (last > a.page_size ? a.page_size : last);
    return ((n - 1) * a.page_size + last + kTileTokens - 1) / kTileTokens;
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

// ---------------------------------------------------------------------------
// Decode pass.
//
// A workgroup owns a run [g0, g1) of 8-token tiles in its entries' tiles laid
// end to end, and has one wave per KV head (blockIdx.y picks the group of up to
// kMaxWavesPerGroup heads).  Balanced mode (chunk_tiles == 0): W workgroups
// take equal runs of all T tiles of the batch.  Fixed mode: a workgroup takes
// run c of chunk_tiles tiles of one entry b alone.  Either way the entries
// are described in LDS (tile prefix sums, first page-table slot, tokens), so
// both modes run the same loop.
//
// The run is processed in pieces of at most kPiece tiles.  All threads first
// resolve every tile's page id into an LDS table, with an info word per tile
// (valid tokens, slot in the page, where entries start and end); then each
// wave streams the piece through three rotating one-tile register buffers
// (two tiles in flight while one is computed), switching entries where the
// info word says so.  Loads never wait on the page table, and the q rows of
// the piece's first entries are staged in LDS with the tables, so entry
// switches cost no memory round trip.  Every load is issued unconditionally
// (a tile past the piece reloads its last tile, a cache hit, and is never
// computed), so at each compute the same two tiles are outstanding on every
// path and the compiler's waits keep them in flight.
constexpr int kPiece = 256;
constexpr int kInfoNtok = 0xF;            // bits 0-3: valid tokens (1..8)
constexpr int kInfoSlotShift = 4;         // bits 4-8: slot of the tile's first token / 8
constexpr int kInfoSegFirst = 1 << 9;     // first tile of an entry within the run
constexpr int kInfoSegLast = 1 << 10;     // last tile of an entry within the run
constexpr int kInfoEntryLast = 1 << 11;   // the tile holding the entry's token L-1
constexpr int kInfoNewRowShift = 12;      // bits 12-14: token L-1 within that tile
constexpr int kInfoEntryShift = 16;       // bits 16-31: entry - first entry of piece

// Tiles of entry b; also its first page-table slot and token count.
__device__ __forceinline__ int entry_desc(const DecodeArgs &a, int b, int &p0, int &len) {
    p0 = a.indptr[b];
    const int n = a.indptr[b + 1] - p0;
    int last = a.last_len[b];
    last = last < 1 ? 1 : (last > a.page_size ? a.page_size : last);
    len = n < 1 ? 0 : (n - 1) * a.page_size + last;
    return (len + kTileTokens - 1) / kTileTokens;
}

// Ints of padding after the entry descriptors so the staged q rows, which
// follow the tile tables, start 16-byte aligned (the tables hold a multiple of
// 4 ints).
__host__ __device__ __forceinline__ int q_pad(int nb) { return (3 - (3 * nb) % 4) % 4; }

// The largest e in [lo, hi] with start[e] <= t (start non-decreasing).
__device__ __forceinline__ int entry_of(const int *start, int lo, int hi, int t) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

template <int D, int G, bool SMALL_PAGE>
__global__ __launch_bounds__(kMaxWavesPerGroup * 64) void decode_kernel(DecodeArgs a) {
    constexpr int NLD = D / 64;                      // 16-byte words per lane per row
    constexpr int PPT = SMALL_PAGE ? kTileTokens : 1;   // page ids per tile
    extern __shared__ uint4 smem_words[];
    int *smem = reinterpret_cast<int *>(smem_words);
    __shared__ int s_wave[17];
    const int lane = threadIdx.x & 63;
    const int rg = lane >> 3;     // token within a tile
    const int j = lane & 7;       // element slice [8j, 8j+8) (+64 for D = 128)
    const int h = __builtin_amdgcn_readfirstlane(blockIdx.y * (blockDim.x >> 6) +
                                                 (threadIdx.x >> 6));
    // Waves past the last head (when Hkv is not a multiple of the group size)
    // do no attention work but still take every barrier.
    const bool has_head = h < a.num_kv_heads;
    const bool fixed = a.chunk_tiles > 0;
    const bool fused = a.k_new != nullptr;
    const int nb = fixed ? 1 : a.batch;
    int *s_start = smem;              // [nb + 1] tile prefix sums
    int *s_p0 = s_start + nb + 1;     // [nb] first page-table slot
    int *s_len = s_p0 + nb;           // [nb] tokens
    int *s_page = s_len + nb;         // [kPiece * PPT] page ids of the piece's tiles
    int *s_info = s_page + kPiece * PPT;   // [kPiece] info words
    // q rows of the piece's first q_slots entries, [q_slots][Hq][D] bf16
    uint16_t *s_q = reinterpret_cast<uint16_t *>(s_info + kPiece + q_pad(nb));

    int g0, g1, fixed_b = 0, fixed_c = 0;
    if (fixed) {
        // Chunk-major order over rows of batch8 = batch rounded up to 8
        // workgroups, entries rotated by the chunk number.  Workgroups are
        // dealt to the 8 XCDs round-robin, so chunk c of entry b lands on XCD
        // (b - c) mod 8: consecutive chunks of an entry, and the first chunks
        // of all entries, spread over every XCD.  Ids past the batch are empty.
        const int batch8 = (a.batch + 7) & ~7;
        fixed_c = blockIdx.x / batch8;
        const int bp = blockIdx.x - fixed_c * batch8;
        fixed_b = (bp + fixed_c) % batch8;
        if (fixed_b >= a.batch)
            return;
        int p0, len;
        const int nt = entry_desc(a, fixed_b, p0, len);
        const int nchunks = (nt + a.chunk_tiles - 1) / a.chunk_tiles;
        if (nchunks > a.max_chunks) {
            // Longer than the launch allows: poison the rows so the broken
            // precondition shows instead of silently truncating.
            if (fixed_c == 0 && has_head) {
                for (int i = lane; i < G * D; i += 64)
                    a.out[((int64_t)fixed_b * a.num_qo_heads + h * G) * D + i] = 0x7FC0;
                if (a.lse != nullptr && lane < G)
                    a.lse[(int64_t)fixed_b * a.num_qo_heads + h * G + lane] = __builtin_nanf("");
            }
            return;
        }
        if (fixed_c >= nchunks)
            return;
        if (threadIdx.x == 0) {
            s_start[0] = 0;
            s_start[1] = nt;
            s_p0[0] = p0;
            s_len[0] = len;
        }
        g0 = fixed_c * a.chunk_tiles;
        g1 = min(nt, g0 + a.chunk_tiles);
        __syncthreads();
    } else {
        // Balanced: per-entry tiles, first slot and tokens, then prefix sums.
        const int nthreads = blockDim.x;
        const int per = (a.batch + nthreads - 1) / nthreads;
        const int e0 = min(a.batch, (int)threadIdx.x * per);
        const int e1 = min(a.batch, e0 + per);
        int local = 0;
        for (int e = e0; e < e1; ++e) {
            int p0, len;
            const int t = entry_desc(a, e, p0, len);
            s_start[e] = t;
            s_p0[e] = p0;
            s_len[e] = len;
            local += t;
        }
        int total = 0;
        int run = block_exclusive_scan(local, s_wave, total);
        for (int e = e0; e < e1; ++e) {
            const int t = s_start[e];
            s_start[e] = run;
            run += t;
        }
        if (threadIdx.x == 0)
            s_start[a.batch] = total;
        __syncthreads();
        if (blockIdx.x == 0 && blockIdx.y == 0)
            for (int e = threadIdx.x; e <= a.batch; e += nthreads)
                a.tile_start[e] = s_start[e];
        // W <= T workgroups take part, so each holds at least one tile (the
        // merge recomputes the same W from T)
        const int64_t T = total;
        const int W = (int)(T < a.num_groups ? T : a.num_groups);
        if ((int)blockIdx.x >= W)
            return;
        g0 = (int)(T * blockIdx.x / W);
        g1 = (int)(T * (blockIdx.x + 1) / W);
    }

    // ---- per-wave state, carried across pieces
    uint32_t qv[G][NLD][4];   // q of the entry being computed
    float m[G], l[G], acc[G][NLD][8];
    const int row_elems_q = a.num_qo_heads * D;

    for (int k0 = g0, k1; k0 < g1; k0 = k1) {
        // A piece: at most kPiece tiles of at most q_slots entries (so every
        // entry's q rows are staged).  Entry e_first holds tile k0, so
        // s_start[e_first + 1] > k0 and the piece is never empty.
        const int e_first = __builtin_amdgcn_readfirstlane(entry_of(s_start, 0, nb - 1, k0));
        k1 = min(g1, k0 + kPiece);
        if (e_first + a.q_slots < nb)
            k1 = min(k1, s_start[e_first + a.q_slots]);
        k1 = __builtin_amdgcn_readfirstlane(k1);
        const int nk = k1 - k0;
        __syncthreads();   // the previous piece's tables are no longer read
        for (int t = threadIdx.x; t < nk * PPT; t += blockDim.x) {
            const int kk = t / PPT;
            const int r = t % PPT;
            const int k = k0 + kk;
            const int e = entry_of(s_start, e_first, nb - 1, k);
            const int lt = k - s_start[e];
            const int tok0 = lt * kTileTokens;
            const int len = s_len[e];
            const int tok = tok0 + r;
            const int page_local = tok >> a.log2_page;
            int page = (tok < len) ? a.indices[s_p0[e] + page_local] : 0;
            page = (page >= 0 && page < a.num_pages) ? page : 0;
            s_page[t] = page;
            if (r == 0) {
                const int ntok = min(kTileTokens, len - tok0);
                const int slot8 = SMALL_PAGE ? 0 : ((tok0 & (a.page_size - 1)) >> 3);
                int info = ntok | (slot8 << kInfoSlotShift) |
                           (((len - 1) & (kTileTokens - 1)) << kInfoNewRowShift) |
                           ((e - e_first) << kInfoEntryShift);
                if (k == max(g0, s_start[e]))
                    info |= kInfoSegFirst;
                if (k == min(g1, s_start[e + 1]) - 1)
                    info |= kInfoSegLast;
                if (lt == (len - 1) / kTileTokens)
                    info |= kInfoEntryLast;
                s_info[kk] = info;
            }
        }
        {
            // q rows of the piece's entries, 16 bytes a thread
            const int e_last = entry_of(s_start, e_first, nb - 1, k1 - 1);
            const int nq = e_last - e_first + 1;   // <= q_slots
            const int words = row_elems_q >> 3;
            for (int t = threadIdx.x; t < nq * words; t += blockDim.x) {
                const int qe = t / words;
                const int w = t - qe * words;
                const int b = fixed ? fixed_b : e_first + qe;
                reinterpret_cast<uint4 *>(s_q + (int64_t)qe * row_elems_q)[w] =
                    reinterpret_cast<const uint4 *>(a.q + (int64_t)b * row_elems_q)[w];
            }
        }
        __syncthreads();
        if (!has_head)
            continue;

        struct Tile {
            uint4 k[NLD];
            uint4 v[NLD];
        };
        const uint16_t *head_base = a.cache + h * D + j * 8;

        auto load_tile = [&](Tile &x, int kk) {
            kk = min(kk, nk - 1);
            const int info = __builtin_amdgcn_readfirstlane(s_info[kk]);
            const uint16_t *row;
            if (SMALL_PAGE) {
                const int page = s_page[kk * PPT + rg];
                row = head_base + (int64_t)page * a.page_stride +
                      (uint32_t)((rg & (a.page_size - 1)) * a.row_stride);
            } else {
                const int page = __builtin_amdgcn_readfirstlane(s_page[kk]);
                const int sl = ((info >> kInfoSlotShift) & 31) * kTileTokens + rg;
                row = head_base + (int64_t)page * a.page_stride + (uint32_t)(sl * a.row_stride);
            }
            // One load sequence on every path (only the addresses differ), so
            // the compiler's waits keep two tiles in flight.
            const uint16_t *kr = row;
            const uint16_t *vr = row + a.half_stride;
            if (fused && (info & kInfoEntryLast) && rg == ((info >> kInfoNewRowShift) & 7)) {
                // the entry's new row comes from k_new / v_new
                const int b = fixed ? fixed_b : e_first + (info >> kInfoEntryShift);
                const int64_t nr = ((int64_t)b * a.num_kv_heads + h) * D + j * 8;
                kr = a.k_new + nr;
                vr = a.v_new + nr;
            }
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                x.k[i] = load16(kr + i * 64);
                x.v[i] = load16(vr + i * 64);
            }
        };

        auto begin_entry = [&](int e) {
            // q of the G query heads of KV head h, staged in LDS
            const uint16_t *qb = s_q + (e - e_first) * row_elems_q + h * G * D + j * 8;
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    const uint4 w = *reinterpret_cast<const uint4 *>(qb + g * D + i * 64);
                    qv[g][i][0] = w.x;
                    qv[g][i][1] = w.y;
                    qv[g][i][2] = w.z;
                    qv[g][i][3] = w.w;
                }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                m[g] = -INFINITY;
                l[g] = 0.f;
#pragma unroll
                for (int i = 0; i < NLD; ++i)
#pragma unroll
                    for (int e8 = 0; e8 < 8; ++e8)
                        acc[g][i][e8] = 0.f;
            }
        };

        auto finish_entry = [&](int e, int info, int kk) {
            const int b = fixed ? fixed_b : e;
            if (fused && (info & kInfoEntryLast) && rg == ((info >> kInfoNewRowShift) & 7)) {
                // append: copy the new row of head h into the cache slot
                int page, sl;
                if (SMALL_PAGE) {
                    page = s_page[kk * PPT + rg];
                    sl = rg & (a.page_size - 1);
                } else {
                    page = s_page[kk];
                    sl = ((info >> kInfoSlotShift) & 31) * kTileTokens + rg;
                }
                const int64_t nr = ((int64_t)b * a.num_kv_heads + h) * D + j * 8;
                uint16_t *dst = a.cache_w + h * D + j * 8 + (int64_t)page * a.page_stride +
                                (int64_t)sl * a.row_stride;
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    *reinterpret_cast<uint4 *>(dst + i * 64) = load16(a.k_new + nr + i * 64);
                    *reinterpret_cast<uint4 *>(dst + a.half_stride + i * 64) =
                        load16(a.v_new + nr + i * 64);
                }
            }
            // merge the 8 row groups; every lane ends with the totals
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float mw = max_across_rows(m[g]);
                const float f = (m[g] == -INFINITY) ? 0.f : exp2_fast(m[g] - mw);
                l[g] = sum_across_rows(l[g] * f);
#pragma unroll
                for (int i = 0; i < NLD; ++i)
#pragma unroll
                    for (int e8 = 0; e8 < 8; ++e8)
                        acc[g][i][e8] = sum_across_rows(acc[g][i][e8] * f);
                m[g] = mw;
            }
            const bool whole = s_start[e] >= g0 && s_start[e + 1] <= g1;
            const int slot = fixed ? fixed_b * a.max_chunks + fixed_c : (int)blockIdx.x + e;
            // row group g writes query head h * G + g
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (rg != g)
                    continue;
                const int hq = h * G + g;
                const float inv = 1.f / l[g];
                if (whole) {
                    uint16_t *o = a.out + ((int64_t)b * a.num_qo_heads + hq) * D + j * 8;
#pragma unroll
                    for (int i = 0; i < NLD; ++i) {
                        uint4 w;
                        w.x = pack_bf16x2(acc[g][i][0] * inv, acc[g][i][1] * inv);
                        w.y = pack_bf16x2(acc[g][i][2] * inv, acc[g][i][3] * inv);
                        w.z = pack_bf16x2(acc[g][i][4] * inv, acc[g][i][5] * inv);
                        w.w = pack_bf16x2(acc[g][i][6] * inv, acc[g][i][7] * inv);
                        *reinterpret_cast<uint4 *>(o + i * 64) = w;
                    }
                    if (a.lse != nullptr && j == 0)
                        a.lse[(int64_t)b * a.num_qo_heads + hq] =
                            (m[g] + log2_fast(l[g])) * kLn2;
                } else {
                    const int64_t prow = (int64_t)slot * a.num_qo_heads + hq;
                    float *o = a.part_o + prow * D + j * 8;
#pragma unroll
                    for (int i = 0; i < NLD; ++i) {
                        *reinterpret_cast<float4 *>(o + i * 64) =
                            make_float4(acc[g][i][0] * inv, acc[g][i][1] * inv,
                                        acc[g][i][2] * inv, acc[g][i][3] * inv);
                        *reinterpret_cast<float4 *>(o + i * 64 + 4) =
                            make_float4(acc[g][i][4] * inv, acc[g][i][5] * inv,
                                        acc[g][i][6] * inv, acc[g][i][7] * inv);
                    }
                    if (j == 0)
                        a.part_lse[prow] = m[g] + log2_fast(l[g]);
                }
            }
        };

        auto compute_tile = [&](const Tile &x, int kk) {
            const int info = __builtin_amdgcn_readfirstlane(s_info[kk]);
            const int e = e_first + (info >> kInfoEntryShift);
            if (info & kInfoSegFirst)
                begin_entry(e);
            const int ntok = info & kInfoNtok;
            const bool edge = ntok < kTileTokens;
            const bool ok = rg < ntok;
            float s[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    d = dot2_bf16(qv[g][i][0], x.k[i].x, d);
                    d = dot2_bf16(qv[g][i][1], x.k[i].y, d);
                    d = dot2_bf16(qv[g][i][2], x.k[i].z, d);
                    d = dot2_bf16(qv[g][i][3], x.k[i].w, d);
                }
                s[g] = sum_row8(d) * a.scale_log2;
                if (edge)
                    s[g] = ok ? s[g] : -INFINITY;
            }
            // Lazy maximum: raise m only when a score passes it by more than kTau.
            bool raise_any = false;
#pragma unroll
            for (int g = 0; g < G; ++g)
                raise_any |= s[g] > m[g] + kTau;
            if (raise_any) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const bool up = s[g] > m[g] + kTau;
                    const float mn = up ? s[g] : m[g];
                    const float alpha = up ? exp2_fast(m[g] - mn) : 1.f;
                    m[g] = mn;
                    l[g] *= alpha;
#pragma unroll
                    for (int i = 0; i < NLD; ++i)
#pragma unroll
                        for (int e8 = 0; e8 < 8; ++e8)
                            acc[g][i][e8] *= alpha;
                }
            }
            float vf[NLD][8];
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const uint4 w = x.v[i];
                vf[i][0] = bf16_lo(w.x);
                vf[i][1] = bf16_hi(w.x);
                vf[i][2] = bf16_lo(w.y);
                vf[i][3] = bf16_hi(w.y);
                vf[i][4] = bf16_lo(w.z);
                vf[i][5] = bf16_hi(w.z);
                vf[i][6] = bf16_lo(w.w);
                vf[i][7] = bf16_hi(w.w);
            }
            if (edge && !ok) {
                // stale rows past the end may hold anything, NaN included
#pragma unroll
                for (int i = 0; i < NLD; ++i)
#pragma unroll
                    for (int e8 = 0; e8 < 8; ++e8)
                        vf[i][e8] = 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float p = exp2_fast(s[g] - m[g]);
                if (edge)
                    p = ok ? p : 0.f;   // also covers -inf - -inf
                l[g] += p;
#pragma unroll
                for (int i = 0; i < NLD; ++i)
#pragma unroll
                    for (int e8 = 0; e8 < 8; ++e8)
                        acc[g][i][e8] = fmaf(p, vf[i][e8], acc[g][i][e8]);
            }
            if (info & kInfoSegLast)
                finish_entry(e, info, kk);
        };

        Tile A, B, C;
        load_tile(A, 0);
        load_tile(B, 1);
        for (int kk = 0;;) {
            load_tile(C, kk + 2);
            compute_tile(A, kk);
            if (++kk >= nk)
                break;
            load_tile(A, kk + 2);
            compute_tile(B, kk);
            if (++kk >= nk)
                break;
            load_tile(B, kk + 2);
            compute_tile(C, kk);
            if (++kk >= nk)
                break;
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of entries split over several workgroups or chunks: one workgroup per
// (entry, KV head).  Thread (col, ks) owns float4 column `col` of the G query
// heads' outputs and the partials k = ks, ks + KS, ...; it merges them online
// (running maximum, rescaled sum) with the loads of four partials in flight,
// and the KS per-thread states are then merged through LDS.
template <int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
    constexpr int COLS = G * D / 4;                    // float4 columns
    constexpr int KS = COLS >= 256 ? 1 : 256 / COLS;   // ways the partials are split
    constexpr int U = 4;                               // partials in flight per thread
    __shared__ float s_m[KS][COLS];
    __shared__ float s_s[KS][COLS];
    __shared__ float4 s_o[KS][COLS];

    const int h = blockIdx.x % a.num_kv_heads;
    const int b = blockIdx.x / a.num_kv_heads;
    int base, count;
    if (a.chunk_tiles > 0) {
        const int nt = entry_tiles(a, b);
        const int nchunks = (nt + a.chunk_tiles - 1) / a.chunk_tiles;
        if (nchunks <= 1 || nchunks > a.max_chunks)
            return;
        base = b * a.max_chunks;
        count = nchunks;
    } else {
        const int sb = a.tile_start[b];
        const int se = a.tile_start[b + 1];
        const int64_t T = a.tile_start[a.batch];
        if (se <= sb)
            return;
        const int64_t W = T < a.num_groups ? T : a.num_groups;
        // workgroup w covers tiles [floor(T w / W), floor(T (w+1) / W)), and
        // none of them is empty since W <= T
        const int w_lo = (int)(((int64_t)(sb + 1) * W - 1) / T);
        const int w_hi = (int)(((int64_t)se * W - 1) / T);
        if (w_lo == w_hi)
            return;
        base = w_lo + b;
        count = w_hi - w_lo + 1;
    }
    const int col = threadIdx.x % COLS;
    const int ks = threadIdx.x / COLS;
    const int g = col / (D / 4);
    const int e4 = (col % (D / 4)) * 4;
    const int hq = h * G + g;
    const int64_t stride_l = a.num_qo_heads;
    const int64_t stride_o = (int64_t)a.num_qo_heads * D;
    const float *pl = a.part_lse + (int64_t)base * stride_l + hq;
    const float *po = a.part_o + (int64_t)base * stride_o + (int64_t)hq * D + e4;

    float m = -INFINITY, sum = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ks < KS) {
        for (int k0 = ks; k0 < count; k0 += KS * U) {
            float lv[U];
            float4 ov[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = min(k0 + u * KS, count - 1);
                lv[u] = pl[k * stride_l];
                ov[u] = *reinterpret_cast<const float4 *>(po + k * stride_o);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (k0 + u * KS >= count)
                    break;
                const float mn = fmaxf(m, lv[u]);
                const float al = exp2_fast(m - mn);   // 0 while m is -inf
                const float w = exp2_fast(lv[u] - mn);
                sum = sum * al + w;
                o.x = fmaf(w, ov[u].x, o.x * al);
                o.y = fmaf(w, ov[u].y, o.y * al);
                o.z = fmaf(w, ov[u].z, o.z * al);
                o.w = fmaf(w, ov[u].w, o.w * al);
                m = mn;
            }
        }
        if (KS > 1) {
            s_m[ks][col] = m;
            s_s[ks][col] = sum;
            s_o[ks][col] = o;
        }
    }
    if (KS > 1) {
        __syncthreads();
        if (ks != 0)
            return;
        m = -INFINITY;
#pragma unroll
        for (int q = 0; q < KS; ++q)
            m = fmaxf(m, s_m[q][col]);
        sum = 0.f;
        o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            const float mq = s_m[q][col];
            const float f = mq == -INFINITY ? 0.f : exp2_fast(mq - m);
            const float4 oq = s_o[q][col];
            sum = fmaf(s_s[q][col], f, sum);
            o.x = fmaf(oq.x, f, o.x);
            o.y = fmaf(oq.y, f, o.y);
            o.z = fmaf(oq.z, f, o.z);
            o.w = fmaf(oq.w, f, o.w);
        }
    }
    if (col >= COLS)
        return;
    const float inv = 1.f / sum;
    uint2 packed;
    packed.x = pack_bf16x2(o.x * inv, o.y * inv);
    packed.y = pack_bf16x2(o.z * inv, o.w * inv);
    *reinterpret_cast<uint2 *>(a.out + ((int64_t)b * a.num_qo_heads + hq) * D + e4) = packed;
    if (a.lse != nullptr && e4 == 0)
        a.lse[(int64_t)b * a.num_qo_heads + hq] = (m + log2_fast(sum)) * kLn2;
}

#ifndef PKV_WAVES_PER_CU
#define PKV_WAVES_PER_CU 0   // 0: as many as the occupancy calculator allows
#endif

// Launch through hipLaunchKernel so the returned status belongs to this
// launch alone (hipGetLastError could report an older, unrelated error).
template <typename Args>
hipError_t launch(const void *kernel, dim3 grid, dim3 block, size_t lds, const Args &args,
                  hipStream_t stream) {
    void *params[] = {const_cast<Args *>(&args)};
    return hipLaunchKernel(kernel, grid, block, params, lds, stream);
}

template <int D, int G>
const void *decode_kernel_for(int page_size) {
    return page_size < kTileTokens
               ? reinterpret_cast<const void *>(&decode_kernel<D, G, true>)
               : reinterpret_cast<const void *>(&decode_kernel<D, G, false>);
}

template <int D>
const void *decode_kernel_d(int group, int page_size) {
    switch (group) {
    case 1: return decode_kernel_for<D, 1>(page_size);
    case 2: return decode_kernel_for<D, 2>(page_size);
    case 3: return decode_kernel_for<D, 3>(page_size);
    case 4: return decode_kernel_for<D, 4>(page_size);
    case 5: return decode_kernel_for<D, 5>(page_size);
    case 6: return decode_kernel_for<D, 6>(page_size);
    case 7: return decode_kernel_for<D, 7>(page_size);
    case 8: return decode_kernel_for<D, 8>(page_size);
    default: return nullptr;
    }
}

const void *decode_kernel_ptr(int head_dim, int group, int page_size) {
    if (head_dim == 64)
        return decode_kernel_d<64>(group, page_size);
    if (head_dim == 128)
        return decode_kernel_d<128>(group, page_size);
    return nullptr;
}

template <int D>
const void *merge_kernel_d(int group) {
    switch (group) {
    case 1: return reinterpret_cast<const void *>(&merge_kernel<D, 1>);
    case 2: return reinterpret_cast<const void *>(&merge_kernel<D, 2>);
    case 3: return reinterpret_cast<const void *>(&merge_kernel<D, 3>);
    case 4: return reinterpret_cast<const void *>(&merge_kernel<D, 4>);
    case 5: return reinterpret_cast<const void *>(&merge_kernel<D, 5>);
    case 6: return reinterpret_cast<const void *>(&merge_kernel<D, 6>);
    case 7: return reinterpret_cast<const void *>(&merge_kernel<D, 7>);
    case 8: return reinterpret_cast<const void *>(&merge_kernel<D, 8>);
    default: return nullptr;
    }
}

// Dynamic LDS of the decode kernel: entry descriptors of nb entries, the
// piece's tile tables, and q_slots staged q rows of q_row_bytes each.
size_t decode_lds_bytes(int nb, int page_size, int q_slots, int q_row_bytes) {
    const size_t ppt = page_size < kTileTokens ? kTileTokens : 1;
    const size_t ints = (size_t)3 * nb + 1 + (size_t)kPiece * (ppt + 1) + q_pad(nb);
    return sizeof(int) * ints + (size_t)q_slots * q_row_bytes;
}

int group_waves(int num_kv_heads) {
    return num_kv_heads < kMaxWavesPerGroup ? num_kv_heads : kMaxWavesPerGroup;
}

// q rows staged per piece: at most 8 and no more than the entries a
// workgroup can see, within 32 KiB and a 64 KiB total for the workgroup's
// LDS (0 when not even one fits: q is then read from memory).
int decode_q_slots(int nb, int page_size, int q_row_bytes) {
    const int64_t tables = (int64_t)decode_lds_bytes(nb, page_size, 0, q_row_bytes);
    int64_t budget = (int64_t)(64 << 10) - tables;
    budget = budget < (32 << 10) ? budget : (32 << 10);
    int64_t n = budget > 0 ? budget / q_row_bytes : 0;
    n = n > 8 ? 8 : n;
    return (int)(n < nb ? n : nb);
}

size_t decode_lds_for(int nb, int page_size, int num_qo_heads, int head_dim) {
    const int row = num_qo_heads * head_dim * 2;
    return decode_lds_bytes(nb, page_size, decode_q_slots(nb, page_size, row), row);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream) {
    return launch(reinterpret_cast<const void *>(&append_kernel), dim3((unsigned)batch),
                  dim3(256), 0, a, stream);
}

hipError_t balanced_groups(int head_dim, int group, int num_kv_heads, int page_size,
                           int batch, int *groups) {
    const int num_qo_heads = group * num_kv_heads;
    const void *k = decode_kernel_ptr(head_dim, group, page_size);
    if (k == nullptr)
        return hipErrorInvalidValue;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess)
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, k, 64 * group_waves(num_kv_heads),
            decode_lds_for(batch, page_size, num_qo_heads, head_dim));
    if (err != hipSuccess)
        return err;
    const int waves = group_waves(num_kv_heads);
    const int head_groups = (num_kv_heads + waves - 1) / waves;
    if (PKV_WAVES_PER_CU > 0)
        per_cu = (PKV_WAVES_PER_CU + waves - 1) / waves;
    if (per_cu < 1)
        per_cu = 1;
    if (cus > kMaxComputeUnits)
        cus = kMaxComputeUnits;
    // workgroups resident at once, shared by the head groups
    int64_t w = ((int64_t)cus * per_cu + head_groups - 1) / head_groups;
    const int64_t bound = balanced_groups_bound(num_kv_heads);
    *groups = (int)(w < bound ? w : bound);
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &args, int head_dim, int group, hipStream_t stream) {
    DecodeArgs a = args;
    const int nb = a.chunk_tiles > 0 ? 1 : a.batch;
    const int q_row = a.num_qo_heads * head_dim * 2;
    a.q_slots = decode_q_slots(nb, a.page_size, q_row);
    const size_t lds = decode_lds_bytes(nb, a.page_size, a.q_slots, q_row);
    const void *k = decode_kernel_ptr(head_dim, group, a.page_size);
    const void *mk = head_dim == 64 ? merge_kernel_d<64>(group)
                                    : (head_dim == 128 ? merge_kernel_d<128>(group) : nullptr);
    if (k == nullptr || mk == nullptr)
        return hipErrorInvalidValue;
    const int waves = group_waves(a.num_kv_heads);
    const dim3 block(64 * waves);
    const unsigned head_groups = (unsigned)((a.num_kv_heads + waves - 1) / waves);
    hipError_t err;
    bool may_split;
    if (a.chunk_tiles > 0) {
        const unsigned batch8 = ((unsigned)a.batch + 7u) & ~7u;
        err = launch(k, dim3(batch8 * (unsigned)a.max_chunks, head_groups), block,
                     lds, a, stream);
        may_split = a.max_chunks > 1;
    } else {
        err = launch(k, dim3((unsigned)a.num_groups, head_groups), block,
                     lds, a, stream);
        may_split = true;
    }
    if (err != hipSuccess || !may_split)
        return err;
    // COLS float4 columns times KS ways: 256 threads for every built shape
    // (COLS = group * head_dim / 4 divides 256 or exceeds it)
    const int cols = group * head_dim / 4;
    const int threads = cols >= 256 ? ((cols + 63) / 64) * 64 : (256 / cols) * cols;
    return launch(mk, dim3((unsigned)a.batch * a.num_kv_heads), dim3(threads), 0, a, stream);
}

}  // namespace pkv
