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
// the keys and values).  A workgroup of four waves takes 128 consecutive
// columns, 32 per wave in two blocks of 16, and walks the entry's tokens up
// to its last column's position in tiles of 32:
//   S^T[t][c] = sum_d K[t][d] Q[c][d]     K tile as the A operand (from LDS),
//                                         Q^T as the B operand (registers)
//   O^T[d][c] += sum_t V^T[d][t] P^T[t][c] V^T from LDS, P^T from the scores
// The MFMA gives lane l the scores of column l % 16 at tokens 4 (l / 16) + r
// of each 16-token half of the tile, which is exactly a B operand of the
// second product when its contraction index k = 8 (l / 16) + e names token
// 4 (l / 16) + e (e < 4) or 16 + 4 (l / 16) + e - 4 (e >= 4) (the order of a
// sum is free); V^T is read in the same token order.  The online softmax of
// a column stays within its four lanes.  P goes in as a bf16 high part and a
// bf16 remainder (two products): a single bf16 P is off by up to half a
// bf16 step of the output, the whole parity bar.
//
// The four waves share each tile's K rows and its V rows, transposed, in
// LDS (two buffers: the next tile's loads are in flight while one is
// computed).  Rows are padded so that the operand reads meet distinct banks.
// The grid lists (entry, KV head) pairs fastest, so the heaviest tiles (the
// last columns, the longest prefixes) of every pair start first and, with
// 8 | batch x Hkv, all tiles of a pair run on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_launch.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kMaskedScore = -1e30f;   // log2-domain score of a masked token
constexpr float kTau = 8.0f;             // lazy-rescale threshold, log2 units
constexpr int kTileTok = 32;             // tokens per tile
constexpr int kCols = 128;               // query columns per workgroup
constexpr int kThreads = 256;            // four waves
constexpr int kStagePages = 1024;        // page ids of an entry held in LDS

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 (round to nearest even), packed low-first: one
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo_up(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_up(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column's
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
// Append of several rows per entry: workgroup (j, b) copies row j of entry b,
// if it exists, into token position L - n_b + j.
__global__ __launch_bounds__(256) void append_rows_kernel(PrefillArgs a) {
    const int j = blockIdx.x, b = blockIdx.y;
    const int r0 = a.qo_indptr[b];
    const int n = a.qo_indptr[b + 1] - r0;
    if (j >= n)
        return;
    const int p0 = a.indptr[b];
    const int np = a.indptr[b + 1] - p0;
    const int last = a.last_len[b];
    if (np < 1 || last < 1 || last > a.page_size)
        return;
    const int len = (np - 1) * a.page_size + last;
    if (n > len)
        return;
    const int t = len - n + j;
    const int page = a.indices[p0 + t / a.page_size];
    if (page < 0 || page >= a.num_pages)
        return;
    uint16_t *dst = a.cache_w + (int64_t)page * a.page_stride +
                    (int64_t)(t % a.page_size) * a.row_stride;
    const uint16_t *ks = a.k_new + (int64_t)(r0 + j) * a.row_stride;
    const uint16_t *vs = a.v_new + (int64_t)(r0 + j) * a.row_stride;
    const int words = a.row_stride >> 3;   // 16-byte words per row
    for (int i = threadIdx.x; i < 2 * words; i += blockDim.x) {
        const bool is_v = i >= words;
        const int w = is_v ? i - words : i;
        const uint4 val = reinterpret_cast<const uint4 *>(is_v ? vs : ks)[w];
        reinterpret_cast<uint4 *>(dst + (is_v ? a.half_stride : 0))[w] = val;
    }
}

// ---------------------------------------------------------------------------
// Causal attention of the new rows; see the file comment.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
    constexpr int DC = D / 32;                 // 32-value chunks of d (first product)
    constexpr int DB = D / 16;                 // 16-row blocks of d (second product)
    constexpr int KP = 2 * D + 16;             // LDS bytes per K row (padded)
    constexpr int VP = 2 * kTileTok + 16;      // LDS bytes per V^T row (padded)
    constexpr int CR = D / 8;                  // 16-byte chunks per K (or V) row
    constexpr int KPT = kTileTok * CR / kThreads;   // K chunks per thread per tile
    constexpr int VJOBS = (kTileTok / 2) * CR;       // V jobs: (token pair, chunk)
    static_assert(KPT >= 1 && VJOBS <= kThreads, "unsupported head_dim");
    __shared__ __attribute__((aligned(16))) char sk[2][kTileTok * KP];
    __shared__ __attribute__((aligned(16))) char sv[2][D * VP];
    __shared__ int s_pages[kStagePages];   // the entry's page list, when it fits

    const int pairs = a.batch * a.num_kv_heads;
    const int pair = blockIdx.x % pairs;
    const int trev = blockIdx.x / pairs;       // 0: the entry's last (heaviest) tile
    const int b = pair / a.num_kv_heads, h = pair - b * a.num_kv_heads;
    const int G = a.num_qo_heads / a.num_kv_heads;

    const int r0 = a.qo_indptr[b];
    const int n = a.qo_indptr[b + 1] - r0;
    if (n < 1 || (n == 1 && a.skip_single))
        return;
    const int ncols = n * G;
    const int ntile = (ncols + kCols - 1) / kCols;
    if (trev >= ntile)
        return;
    const int p0 = a.indptr[b];
    const int np = a.indptr[b + 1] - p0;
    const int last = a.last_len[b];
    if (np < 1 || last < 1 || last > a.page_size)
        return;
    const int len = (np - 1) * a.page_size + last;
    if (n > len)
        return;
    const int col0 = (ntile - 1 - trev) * kCols;
    const int pmax = len - n + (min(ncols, col0 + kCols) - 1) / G;   // last position
    const int32_t *pages = a.indices + p0;

    const int tid = threadIdx.x;
    const int wv = tid >> 6, l = tid & 63;
    const int q = l >> 4, c = l & 15;

    // this lane's two columns (blocks cb = 0, 1 of the wave's 32)
    int crow[2], chead[2], cpos[2];
    bool cok[2];
    bf16x8_t qb[2][DC];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int col = col0 + 32 * wv + 16 * cb + c;
        cok[cb] = col < ncols;
        crow[cb] = cok[cb] ? col / G : 0;
        chead[cb] = cok[cb] ? h * G + col % G : 0;
        cpos[cb] = cok[cb] ? len - n + crow[cb] : -1;
        const uint4 *src = reinterpret_cast<const uint4 *>(
            a.q + ((int64_t)(r0 + crow[cb]) * a.num_qo_heads + chead[cb]) * D + 8 * q);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            qb[cb][dc] = as_bf16x8(cok[cb] ? src[4 * dc] : make_uint4(0u, 0u, 0u, 0u));
    }
    // smallest position among the wave's valid columns (the first column's:
    // positions grow with the column)
    const int wave_min_pos = len - n + min(col0 + 32 * wv, ncols - 1) / G;
    f32x4_t o[2][DB];
    float m[2], lsum[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
            o[cb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m[cb] = kMaskedScore;   // running maximum of the column (log2 domain)
        lsum[cb] = 0.f;         // this lane's share of the column's weight sum
    }
    const float c2 = a.scale_log2;

    // Global -> register loads of one tile: K chunks tid + 256 i (row = id /
    // CR), and V as (token pair, chunk) jobs for the transposed store.  Tokens
    // past the entry's end read its last token again (finite; masked).
    const uint16_t *kbase = a.cache + (int64_t)h * D;
    // the page ids the walk needs, staged once (a tile's loads then wait for
    // no page-table read)
    const bool staged = np <= kStagePages;
    if (staged)
        for (int i = tid; i < np; i += kThreads) {
            const int page = pages[i];
            s_pages[i] = (page >= 0 && page < a.num_pages) ? page : 0;   // bad table: no fault
        }
    __syncthreads();
    const int pmask = a.page_size - 1;   // page sizes are powers of two
    auto row_ptr = [&](int t) {
        t = min(t, len - 1);
        int page;
        if (staged) {
            page = s_pages[t >> a.page_shift];
        } else {
            page = pages[t >> a.page_shift];
            page = (page >= 0 && page < a.num_pages) ? page : 0;
        }
        return kbase + (int64_t)page * a.page_stride + (int64_t)(t & pmask) * a.row_stride;
    };
    // Two register sets of tile loads in flight: the loads of tile t are
    // issued while tile t - 3 is computed and stored to LDS while tile t - 1
    // is; past the last tile they read its last tokens again (unconditional,
    // so the waits for the older set stay exact).
    uint4 kr[2][KPT], vr[2][2];
    auto load_tile = [&](auto setc, int t0) {
        constexpr int S = decltype(setc)::value;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int id = tid + kThreads * i;
            kr[S][i] = reinterpret_cast<const uint4 *>(row_ptr(t0 + id / CR))[id % CR];
        }
        if (tid < VJOBS) {
            const int tp = tid % (kTileTok / 2), ch = tid / (kTileTok / 2);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                vr[S][u] = reinterpret_cast<const uint4 *>(row_ptr(t0 + 2 * tp + u) +
                                                           a.half_stride)[ch];
        }
    };
    // Registers -> LDS buffer: K rows as they are; V transposed, V^T[d][t]
    // with the token pair (2 tp, 2 tp + 1) as one 4-byte word per d.
    auto store_tile = [&](auto setc, int buf) {
        constexpr int S = decltype(setc)::value;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int id = tid + kThreads * i;
            *reinterpret_cast<uint4 *>(sk[buf] + (id / CR) * KP + (id % CR) * 16) = kr[S][i];
        }
        if (tid < VJOBS) {
            const int tp = tid % (kTileTok / 2), ch = tid / (kTileTok / 2);
            const uint32_t a0[4] = {vr[S][0].x, vr[S][0].y, vr[S][0].z, vr[S][0].w};
            const uint32_t a1[4] = {vr[S][1].x, vr[S][1].y, vr[S][1].z, vr[S][1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // d = 8 ch + 2 e (low halves) and 8 ch + 2 e + 1 (high halves)
                const uint32_t lo = (a0[e] & 0xFFFFu) | (a1[e] << 16);
                const uint32_t hi = (a0[e] >> 16) | (a1[e] & 0xFFFF0000u);
                char *dst = sv[buf] + (8 * ch + 2 * e) * VP + 4 * tp;
                *reinterpret_cast<uint32_t *>(dst) = lo;
                *reinterpret_cast<uint32_t *>(dst + VP) = hi;
            }
        }
    };

    const int ntiles = pmax / kTileTok + 1;
    auto tile_t0 = [&](int i) { return min(i, ntiles - 1) * kTileTok; };
    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;
    auto compute_tile = [&](int it, int buf) {
        const int t0 = it * kTileTok;
        const char *kb = sk[buf];
        const char *vb = sv[buf];
        // S^T blocks: tokens 16 tb + (rows of the MFMA), columns of block cb
        f32x4_t s[2][2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            bf16x8_t ka[DC];
#pragma unroll
            for (int dc = 0; dc < DC; ++dc)
                ka[dc] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    kb + (16 * tb + c) * KP + (32 * dc + 8 * q) * 2));
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dc = 0; dc < DC; ++dc)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[dc], qb[cb][dc], acc, 0, 0, 0);
                s[tb][cb] = acc;
            }
        }
        // online softmax per column; P^T operands in the token order above.
        // Tiles wholly below every position of the wave need no mask.
        const bool masked = t0 + kTileTok - 1 > wave_min_pos;
        bf16x8_t phi[2], plo[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            float x[8];
            float tmax = kMaskedScore;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = t0 + 16 * tb + 4 * q + r;
                    float v = s[tb][cb][r] * c2;
                    if (masked)
                        v = (t <= cpos[cb]) ? v : kMaskedScore;
                    x[4 * tb + r] = v;
                    tmax = fmaxf(tmax, v);
                }
            // lazy maximum: raised (to the tile's column maximum) only when a
            // score passes it by more than kTau, so weights stay below
            // 2^kTau and most tiles rescale nothing
            if (__builtin_amdgcn_ballot_w64(tmax > m[cb] + kTau) != 0) {
                tmax = column_max(tmax);
                const float mn = fmaxf(m[cb], tmax);
                const float alpha = __builtin_amdgcn_exp2f(m[cb] - mn);
                m[cb] = mn;
                lsum[cb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[cb][db] *= alpha;
            }
            const float mn = m[cb];
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = __builtin_amdgcn_exp2f(x[e] - mn);
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
        // O^T += V^T P^T: lane reads V^T[16 db + c] at tokens 4 q .. 4 q + 3
        // and 16 + 4 q .. 16 + 4 q + 3
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const char *row = vb + (16 * db + c) * VP + 8 * q;
            const uint2 v0 = *reinterpret_cast<const uint2 *>(row);
            const uint2 v1 = *reinterpret_cast<const uint2 *>(row + 32);
            const bf16x8_t va = __builtin_bit_cast(bf16x8_t, u32x4_t{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                o[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi[cb], o[cb][db], 0, 0, 0);
                o[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo[cb], o[cb][db], 0, 0, 0);
            }
        }
    };
    load_tile(Set0{}, 0);
    store_tile(Set0{}, 0);
    __syncthreads();
    load_tile(Set1{}, tile_t0(1));
    load_tile(Set0{}, tile_t0(2));
    for (int it = 0; it < ntiles; it += 2) {
        // even tile from buffer 0; tile it + 1 (set 1) to buffer 1, then set 1
        // fetches tile it + 3
        compute_tile(it, 0);
        if (it + 1 >= ntiles)
            break;
        store_tile(Set1{}, 1);
        __syncthreads();
        load_tile(Set1{}, tile_t0(it + 3));
        // odd tile from buffer 1; tile it + 2 (set 0) to buffer 0, set 0
        // fetches tile it + 4
        compute_tile(it + 1, 1);
        if (it + 2 >= ntiles)
            break;
        store_tile(Set0{}, 0);
        __syncthreads();
        load_tile(Set0{}, tile_t0(it + 4));
    }

#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        // the column's weight sum over its four lanes, then the outputs
        const float ls = column_sum(lsum[cb]);
        if (!cok[cb])
            continue;
        const float inv = 1.f / ls;
        uint16_t *orow = a.out + ((int64_t)(r0 + crow[cb]) * a.num_qo_heads + chead[cb]) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            // lane holds O^T[16 db + 4 q + r][c]
            const uint32_t w0 = bf16x2_rne(o[cb][db][0] * inv, o[cb][db][1] * inv);
            const uint32_t w1 = bf16x2_rne(o[cb][db][2] * inv, o[cb][db][3] * inv);
            *reinterpret_cast<uint2 *>(orow + 16 * db + 4 * q) = make_uint2(w0, w1);
        }
        if (a.lse != nullptr && q == 0)
            a.lse[(int64_t)(r0 + crow[cb]) * a.num_qo_heads + chead[cb]] =
                (m[cb] + __log2f(ls)) * 0.6931471805599453f;
    }
}

}  // namespace

bool prefill_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_prefill(const PrefillArgs &a, bool append, hipStream_t stream) {
    PrefillArgs args = a;
    void *params[] = {&args};
    if (!prefill_supported(a.head_dim) || a.batch > 65535 || a.num_kv_heads > 65535)
        return hipErrorInvalidValue;
    hipError_t err = hipSuccess;
    if (append) {
        err = hipLaunchKernel(reinterpret_cast<const void *>(&append_rows_kernel),
                              dim3((unsigned)a.max_rows, (unsigned)a.batch), dim3(256), params,
                              0, stream);
        if (err != hipSuccess)
            return err;
    }
    const int G = a.num_qo_heads / a.num_kv_heads;
    const int64_t tiles = ((int64_t)a.max_rows * G + kCols - 1) / kCols;
    const int64_t blocks = tiles * a.batch * a.num_kv_heads;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const void *k = a.head_dim == 128 ? reinterpret_cast<const void *>(&prefill_kernel<128>)
                                      : reinterpret_cast<const void *>(&prefill_kernel<64>);
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(kThreads), params, 0, stream);
}

}  // namespace pkv
