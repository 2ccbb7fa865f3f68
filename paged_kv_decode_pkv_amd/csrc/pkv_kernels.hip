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
//    not MFMA.  q.k runs on v_dot2_f32_bf16 straight from the bf16 words:
//    no conversion of K, products exact, fp32 accumulation.
//  * Eight lanes cover one token row of one KV head; each lane owns D/8
//    contiguous elements.  One 16-byte load per lane then reads 8 whole rows
//    of 128 bytes (D = 64) or the first or second half of 8 rows of 256 bytes
//    (D = 128): every request is full cache-line segments.
//  * The 8-lane partial dot products are summed with three DPP steps
//    (quad_perm, quad_perm, row_half_mirror), so every lane of a row holds
//    the score without LDS traffic.
//  * Each group of 8 lanes (a "row group") keeps its own online-softmax state
//    in the exp2 domain.  The running maximum is raised only when a new score
//    exceeds it by more than kTau (log2 units): between raises no rescaling
//    is done, and exp2 arguments stay <= kTau, so nothing overflows.
//  * A workgroup owns one (entry, KV head, chunk of pages); its waves take
//    the chunk's 8-token tiles round robin with a two-block register
//    pipeline (the next block's loads are in flight while the current one is
//    computed).  Row groups and waves are merged through DPP/LDS at the end.
//  * A chunk is a fixed run of pages, so how an entry is split depends only
//    on its own length: results do not depend on the rest of the batch.
//    Entries with one chunk write bf16 out / fp32 lse directly; longer ones
//    write fp32 partials that the merge kernel combines by log-sum-exp.
//
// All cache offsets are 64-bit.  Page ids outside [0, num_pages) are read as
// scratch page 0 and an append with an out-of-range page or slot writes
// nothing, so a malformed table can give wrong rows but never a fault.

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
__device__ __forceinline__ float xor_rows(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}
__device__ __forceinline__ float max_across_rows(float x) {
    x = fmaxf(x, dpp<0x128>(x));        // row_ror:8 within 16 lanes = lane ^ 8
    x = fmaxf(x, xor_rows(x, 16));
    x = fmaxf(x, xor_rows(x, 32));
    return x;
}
__device__ __forceinline__ float sum_across_rows(float x) {
    x += dpp<0x128>(x);
    x += xor_rows(x, 16);
    x += xor_rows(x, 32);
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint4 load16(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// ---------------------------------------------------------------------------
// Append: one workgroup per entry copies its K row then its V row, 16 bytes a
// thread.
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
// Split decode pass.  Grid: one workgroup per (KV head h, chunk c, entry b),
// h fastest.  D: head dim (64 | 128); G: query heads per KV head; NW: waves
// per workgroup; TB: tiles per pipeline block; SMALL_PAGE: page_size < 8, so
// one 8-token tile may span several pages.
template <int D, int G, int NW, int TB, bool SMALL_PAGE>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(DecodeArgs a) {
    constexpr int NLD = D / 64;   // 16-byte words per lane per token row
    __shared__ float sm_m[NW][G];
    __shared__ float sm_l[NW][G];
    __shared__ float sm_acc[NW][G][D];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
    const int rg = lane >> 3;   // row group: token within a tile
    const int j = lane & 7;     // element slice [8j, 8j+8) (+64 for D = 128)

    int id = blockIdx.x;
    const int h = id % a.num_kv_heads;
    id /= a.num_kv_heads;
    const int c = id % a.max_chunks;
    const int b = id / a.max_chunks;

    const int p0 = a.indptr[b];
    const int npages = a.indptr[b + 1] - p0;
    if (npages < 1)
        return;
    const int nchunks = (npages + a.chunk_pages - 1) / a.chunk_pages;
    const int hq0 = h * G;
    if (nchunks > a.max_chunks) {
        // The entry is longer than the launch allows: poison its rows so the
        // broken precondition is visible instead of silently truncated.
        if (c == 0) {
            const float nan = __builtin_nanf("");
            for (int i = threadIdx.x; i < G * D; i += NW * 64)
                a.out[((int64_t)b * a.num_qo_heads + hq0) * D + i] = 0x7FC0;
            if (a.lse != nullptr && threadIdx.x < G)
                a.lse[(int64_t)b * a.num_qo_heads + hq0 + threadIdx.x] = nan;
        }
        return;
    }
    if (c >= nchunks)
        return;
    int last = a.last_len[b];
    last = last < 1 ? 1 : (last > a.page_size ? a.page_size : last);
    const int len = (npages - 1) * a.page_size + last;
    const int tok0 = c * a.chunk_pages * a.page_size;
    const int clen = min(a.chunk_pages * a.page_size, len - tok0);
    const int cpages = min(a.chunk_pages, npages - c * a.chunk_pages);
    const int ntiles = (clen + 7) >> 3;

    // Page ids of this chunk, one per lane (chunk_pages <= 64).
    int my_page = lane < cpages ? a.indices[p0 + c * a.chunk_pages + lane] : 0;
    my_page = (my_page >= 0 && my_page < a.num_pages) ? my_page : 0;

    // q rows of the G query heads that read KV head h, this lane's slice.
    uint32_t qv[G][NLD][4];
    {
        const uint16_t *qb = a.q + ((int64_t)b * a.num_qo_heads + hq0) * D + j * 8;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const uint4 w = load16(qb + g * D + i * 64);
                qv[g][i][0] = w.x;
                qv[g][i][1] = w.y;
                qv[g][i][2] = w.z;
                qv[g][i][3] = w.w;
            }
    }

    float m[G], l[G], acc[G][NLD][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[g][i][e] = 0.f;
    }

    // This wave's tiles are wave, wave + NW, ...; nt of them in nblk blocks.
    const int nt = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
    const int nblk = (nt + TB - 1) / TB;
    const uint16_t *head_base = a.cache + h * D + j * 8;

    struct Block {
        uint4 k[TB][NLD];
        uint4 v[TB][NLD];
    };

    // Issue the loads of block kb.  Tiles past the wave's last one reload the
    // last tile (an L1/L2 hit) and are masked in compute.
    auto load_block = [&](Block &blk, int kb) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int kt = min(kb * TB + tb, nt - 1);
            const int t = wave + kt * NW;
            const int tok = t * 8 + rg;
            int page;
            if (SMALL_PAGE)
                page = __shfl(my_page, tok >> a.log2_page, 64);
            else
                page = __builtin_amdgcn_readlane(my_page, (t * 8) >> a.log2_page);
            const int slot = tok & (a.page_size - 1);
            const uint16_t *row = head_base + (int64_t)page * a.page_stride +
                                  (int64_t)(slot * a.row_stride);
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                blk.k[tb][i] = load16(row + i * 64);
                blk.v[tb][i] = load16(row + a.half_stride + i * 64);
            }
        }
    };

    auto compute_block = [&](const Block &blk, int kb) {
        // Does this block hold a token at or past the chunk end?  (uniform)
        const bool edge = (wave + ((kb + 1) * TB - 1) * NW + 1) * 8 > clen;
        float s[TB][G];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    d = dot2_bf16(qv[g][i][0], blk.k[tb][i].x, d);
                    d = dot2_bf16(qv[g][i][1], blk.k[tb][i].y, d);
                    d = dot2_bf16(qv[g][i][2], blk.k[tb][i].z, d);
                    d = dot2_bf16(qv[g][i][3], blk.k[tb][i].w, d);
                }
                s[tb][g] = sum_row8(d) * a.scale_log2;
            }
        bool ok[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int tok = (wave + (kb * TB + tb) * NW) * 8 + rg;
            ok[tb] = tok < clen;
        }
        if (edge) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    s[tb][g] = ok[tb] ? s[tb][g] : -INFINITY;
        }
        // Lazy maximum: raise m only when a score passes it by more than kTau.
        float mb[G];
        bool raise_any = false;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            mb[g] = s[0][g];
#pragma unroll
            for (int tb = 1; tb < TB; ++tb)
                mb[g] = fmaxf(mb[g], s[tb][g]);
            raise_any |= mb[g] > m[g] + kTau;
        }
        if (raise_any) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const bool up = mb[g] > m[g] + kTau;
                const float mn = up ? mb[g] : m[g];
                const float alpha = up ? exp2_fast(m[g] - mn) : 1.f;
                m[g] = mn;
                l[g] *= alpha;
#pragma unroll
                for (int i = 0; i < NLD; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[g][i][e] *= alpha;
            }
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            float vf[NLD][8];
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const uint4 w = blk.v[tb][i];
                vf[i][0] = bf16_lo(w.x);
                vf[i][1] = bf16_hi(w.x);
                vf[i][2] = bf16_lo(w.y);
                vf[i][3] = bf16_hi(w.y);
                vf[i][4] = bf16_lo(w.z);
                vf[i][5] = bf16_hi(w.z);
                vf[i][6] = bf16_lo(w.w);
                vf[i][7] = bf16_hi(w.w);
            }
            if (edge && !ok[tb]) {
                // stale rows past the end may hold anything, NaN included
#pragma unroll
                for (int i = 0; i < NLD; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        vf[i][e] = 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float p = exp2_fast(s[tb][g] - m[g]);
                if (edge)
                    p = ok[tb] ? p : 0.f;   // also covers -inf - -inf
                l[g] += p;
#pragma unroll
                for (int i = 0; i < NLD; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[g][i][e] = fmaf(p, vf[i][e], acc[g][i][e]);
            }
        }
    };

    // Two-buffer pipeline written so that every compute is preceded, on every
    // path, by exactly the loads of the other buffer: the compiler's wait then
    // leaves that other buffer's loads in flight.
    if (nblk > 0) {
        Block A, B;
        load_block(A, 0);
        int kb = 0;
        for (;;) {
            if (kb + 1 >= nblk) {
                compute_block(A, kb);
                break;
            }
            load_block(B, kb + 1);
            compute_block(A, kb);
            ++kb;
            if (kb + 1 >= nblk) {
                compute_block(B, kb);
                break;
            }
            load_block(A, kb + 1);
            compute_block(B, kb);
            ++kb;
        }
    }

    // Merge the 8 row groups of this wave.
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mw = max_across_rows(m[g]);
        const float f = (m[g] == -INFINITY) ? 0.f : exp2_fast(m[g] - mw);
        l[g] = sum_across_rows(l[g] * f);
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[g][i][e] = sum_across_rows(acc[g][i][e] * f);
        m[g] = mw;
    }
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int i = 0; i < NLD; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sm_acc[wave][g][i * 64 + j * 8 + e] = acc[g][i][e];
            if (j == 0) {
                sm_m[wave][g] = m[g];
                sm_l[wave][g] = l[g];
            }
        }
    }
    __syncthreads();

    // Merge the waves and write: one thread per pair of output elements.
    for (int pi = threadIdx.x; pi < G * D / 2; pi += NW * 64) {
        const int g = pi / (D / 2);
        const int e2 = (pi % (D / 2)) * 2;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            mx = fmaxf(mx, sm_m[w][g]);
        float sum = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = sm_m[w][g];
            const float f = (mw == -INFINITY) ? 0.f : exp2_fast(mw - mx);
            sum += sm_l[w][g] * f;
            o0 += sm_acc[w][g][e2] * f;
            o1 += sm_acc[w][g][e2 + 1] * f;
        }
        const float inv = 1.f / sum;
        const int hq = hq0 + g;
        if (nchunks == 1) {
            const int64_t o = ((int64_t)b * a.num_qo_heads + hq) * D + e2;
            *reinterpret_cast<uint32_t *>(a.out + o) = pack_bf16x2(o0 * inv, o1 * inv);
            if (a.lse != nullptr && e2 == 0)
                a.lse[(int64_t)b * a.num_qo_heads + hq] = (mx + log2_fast(sum)) * kLn2;
        } else {
            const int64_t row = ((int64_t)b * a.max_chunks + c) * a.num_qo_heads + hq;
            *reinterpret_cast<float2 *>(a.part_o + row * D + e2) =
                make_float2(o0 * inv, o1 * inv);
            if (e2 == 0)
                a.part_lse[row] = mx + log2_fast(sum);
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of the partials of split entries: one workgroup per (entry, KV head),
// one thread per pair of output elements of the G query heads.
template <int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
    const int h = blockIdx.x % a.num_kv_heads;
    const int b = blockIdx.x / a.num_kv_heads;
    const int p0 = a.indptr[b];
    const int npages = a.indptr[b + 1] - p0;
    if (npages < 1)
        return;
    const int nchunks = (npages + a.chunk_pages - 1) / a.chunk_pages;
    if (nchunks <= 1 || nchunks > a.max_chunks)
        return;
    for (int pi = threadIdx.x; pi < G * D / 2; pi += blockDim.x) {
        const int g = pi / (D / 2);
        const int e2 = (pi % (D / 2)) * 2;
        const int hq = h * G + g;
        const int64_t row0 = (int64_t)b * a.max_chunks * a.num_qo_heads + hq;
        float mx = -INFINITY;
        for (int c = 0; c < nchunks; ++c)
            mx = fmaxf(mx, a.part_lse[row0 + (int64_t)c * a.num_qo_heads]);
        float sum = 0.f, o0 = 0.f, o1 = 0.f;
        for (int c = 0; c < nchunks; ++c) {
            const int64_t row = row0 + (int64_t)c * a.num_qo_heads;
            const float w = exp2_fast(a.part_lse[row] - mx);
            const float2 v = *reinterpret_cast<const float2 *>(a.part_o + row * D + e2);
            sum += w;
            o0 = fmaf(w, v.x, o0);
            o1 = fmaf(w, v.y, o1);
        }
        const float inv = 1.f / sum;
        const int64_t o = ((int64_t)b * a.num_qo_heads + hq) * D + e2;
        *reinterpret_cast<uint32_t *>(a.out + o) = pack_bf16x2(o0 * inv, o1 * inv);
        if (a.lse != nullptr && e2 == 0)
            a.lse[(int64_t)b * a.num_qo_heads + hq] = (mx + log2_fast(sum)) * kLn2;
    }
}

constexpr int kWaves = 4;       // waves per decode workgroup
constexpr int kTilesPerBlock = 2;

// Launch through hipLaunchKernel so the returned status belongs to this
// launch alone (hipGetLastError could report an older, unrelated error).
template <typename Args>
hipError_t launch(const void *kernel, dim3 grid, dim3 block, const Args &args,
                  hipStream_t stream) {
    void *params[] = {const_cast<Args *>(&args)};
    return hipLaunchKernel(kernel, grid, block, params, 0, stream);
}

template <int D, int G>
hipError_t launch_decode_dg(const DecodeArgs &a, int batch, hipStream_t stream) {
    const dim3 grid((unsigned)a.num_kv_heads * (unsigned)a.max_chunks * (unsigned)batch);
    const void *k = a.page_size < 8
        ? reinterpret_cast<const void *>(
              &decode_split_kernel<D, G, kWaves, kTilesPerBlock, true>)
        : reinterpret_cast<const void *>(
              &decode_split_kernel<D, G, kWaves, kTilesPerBlock, false>);
    hipError_t err = launch(k, grid, dim3(kWaves * 64), a, stream);
    if (err != hipSuccess || a.max_chunks <= 1)
        return err;
    constexpr int pairs = G * D / 2;
    constexpr int threads = pairs >= 256 ? 256 : ((pairs + 63) / 64) * 64;
    return launch(reinterpret_cast<const void *>(&merge_kernel<D, G>),
                  dim3((unsigned)batch * a.num_kv_heads), dim3(threads), a, stream);
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &a, int group, int batch, hipStream_t s) {
    switch (group) {
    case 1: return launch_decode_dg<D, 1>(a, batch, s);
    case 2: return launch_decode_dg<D, 2>(a, batch, s);
    case 3: return launch_decode_dg<D, 3>(a, batch, s);
    case 4: return launch_decode_dg<D, 4>(a, batch, s);
    case 5: return launch_decode_dg<D, 5>(a, batch, s);
    case 6: return launch_decode_dg<D, 6>(a, batch, s);
    case 7: return launch_decode_dg<D, 7>(a, batch, s);
    case 8: return launch_decode_dg<D, 8>(a, batch, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream) {
    return launch(reinterpret_cast<const void *>(&append_kernel), dim3((unsigned)batch),
                  dim3(256), a, stream);
}

hipError_t launch_decode(const DecodeArgs &a, int head_dim, int group, int batch,
                         hipStream_t stream) {
    if (head_dim == 64)
        return launch_decode_d<64>(a, group, batch, stream);
    if (head_dim == 128)
        return launch_decode_d<128>(a, group, batch, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
