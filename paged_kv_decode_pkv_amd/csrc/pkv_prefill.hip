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
// products run on the matrix cores (v_mfma_f32_16x16x16_bf16).  One wave
// takes two groups of 16 columns: (row, query head) pairs of one entry and
// KV head, the G heads of a row side by side; the groups share each tile's
// K/V loads, its V staging and its V^T reads.  Per 16-token tile of the
// entry's pages and per group:
//   S^T[t][c] = sum_d K[t][d] Q[c][d]      8 MFMAs (K = 16 values of d each)
//   O^T[d][c] += sum_t V[t][d] P[c][t]     8 MFMAs per half of P (see below)
// With lane l = 16 q + c (c = column, q = lane group), the MFMA gives lane l
// the scores of column c for tokens 4q .. 4q + 3 of the tile, exactly the
// B-operand slots of P^T in the second product, and it holds column c of
// O^T: the online softmax of a column (its running maximum and sum, the
// rescale of its outputs) stays within the lane and the three other lanes of
// its column.  Within a 16-value group of d the order of the sum is free, so
// lane group q takes d = 32 q + 4 m + r (m = MFMA index, r = element): each
// lane reads 64 contiguous bytes of a K row (and of its q row), and 64 lanes
// read a whole 16-token K tile.  The V tile goes through LDS (rows padded to
// 272 bytes, so the four lane groups' transposed reads hit distinct banks):
// the A operand of the second product wants four tokens at one d.
// P is split into a bf16 high part and a bf16 remainder, two MFMAs each, so
// the weights keep about 16 significant bits (a single bf16 P costs a few
// thousandths of the output, too much for the parity bar).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_launch.h"

namespace pkv {
namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kMaskedScore = -1e30f;   // log2-domain score of a masked token
constexpr int kRowPad = 272;             // LDS bytes per staged V row (256 + 16)
constexpr int kColumnGroups = 2;         // groups of 16 columns per wave

__device__ __forceinline__ short bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (short)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_val(short s) {
    return __uint_as_float((uint32_t)(uint16_t)s << 16);
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

// This lane's 64 bytes of the K row and of the V row of token tl; past the
// entry's last token the last token's rows are read again (their weight is
// zero, and a real token's values are finite).  kbase points at the lane's
// bytes of the KV head's row in a page.
__device__ __forceinline__ void load_tile(const PrefillArgs &a, const int32_t *pages,
                                          const uint16_t *kbase, int len, int tl, uint4 *kr,
                                          uint4 *vr) {
    const int t = min(tl, len - 1);
    int page = pages[t / a.page_size];
    page = (page >= 0 && page < a.num_pages) ? page : 0;   // bad table: no fault
    const uint16_t *row = kbase + (int64_t)page * a.page_stride +
                          (int64_t)(t % a.page_size) * a.row_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kr[i] = reinterpret_cast<const uint4 *>(row)[i];
        vr[i] = reinterpret_cast<const uint4 *>(row + a.half_stride)[i];
    }
}

// One 16-token tile of a wave's NG groups of 16 columns: S^T of each group,
// the causal mask, the online softmax update of each column and O^T += V^T
// P^T.  The groups share the tile's K/V loads, the V staging and the V^T
// reads.  kr / vr hold this lane's 64 bytes of the K and V rows of token
// t0 + c.
template <int NG>
__device__ __forceinline__ void attend_tile(const uint4 *kr, const uint4 *vr, int t0, int c,
                                            int q, const int *pos, int len, float c2,
                                            const bf16x4_t (*qb)[8], char *vt,
                                            f32x4_t (*o)[8], float *m, float *lsum) {
    // stage V: row c of the tile, bytes 64 q .. 64 q + 63
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4 *>(vt + c * kRowPad + 64 * q + 16 * i) = vr[i];

    bf16x4_t phi[NG], plo[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        // S^T tile of the group
        f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = kr[i];
            const bf16x4_t k0 = {(short)(v.x & 0xFFFF), (short)(v.x >> 16),
                                 (short)(v.y & 0xFFFF), (short)(v.y >> 16)};
            const bf16x4_t k1 = {(short)(v.z & 0xFFFF), (short)(v.z >> 16),
                                 (short)(v.w & 0xFFFF), (short)(v.w >> 16)};
            s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(k0, qb[gi][2 * i], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(k1, qb[gi][2 * i + 1], s, 0, 0, 0);
        }
        // scores of column c, tokens t0 + 4 q + r; causal and length mask
        float sc[4];
        float tmax = kMaskedScore;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * q + r;
            sc[r] = (t <= pos[gi] && t < len) ? s[r] * c2 : kMaskedScore;
            tmax = fmaxf(tmax, sc[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m[gi], tmax);
        const float alpha = exp2f(m[gi] - mn);
        m[gi] = mn;
        lsum[gi] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[gi][i] *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = exp2f(sc[r] - mn);
            lsum[gi] += p;
            phi[gi][r] = bf16_rne(p);
            plo[gi][r] = bf16_rne(p - bf16_val(phi[gi][r]));
        }
    }
    // O^T += V^T P^T: A operand = V[t0 + 4 q + r][16 blk + c]
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
        bf16x4_t va;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            va[r] = *reinterpret_cast<const short *>(vt + (4 * q + r) * kRowPad +
                                                     2 * (16 * blk + c));
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            o[gi][blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi[gi], o[gi][blk], 0,
                                                                   0, 0);
            o[gi][blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo[gi], o[gi][blk], 0,
                                                                   0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Causal attention of the new rows: one wave per (16-column block, KV head,
// entry).  D = 128.
template <int NG>
__global__ __launch_bounds__(64) void prefill_kernel(PrefillArgs a) {
    constexpr int D = 128;
    constexpr int W = 16 * NG;   // columns per wave
    __shared__ __attribute__((aligned(16))) char vt[16 * kRowPad];
    const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int l = threadIdx.x;
    const int c = l & 15, q = l >> 4;
    const int G = a.num_qo_heads / a.num_kv_heads;

    const int r0 = a.qo_indptr[b];
    const int n = a.qo_indptr[b + 1] - r0;
    const int ncols = n * G;
    if (cb * W >= ncols)
        return;   // whole wave
    const int p0 = a.indptr[b];
    const int np = a.indptr[b + 1] - p0;
    const int last = a.last_len[b];
    if (np < 1 || last < 1 || last > a.page_size)
        return;
    const int len = (np - 1) * a.page_size + last;
    if (n > len)
        return;
    const int32_t *pages = a.indices + p0;
    const int last_col = min(ncols, cb * W + W) - 1;
    const int pmax = len - n + last_col / G;   // largest position of the block

    // this lane's columns (one per group): row j, head g of the KV head's group
    int jj[NG], gg[NG], pos[NG];
    bool valid[NG];
    bf16x4_t qb[NG][8];
    f32x4_t o[NG][8];
    float m[NG], lsum[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int col = cb * W + 16 * gi + c;
        valid[gi] = col < ncols;
        jj[gi] = valid[gi] ? col / G : 0;
        gg[gi] = valid[gi] ? col % G : 0;
        pos[gi] = valid[gi] ? len - n + jj[gi] : -1;
        // q: this lane's 32 values of d (lane group q takes d = 32 q .. 32 q + 31)
        const uint4 *src = reinterpret_cast<const uint4 *>(
            a.q + ((int64_t)(r0 + jj[gi]) * a.num_qo_heads + h * G + gg[gi]) * D + 32 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = valid[gi] ? src[i] : make_uint4(0u, 0u, 0u, 0u);
            qb[gi][2 * i] = bf16x4_t{(short)(v.x & 0xFFFF), (short)(v.x >> 16),
                                     (short)(v.y & 0xFFFF), (short)(v.y >> 16)};
            qb[gi][2 * i + 1] = bf16x4_t{(short)(v.z & 0xFFFF), (short)(v.z >> 16),
                                         (short)(v.w & 0xFFFF), (short)(v.w >> 16)};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[gi][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m[gi] = kMaskedScore;   // running maximum of the column (log2 domain)
        lsum[gi] = 0.f;         // this lane's share of the column's weight sum
    }
    const float c2 = a.scale_log2;
    const uint16_t *kbase = a.cache + (int64_t)h * D + 32 * q;

    // K rows and V rows of token t0 + c of a tile (this lane's 64 bytes of
    // each), in two register sets: the next tile's loads are issued before
    // the current tile is computed (unconditional loads of a clamped token
    // past the end, so the compiler can wait for exactly the older set)
    uint4 ka[4], va[4], kb[4], vb[4];
    load_tile(a, pages, kbase, len, c, ka, va);
    for (int t0 = 0; t0 <= pmax; t0 += 32) {
        load_tile(a, pages, kbase, len, t0 + 16 + c, kb, vb);
        attend_tile<NG>(ka, va, t0, c, q, pos, len, c2, qb, vt, o, m, lsum);
        if (t0 + 16 > pmax)
            break;
        load_tile(a, pages, kbase, len, t0 + 32 + c, ka, va);
        attend_tile<NG>(kb, vb, t0 + 16, c, q, pos, len, c2, qb, vt, o, m, lsum);
    }

#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        // the column's weight sum over its four lanes, then the outputs
        float ls = lsum[gi];
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        if (!valid[gi])
            continue;
        const float inv = 1.f / ls;
        uint16_t *orow =
            a.out + ((int64_t)(r0 + jj[gi]) * a.num_qo_heads + h * G + gg[gi]) * D;
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            // lane holds O^T[16 blk + 4 q + r][c]
            const uint32_t w0 = (uint32_t)(uint16_t)bf16_rne(o[gi][blk][0] * inv) |
                                ((uint32_t)(uint16_t)bf16_rne(o[gi][blk][1] * inv) << 16);
            const uint32_t w1 = (uint32_t)(uint16_t)bf16_rne(o[gi][blk][2] * inv) |
                                ((uint32_t)(uint16_t)bf16_rne(o[gi][blk][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(orow + 16 * blk + 4 * q) = make_uint2(w0, w1);
        }
        if (a.lse != nullptr && q == 0)
            a.lse[(int64_t)(r0 + jj[gi]) * a.num_qo_heads + h * G + gg[gi]] =
                (m[gi] + __log2f(ls)) * 0.6931471805599453f;
    }
}

}  // namespace

bool prefill_supported(int head_dim) { return head_dim == 128; }

hipError_t launch_prefill(const PrefillArgs &a, bool append, hipStream_t stream) {
    PrefillArgs args = a;
    void *params[] = {&args};
    if (a.head_dim != 128 || a.batch > 65535 || a.num_kv_heads > 65535)
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
    const int64_t blocks = ((int64_t)a.max_rows * G + 16 * kColumnGroups - 1) /
                           (16 * kColumnGroups);
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidValue;
    return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_kernel<kColumnGroups>),
                           dim3((unsigned)blocks, (unsigned)a.num_kv_heads, (unsigned)a.batch),
                           dim3(64), params, 0, stream);
}

}  // namespace pkv
