// pkv_launch.h -- internal interface between the C ABI (pkv_api.cpp) and the
// gfx950 kernels (pkv_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace pkv {

// Arguments of the append kernel (all offsets in bf16 elements).
struct AppendArgs {
    uint16_t *cache;          // first element of this layer's slab
    const uint16_t *k_new;    // [batch, Hkv, D]
    const uint16_t *v_new;
    const int32_t *indptr;
    const int32_t *indices;
    const int32_t *last_len;
    int64_t page_stride;      // 2 * page_size * Hkv * D
    int32_t half_stride;      // page_size * Hkv * D (K half -> V half)
    int32_t row_elems;        // Hkv * D: one slot of one page half
    int32_t num_pages;
    int32_t page_size;
};

// Arguments of the split-decode and merge kernels.
struct DecodeArgs {
    const uint16_t *cache;    // first element of this layer's slab
    const uint16_t *q;        // [batch, Hq, D]
    const int32_t *indptr;
    const int32_t *indices;
    const int32_t *last_len;
    uint16_t *out;            // [batch, Hq, D] bf16
    float *lse;               // [batch, Hq] or nullptr
    float *part_o;            // [batch, max_chunks, Hq, D] fp32 (split only)
    float *part_lse;          // [batch, max_chunks, Hq] fp32, log2 domain
    int64_t page_stride;
    int32_t half_stride;
    int32_t row_stride;       // Hkv * D
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t max_chunks;
    int32_t chunk_pages;
    int32_t page_size;
    int32_t log2_page;
    float scale_log2;         // sm_scale * log2(e)
};

// Largest chunk length the decode kernel accepts: a chunk's page ids are held
// one per lane of a 64-wide wavefront.
constexpr int kMaxChunkPages = 64;
constexpr int kDefaultChunkPages = 16;

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream);
// Enqueues the split pass, then (when max_chunks > 1) the merge.  Returns
// hipErrorInvalidValue for a (head_dim, group) pair that is not built.
hipError_t launch_decode(const DecodeArgs &a, int head_dim, int group, int batch,
                         hipStream_t stream);

}  // namespace pkv
