// pkv_launch.h -- internal interface between the C ABI (pkv_api.cpp) and the
// gfx950 kernels (pkv_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace pkv {

// Arguments of the standalone append kernel (offsets in bf16 elements).
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

// Arguments of the decode and merge kernels.
struct DecodeArgs {
    const uint16_t *cache;    // first element of this layer's slab
    uint16_t *cache_w;        // same slab, written by the fused append, or null
    const uint16_t *q;        // [batch, Hq, D]
    const uint16_t *k_new;    // fused append rows [batch, Hkv, D], or null
    const uint16_t *v_new;
    const int32_t *indptr;
    const int32_t *indices;
    const int32_t *last_len;
    uint16_t *out;            // [batch, Hq, D] bf16
    float *lse;               // [batch, Hq] or null
    float *part_o;            // [slots, Hq, D] fp32 partial outputs
    float *part_lse;          // [slots, Hq] fp32 partial lse, log2 domain
    int32_t *tile_start;      // [batch + 1] tile prefix sums (balanced mode)
    int64_t page_stride;
    int32_t half_stride;
    int32_t row_stride;       // Hkv * D
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t batch;
    int32_t page_size;
    int32_t log2_page;
    int32_t chunk_tiles;      // fixed mode: 8-token tiles per chunk; 0 = balanced
    int32_t max_chunks;       // fixed mode: chunks per entry the launch covers
    int32_t num_groups;       // balanced mode: workgroups sharing the tiles
    int32_t q_slots;          // q rows a workgroup stages in LDS per piece (set at launch)
    float scale_log2;         // sm_scale * log2(e)
};

// Largest batch the balanced schedule keeps in LDS (its tile prefix sums);
// larger batches use fixed chunks of kFallbackChunkPages pages.
constexpr int kMaxBalancedBatch = 4096;
constexpr int kFallbackChunkPages = 16;
constexpr int kMaxChunkPages = 1 << 16;
// Upper bound on compute units, for sizing workspace without a device query.
constexpr int kMaxComputeUnits = 320;
constexpr int kMaxWavesPerCU = 32;
constexpr int kMaxKvHeads = 16;
// A decode workgroup has one wave per KV head, at most 8; more heads use more
// workgroups along the grid's y axis.  The kernel keeps to 256 registers a
// wave (two waves per SIMD), the most VALU instructions can address.
constexpr int kMaxWavesPerGroup = 8;

// Tiles are 8 tokens: one token row per 8-lane group of a 64-wide wavefront.
constexpr int kTileTokens = 8;

inline int64_t balanced_groups_bound(int num_kv_heads) {
    const int waves = num_kv_heads < kMaxWavesPerGroup ? num_kv_heads : kMaxWavesPerGroup;
    return ((int64_t)kMaxComputeUnits * kMaxWavesPerCU + waves - 1) / waves;
}

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream);

// Number of workgroups the balanced schedule uses on the current device.
hipError_t balanced_groups(int head_dim, int group, int num_kv_heads, int page_size,
                           int batch, int *groups);

// Enqueues the decode pass, then the merge of entries split over several
// workgroups.  hipErrorInvalidValue for a (head_dim, group) that is not built.
hipError_t launch_decode(const DecodeArgs &a, int head_dim, int group, hipStream_t stream);

}  // namespace pkv
