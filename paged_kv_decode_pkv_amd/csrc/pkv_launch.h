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

// Tiles are up to 8 consecutive tokens of one page: page_size / 8 tiles per
// page (one tile when page_size < 8), the last page of an entry cut at its
// last row.
constexpr int kTileTokens = 8;

// The plan of a decode step (pkv_plan) lives in the workspace:
//   cnt     int32 [batch * Hkv]   arrival counters of split entries; zero
//                                 between launches (the plan zeroes them, the
//                                 merging wave resets its own)
//   ent     int4  [batch]         per entry: first partial slot, number of
//                                 segments (0: no tiles, -1: over the page
//                                 bound), and the append target page / slot
//   blocks  int4  [num_blocks][block_stride]
//                                 per decode workgroup: a header {tiles, run,
//                                 plan signature, 0} and then one record per
//                                 tile {page, info, entry, partial slot}
// The plan signature is a nonzero 32-bit hash of the arguments the plan was
// made for (batch, heads, page size, head_dim, page bound, chunk, pool pages,
// workgroups, record stride, tiles per page); a decode launch compares it
// with the hash of its own arguments before it uses any record.
//   part_o  fp16  [slots, Hq, D]  partial outputs of split entries, each
//                                 (slot, KV head) scaled by a power of two
//                                 2^-s that keeps them below 1 in magnitude
//   part_lse fp32 [slots, Hq, 2]  their log-sum-exp (base 2) and s
// Bits of a record's info word:
constexpr int kInfoNtokMask = 0x7;        // tokens in the tile - 1
constexpr int kInfoSlotShift = 3;         // bits 3-11: page slot of the first token
constexpr int kInfoSlotMask = 0x1FF;
constexpr int kInfoSegFirst = 1 << 12;    // first tile of its segment
constexpr int kInfoSegLast = 1 << 13;     // last tile of its segment
constexpr int kInfoSegWhole = 1 << 14;    // the segment is the whole entry
constexpr int kInfoHasNew = 1 << 15;      // the tile holds the entry's token L-1
constexpr int kInfoNewRowShift = 16;      // bits 16-18: that token's row in the tile

struct PlanArgs {
    int32_t plan_sig;         // signature written into every block header
    const int32_t *indptr;
    const int32_t *indices;
    const int32_t *last_len;
    int32_t *blocks;          // int4 records, see above
    int32_t *ent;             // int4 per entry
    int32_t *cnt;
    int32_t batch;
    int32_t num_pages;
    int32_t page_size;
    int32_t tiles_per_page;
    int32_t num_kv_heads;
    int32_t num_blocks;       // decode workgroups along x
    int32_t block_stride;     // int4 records per block: 1 + capacity
    int32_t chunk_tiles;      // fixed mode: tiles per chunk; 0 = balanced
    int32_t max_chunks;       // fixed mode: chunks per entry
    int32_t max_pages;        // entries listing more pages are poisoned
    // Mixed step (qo_indptr non-null): `batch` counts rows, and row r is
    // planned as the entry b whose single new row it is (qo_indptr[b] = r,
    // qo_indptr[b + 1] = r + 1); the rows of entries with several new rows
    // get no tiles.  num_entries entries; the page table is indexed by b.
    const int32_t *qo_indptr;
    int32_t num_entries;
    // and the entries with several new rows, for the prefill half:
    // {plan_sig, count, entry ids in order}, at most list_cap ids
    int32_t *list;
    int32_t list_cap;
};

struct RunArgs {
    int32_t plan_sig;         // the signature this launch's arguments give
    int32_t num_pages;        // pool pages: page ids past it are read as page 0
    int32_t page_size;
    const uint16_t *cache;    // first element of this layer's slab
    uint16_t *cache_w;        // same slab, written by the fused append, or null
    const uint16_t *q;        // [batch, Hq, D]
    const uint16_t *k_new;    // fused append rows [batch, Hkv, D], or null
    const uint16_t *v_new;
    uint16_t *out;            // [batch, Hq, D] bf16
    float *lse;               // [batch, Hq] or null
    uint16_t *part_o;         // fp16 [slots, Hq, D], scaled by 2^-s
    float *part_lse;          // [slots, Hq] pairs {base-2 lse, s}
    int64_t part_o_bytes;     // sizes of the two partial arrays
    int64_t part_lse_bytes;
    int32_t *cnt;
    int64_t page_stride;      // 2 * page_size * Hkv * D
    int32_t half_stride;      // page_size * Hkv * D
    int32_t row_stride;       // Hkv * D
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t batch;
    int32_t block_stride;
    float scale_log2;         // sm_scale * log2(e)
    // Fused q/k RMSNorm + rotary embedding of the segment's q rows and of the
    // appended k row (q_w null: off); see NormRopeArgs for the formulas.
    const uint16_t *q_w;      // [D]
    const uint16_t *k_w;      // [D]
    const int32_t *positions; // [batch], or [batch, 3] (t, h, w) for multimodal RoPE
    float eps;
    double log2_theta;        // log2 of the rotary base
    int32_t pos_stride;       // 1, or 3 for multimodal RoPE
    // multimodal RoPE: the position component (0, 1, 2) pair i follows, two
    // bits per pair, pair i at bit 2 (i % 16) of word i / 16
    uint32_t axis_bits[4];
};

// Largest batch the balanced plan handles (its tile prefix sums sit in LDS);
// larger batches use fixed chunks of kFallbackChunkPages pages.
constexpr int kMaxBalancedBatch = 4096;
constexpr int kFallbackChunkPages = 16;
// Largest batch of any plan (fixed chunks keep three int arrays per entry in
// the plan kernel's LDS), and the largest for which fixed mode ranks the
// entries' last chunks by size (an all-pairs count in LDS; above it they are
// dealt in entry order).
constexpr int kMaxPlanBatch = 8192;
constexpr int kRankedBatch = 256;

// Dynamic LDS bytes of the plan kernel.
inline size_t plan_lds_bytes(int batch, bool fixed, bool mixed = false) {
    const size_t b = (size_t)batch;
    const size_t base = !fixed ? 2 * sizeof(int) * (b + 1)
                               : sizeof(int) * ((b + 1) + 2 * b + (batch <= kRankedBatch ? b : 0));
    return base + (mixed ? sizeof(int) * b : 0);   // mixed: the row -> entry map
}
constexpr int kMaxChunkPages = 1 << 16;
// Upper bounds for sizing workspace without a device query.
constexpr int kMaxComputeUnits = 320;
constexpr int kMaxWavesPerCU = 32;
constexpr int kMaxKvHeads = 16;
// A decode workgroup has one wave per KV head of its head group; groups are
// the largest divisor of the head count up to 8 heads, so every group is full
// (the workgroup's waves all take the same barriers), and more heads use more
// workgroups along the grid's y axis.
constexpr int kMaxWavesPerGroup = 8;
// The decode kernel stages tiles through a ring of at most this many LDS
// buffers and reads that many records of its block at once, before it knows
// how many the block has: the block region is padded by as many records.
// Two tiles in flight per wave measured best: three or four (more buffers)
// streamed 1-3 % slower on the Qwen3-4B-like and Qwen3-0.6B-like layers.
constexpr int kMaxStageBuffers = 2;

inline int group_waves(int num_kv_heads) {
    for (int w = num_kv_heads < kMaxWavesPerGroup ? num_kv_heads : kMaxWavesPerGroup; w > 1;
         --w)
        if (num_kv_heads % w == 0)
            return w;
    return 1;
}

// Cost units of the balanced split: a tile, and the extra work of an entry
// (starting and ending a segment: its q rows, a partly filled last tile, the
// first tile's rescale, the merge of row groups and the stores; measured at
// about two and a half tiles of decode time).
constexpr int kTileCost = 4;
constexpr int kEntryCost = 10;

// Shortest run of the balanced split, in tiles: a small workload takes fewer
// runs than there are workgroups rather than runs of a tile or two, whose
// start, partial and share of the merge cost more than their tiles.
constexpr int kMinRunTiles = 4;

// Records one balanced block may receive.  The cost axis (kTileCost T +
// kEntryCost Z for T tiles in Z entries) is cut into R runs, R = W when the
// axis holds W runs of kMinRunTiles tiles, else fewer (at least 1): a run
// then holds at most (kTileCost T + kEntryCost Z) / (kTileCost W) + 1 tiles
// (the first term's two rounded-up parts and the last term bound it), or
// less than 2 kMinRunTiles + 1.
inline int64_t balanced_capacity(int64_t max_tiles, int64_t batch, int64_t blocks) {
    const int64_t full = (max_tiles + blocks - 1) / blocks +
                         (kEntryCost * batch + kTileCost * blocks - 1) / (kTileCost * blocks) + 2;
    return full > 2 * kMinRunTiles + 2 ? full : 2 * kMinRunTiles + 2;
}

// Records one fixed-mode block may receive: the snake deals each of W
// workgroups at most ceil(T / W) of the T chunks, each of at most
// min(chunk_tiles, entry_tiles) tiles.
inline int64_t fixed_capacity(int64_t chunks, int64_t chunk_tiles, int64_t entry_tiles,
                              int64_t blocks) {
    const int64_t c = chunk_tiles < entry_tiles ? chunk_tiles : entry_tiles;
    return (chunks + blocks - 1) / blocks * (c > 0 ? c : 1);
}

inline int64_t balanced_blocks_bound(int num_kv_heads) {
    const int waves = group_waves(num_kv_heads);
    return ((int64_t)kMaxComputeUnits * kMaxWavesPerCU + waves - 1) / waves;
}

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream);

// Arguments of the fused q/k RMSNorm + rotary embedding + KV write kernel
// (offsets in bf16 elements).
struct NormRopeArgs {
    uint16_t *cache;          // first element of this layer's slab
    const uint16_t *q;        // [batch, Hq, D]
    const uint16_t *k_new;    // [batch, Hkv, D]
    const uint16_t *v_new;
    const uint16_t *q_w;      // [D] RMSNorm weights of the q heads
    const uint16_t *k_w;      // [D] of the k heads
    uint16_t *q_out;          // [batch, Hq, D], may be q
    const int32_t *positions; // [batch], or [batch, 3] (t, h, w) for multimodal RoPE
    const int32_t *indptr;
    const int32_t *indices;
    const int32_t *last_len;
    int64_t page_stride;      // 2 * page_size * Hkv * D
    int32_t half_stride;      // page_size * Hkv * D
    int32_t row_elems;        // Hkv * D
    int32_t num_pages;
    int32_t page_size;
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t batch;
    float eps;
    int32_t pos_stride;       // 1, or 3 for multimodal RoPE
    // multimodal RoPE: the position component (0, 1, 2) pair i follows, two
    // bits per pair, pair i at bits 2 (i % 16) of word i / 16
    uint32_t axis_bits[4];
    // rotation rate of pair i in turns per position: theta^(-2i/D) / (2 pi)
    double turns[64];
};

// Arguments of the paged prefill (several new rows per entry) kernels; offsets
// in bf16 elements.
struct PrefillArgs {
    const uint16_t *cache;    // first element of this layer's slab
    uint16_t *cache_w;        // same slab, written by the append, or null
    const uint16_t *q;        // [rows, Hq, D]
    const uint16_t *k_new;    // [rows, Hkv, D] or null
    const uint16_t *v_new;
    uint16_t *out;            // [rows, Hq, D]
    float *lse;               // [rows, Hq] or null
    const int32_t *qo_indptr; // [batch + 1] rows per entry
    const int32_t *indptr;
    const int32_t *indices;
    const int32_t *last_len;
    int64_t page_stride;      // 2 * page_size * Hkv * D
    int32_t half_stride;      // page_size * Hkv * D
    int32_t row_stride;       // Hkv * D
    int32_t num_pages;
    int32_t page_size;
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t batch;
    int32_t max_rows;         // host bound on any entry's new rows
    int32_t pair_tiles;       // workgroups per (entry, KV head): ceil(T / 2) for the
                              // T = ceil(max_rows * G / 128) column tiles
    int32_t skip_single;      // 1: entries with one new row are left to the decode
    int32_t page_shift;       // log2(page_size)
    float scale_log2;         // sm_scale * log2(e)
    // Mixed step (non-null): the entries to compute, as a mixed plan wrote
    // them: {signature, count, entry ids...}, at most list_cap ids; a list
    // whose signature is not list_sig is ignored.
    const int32_t *list;
    int32_t list_sig;
    int32_t list_cap;
};

// Compute units of the current device (queried once per device).
hipError_t compute_units(int *cus);

// True when the prefill kernels are built for head_dim.
bool prefill_supported(int head_dim);

// Enqueues the attention of the new rows, with their append when
// a.cache_w is set.
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// True when the fused norm/rope/write kernel is built for head_dim.
bool norm_rope_supported(int head_dim);

hipError_t launch_norm_rope(const NormRopeArgs &a, hipStream_t stream);

// Workgroups per head group the balanced plan uses on the current device
// (what the device holds at once).
hipError_t balanced_blocks(int head_dim, int group, int num_kv_heads, int *blocks);

// True when the decode kernel is built for (head_dim, group).
bool run_supported(int head_dim, int group);

// True when the decode kernel with the fused q/k norm + rotary embedding is
// built for (head_dim, group).
bool run_norm_rope_supported(int head_dim, int group);

hipError_t launch_plan(const PlanArgs &a, hipStream_t stream);

// Bytes of the file-scope device array behind pkv_decode_static.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;

// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress and kept).  No allocation.
hipError_t static_scratch(void **ptr);

// Enqueues the decode kernel: num_blocks x head-group workgroups.
hipError_t launch_run(const RunArgs &a, const int32_t *blocks, const int32_t *ent,
                      int num_blocks, int head_dim, int group, hipStream_t stream);

}  // namespace pkv
