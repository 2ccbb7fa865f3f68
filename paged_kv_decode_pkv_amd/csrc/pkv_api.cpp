// pkv_api.cpp -- the C ABI declared in include/pkv.h: host-side argument
// checks, then one enqueue per kernel.  No allocation, no synchronisation, no
// host read of device memory, so every call is HIP-graph capturable.

#include "pkv.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "pkv_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t err) {
    if (err == hipSuccess)
        return PKV_OK;
    g_last_hip_error = (int)err;
    return PKV_ERR_HIP;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Largest head count any call accepts (query or key/value heads): head
// indices and their sums stay far inside 32 bits.
constexpr int32_t kMaxHeads = 65535;

int check_desc(const pkv_cache_desc_t &d) {
    if (d.num_layers < 1 || d.num_pages < 1 || d.num_kv_heads < 1 || d.head_dim < 1)
        return PKV_ERR_BAD_SHAPE;
    if (!is_pow2(d.page_size) || d.page_size > 256)
        return d.page_size < 1 ? PKV_ERR_BAD_SHAPE : PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

int64_t page_elems(const pkv_cache_desc_t &d) {
    return 2 * (int64_t)d.page_size * d.num_kv_heads * d.head_dim;
}

// Workspace layout of a plan and how its work is split.  Every offset
// depends on host arguments only (the balanced split's workgroup count W is a
// device property, so regions are sized for its bound).
struct Layout {
    int32_t chunk_tiles = 0;    // 0: balanced
    int32_t max_chunks = 1;
    int32_t tiles_per_page = 1;
    int64_t max_tiles = 0;      // tiles of batch entries of max_pages_per_req pages
    int64_t slots = 0;          // partial rows per query head
    int64_t off_ent = 0, off_blocks = 0, off_part_o = 0, off_part_lse = 0;
    int64_t off_list = 0;       // a mixed plan's prefill list
    int32_t list_cap = 0;       // entry ids it holds
    int64_t ws_bytes = 0;
};

Layout make_layout(const pkv_cache_desc_t &d, int32_t num_qo_heads, int32_t batch,
                   int32_t max_pages_per_req, int32_t kv_chunk_pages) {
    Layout p;
    const int64_t tt = pkv::kTileTokens;
    p.tiles_per_page = (int32_t)((d.page_size + tt - 1) / tt);
    const int64_t entry_tiles = (int64_t)max_pages_per_req * p.tiles_per_page;
    p.max_tiles = (int64_t)batch * entry_tiles;
    int32_t chunk_pages = kv_chunk_pages;
    if (chunk_pages == 0 && batch > pkv::kMaxBalancedBatch)
        chunk_pages = pkv::kFallbackChunkPages;
    int64_t block_ints4;   // int4 records of all blocks (headers included)
    if (chunk_pages > 0) {
        p.chunk_tiles = (int32_t)((int64_t)chunk_pages * p.tiles_per_page);
        p.max_chunks = (int32_t)((entry_tiles + p.chunk_tiles - 1) / p.chunk_tiles);
        if (p.max_chunks < 1)
            p.max_chunks = 1;
        p.slots = (int64_t)batch * p.max_chunks;
        // the chunks are dealt to W <= wb workgroups, each holding at most
        // fixed_capacity records: W (1 + capacity) <= wb (1 + c) + T c for
        // T = batch * max_chunks chunks of at most c tiles
        const int64_t wb = pkv::balanced_blocks_bound(d.num_kv_heads);
        const int64_t c = p.chunk_tiles < entry_tiles ? p.chunk_tiles : entry_tiles;
        block_ints4 = wb * (1 + c) + p.slots * c;
    } else {
        const int64_t wb = pkv::balanced_blocks_bound(d.num_kv_heads);
        p.slots = wb + batch;
        // W blocks of 1 + balanced_capacity records each, for any W <= wb:
        // at most W (1 + max_tiles / W + 1 + E batch / W + 1 + 2) with E =
        // kEntryCost / kTileCost, or W (1 + 2 kMinRunTiles + 2), in total
        const int64_t full = p.max_tiles +
                             (pkv::kEntryCost * (int64_t)batch + pkv::kTileCost - 1) /
                                 pkv::kTileCost +
                             5 * wb;
        const int64_t shortest = wb * (3 + 2 * (int64_t)pkv::kMinRunTiles);
        block_ints4 = full > shortest ? full : shortest;
    }
    p.off_ent = align256((int64_t)batch * d.num_kv_heads * 4);
    p.off_blocks = p.off_ent + align256((int64_t)batch * 16);
    block_ints4 += pkv::kMaxStageBuffers;   // records read ahead past the last block
    p.off_part_o = p.off_blocks + align256(block_ints4 * 16);
    const int64_t rows = p.slots * num_qo_heads;
    p.off_part_lse = p.off_part_o + align256(rows * d.head_dim * 2);
    p.off_list = p.off_part_lse + align256(rows * 8);
    // a mixed plan over `batch` rows lists at most batch / 2 entries with
    // several rows (and one more under a malformed qo_indptr is dropped)
    p.list_cap = batch / 2 + 1;
    p.ws_bytes = p.off_list + align256(((int64_t)p.list_cap + 2) * 4);
    return p;
}

int check_decode_args(const pkv_cache_desc_t &desc, int32_t layer, int32_t num_qo_heads,
                      int32_t batch, float sm_scale, int32_t max_pages_per_req,
                      int32_t kv_chunk_pages) {
    int rc = check_desc(desc);
    if (rc != PKV_OK)
        return rc;
    if (layer < 0 || layer >= desc.num_layers || batch < 0 || num_qo_heads < 1 ||
        num_qo_heads % desc.num_kv_heads != 0 || !isfinite(sm_scale) ||
        max_pages_per_req < 1 || kv_chunk_pages < 0)
        return PKV_ERR_BAD_SHAPE;
    if (kv_chunk_pages > pkv::kMaxChunkPages || batch > pkv::kMaxPlanBatch)
        return PKV_ERR_UNSUPPORTED;
    const int group = num_qo_heads / desc.num_kv_heads;
    if ((desc.head_dim != 64 && desc.head_dim != 128) || group > 8 ||
        desc.num_kv_heads > pkv::kMaxKvHeads || !pkv::run_supported(desc.head_dim, group))
        return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

// Checks shared by pkv_plan and pkv_run; fills the layout and the number of
// decode workgroups along x.
int prepare(const pkv_cache_desc_t &desc, int32_t num_qo_heads, int32_t batch,
            int32_t max_pages_per_req, int32_t kv_chunk_pages, const void *workspace,
            size_t workspace_bytes, Layout &lay, int &num_blocks, int &block_stride) {
    lay = make_layout(desc, num_qo_heads, batch, max_pages_per_req, kv_chunk_pages);
    // tile and block indices, and byte offsets into the partial arrays, are
    // 32-bit in the kernels
    if (lay.max_tiles > 0x3fffffffLL || lay.ws_bytes - lay.off_part_o > 0x7fffffffLL)
        return PKV_ERR_BAD_SHAPE;
    if (workspace == nullptr || workspace_bytes < (size_t)lay.ws_bytes)
        return PKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return PKV_ERR_ALIGNMENT;
    // both modes keep the workgroups the GPU holds at once busy
    const int group = num_qo_heads / desc.num_kv_heads;
    hipError_t err = pkv::balanced_blocks(desc.head_dim, group, desc.num_kv_heads, &num_blocks);
    if (err != hipSuccess)
        return hip_status(err);
    if (lay.chunk_tiles > 0) {
        const int64_t cap = pkv::fixed_capacity(lay.slots, lay.chunk_tiles,
                                                lay.max_tiles / (batch > 0 ? batch : 1),
                                                num_blocks);
        if ((int64_t)num_blocks * (1 + cap) > 0x3fffffffLL)
            return PKV_ERR_BAD_SHAPE;
        block_stride = (int)(1 + cap);
    } else {
        block_stride = (int)(1 + pkv::balanced_capacity(lay.max_tiles, batch, num_blocks));
    }
    return PKV_OK;
}

// The signature of a plan: a nonzero hash (FNV-1a) of the arguments it is
// made for.  pkv_plan writes it into every block header and each pkv_run
// compares it with the hash of its own arguments, so a run on a plan made for
// other arguments (or on a workspace that holds no plan) is caught before it
// uses a record.
int32_t plan_signature(const pkv_cache_desc_t &desc, int32_t num_qo_heads, int32_t batch,
                       int32_t max_pages_per_req, int32_t kv_chunk_pages, const Layout &lay,
                       int num_blocks, int block_stride, bool mixed) {
    const int32_t v[] = {batch, num_qo_heads, desc.num_kv_heads, desc.page_size,
                         desc.head_dim, max_pages_per_req, kv_chunk_pages, desc.num_pages,
                         num_blocks, block_stride, lay.tiles_per_page, mixed ? 1 : 0};
    uint32_t h = 2166136261u;
    for (int32_t x : v)
        for (int k = 0; k < 4; ++k) {
            h ^= ((uint32_t)x >> (8 * k)) & 0xFFu;
            h *= 16777619u;
        }
    return (int32_t)(h | 1u);
}

// Host checks of a pkv_plan call; on success `args` is ready to launch.
int prepare_plan(pkv_cache_desc_t desc, int32_t num_qo_heads, const int32_t *page_indptr,
                 const int32_t *page_indices, const int32_t *last_page_len, int32_t batch,
                 int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
                 size_t workspace_bytes, pkv::PlanArgs &a, bool mixed = false) {
    int rc = check_decode_args(desc, 0, num_qo_heads, batch, 1.f, max_pages_per_req,
                               kv_chunk_pages);
    if (rc != PKV_OK)
        return rc;
    if (!page_indptr || !page_indices || !last_page_len)
        return PKV_ERR_NULL_PTR;
    Layout lay;
    int num_blocks = 0, block_stride = 0;
    rc = prepare(desc, num_qo_heads, batch, max_pages_per_req, kv_chunk_pages, workspace,
                 workspace_bytes, lay, num_blocks, block_stride);
    if (rc != PKV_OK)
        return rc;
    char *ws = static_cast<char *>(workspace);
    a.indptr = page_indptr;
    a.indices = page_indices;
    a.last_len = last_page_len;
    a.blocks = reinterpret_cast<int32_t *>(ws + lay.off_blocks);
    a.ent = reinterpret_cast<int32_t *>(ws + lay.off_ent);
    a.cnt = reinterpret_cast<int32_t *>(ws);
    a.plan_sig = plan_signature(desc, num_qo_heads, batch, max_pages_per_req, kv_chunk_pages,
                                lay, num_blocks, block_stride, mixed);
    a.batch = batch;
    a.qo_indptr = nullptr;   // set by the mixed plan
    a.num_entries = batch;
    a.list = reinterpret_cast<int32_t *>(ws + lay.off_list);
    a.list_cap = lay.list_cap;
    a.num_pages = desc.num_pages;
    a.page_size = desc.page_size;
    a.tiles_per_page = lay.tiles_per_page;
    a.num_kv_heads = desc.num_kv_heads;
    a.num_blocks = num_blocks;
    a.block_stride = block_stride;
    a.chunk_tiles = lay.chunk_tiles;
    a.max_chunks = lay.max_chunks;
    a.max_pages = max_pages_per_req;
    return PKV_OK;
}

// Host checks of a pkv_run call; on success `args` and the launch shape are set.
struct RunLaunch {
    pkv::RunArgs args;
    const int32_t *blocks = nullptr;
    const int32_t *ent = nullptr;
    const int32_t *list = nullptr;   // a mixed plan's prefill list
    int32_t list_cap = 0;
    int num_blocks = 0;
    int group = 0;
};

int prepare_run(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *k_new,
                const void *v_new, const void *q, int32_t num_qo_heads, int32_t batch,
                float sm_scale, void *out, float *lse, int32_t max_pages_per_req,
                int32_t kv_chunk_pages, void *workspace, size_t workspace_bytes,
                RunLaunch &r, bool mixed = false) {
    int rc = check_decode_args(desc, layer, num_qo_heads, batch, sm_scale, max_pages_per_req,
                               kv_chunk_pages);
    if (rc != PKV_OK)
        return rc;
    const bool fused = k_new != nullptr || v_new != nullptr;
    if (!kv_cache || !q || !out || (fused && (!k_new || !v_new)))
        return PKV_ERR_NULL_PTR;
    if (!aligned16(kv_cache) || !aligned16(q) || !aligned16(out) ||
        (fused && (!aligned16(k_new) || !aligned16(v_new))))
        return PKV_ERR_ALIGNMENT;
    Layout lay;
    int num_blocks = 0, block_stride = 0;
    rc = prepare(desc, num_qo_heads, batch, max_pages_per_req, kv_chunk_pages, workspace,
                 workspace_bytes, lay, num_blocks, block_stride);
    if (rc != PKV_OK)
        return rc;
    char *ws = static_cast<char *>(workspace);
    pkv::RunArgs &a = r.args;
    const int64_t layer_off = (int64_t)layer * desc.num_pages * page_elems(desc);
    a.cache = static_cast<const uint16_t *>(kv_cache) + layer_off;
    a.cache_w = fused ? static_cast<uint16_t *>(kv_cache) + layer_off : nullptr;
    a.q = static_cast<const uint16_t *>(q);
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.part_o = reinterpret_cast<uint16_t *>(ws + lay.off_part_o);
    a.part_lse = reinterpret_cast<float *>(ws + lay.off_part_lse);
    a.part_o_bytes = lay.off_part_lse - lay.off_part_o;
    a.part_lse_bytes = lay.ws_bytes - lay.off_part_lse;
    a.cnt = reinterpret_cast<int32_t *>(ws);
    a.plan_sig = plan_signature(desc, num_qo_heads, batch, max_pages_per_req, kv_chunk_pages,
                                lay, num_blocks, block_stride, mixed);
    a.num_pages = desc.num_pages;
    a.page_size = desc.page_size;
    a.page_stride = page_elems(desc);
    a.half_stride = desc.page_size * desc.num_kv_heads * desc.head_dim;
    a.row_stride = desc.num_kv_heads * desc.head_dim;
    a.num_qo_heads = num_qo_heads;
    a.num_kv_heads = desc.num_kv_heads;
    a.batch = batch;
    a.block_stride = block_stride;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    a.q_w = nullptr;
    a.k_w = nullptr;
    a.positions = nullptr;
    a.pos_stride = 1;
    a.axis_bits[0] = a.axis_bits[1] = a.axis_bits[2] = a.axis_bits[3] = 0;
    a.eps = 0.f;
    a.log2_theta = 0.0;
    r.blocks = reinterpret_cast<const int32_t *>(ws + lay.off_blocks);
    r.ent = reinterpret_cast<const int32_t *>(ws + lay.off_ent);
    r.list = reinterpret_cast<const int32_t *>(ws + lay.off_list);
    r.list_cap = lay.list_cap;
    r.num_blocks = num_blocks;
    r.group = num_qo_heads / desc.num_kv_heads;
    return PKV_OK;
}

int launch_run(const RunLaunch &r, const pkv_cache_desc_t &desc, hipStream_t stream) {
    return hip_status(pkv::launch_run(r.args, r.blocks, r.ent, r.num_blocks, desc.head_dim,
                                      r.group, stream));
}

// pkv_decode and pkv_append_decode: every host check of both halves first,
// then the plan and the run.
int plan_and_run(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *k_new,
                 const void *v_new, const void *q, int32_t num_qo_heads,
                 const int32_t *page_indptr, const int32_t *page_indices,
                 const int32_t *last_page_len, int32_t batch, float sm_scale, void *out,
                 float *lse, int32_t max_pages_per_req, int32_t kv_chunk_pages,
                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_decode_args(desc, layer, num_qo_heads, batch, sm_scale, max_pages_per_req,
                               kv_chunk_pages);
    if (rc != PKV_OK || batch == 0)
        return rc;
    if (!page_indptr || !page_indices || !last_page_len)
        return PKV_ERR_NULL_PTR;
    RunLaunch r;
    rc = prepare_run(kv_cache, desc, layer, k_new, v_new, q, num_qo_heads, batch, sm_scale,
                     out, lse, max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes,
                     r);
    if (rc != PKV_OK)
        return rc;
    pkv::PlanArgs pa;
    rc = prepare_plan(desc, num_qo_heads, page_indptr, page_indices, last_page_len, batch,
                      max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes, pa);
    if (rc != PKV_OK)
        return rc;
    rc = hip_status(pkv::launch_plan(pa, stream));
    if (rc != PKV_OK)
        return rc;
    return launch_run(r, desc, stream);
}


// pkv_run_qk_norm_rope and its multimodal variant (pair_axis read on the
// host: the component each rotary pair follows).
int run_norm_rope(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *k_new,
                  const void *v_new, const void *q, int32_t num_qo_heads, int32_t batch,
                  const void *q_norm_weight, const void *k_norm_weight, float eps,
                  float rope_theta, const int32_t *positions, const uint8_t *pair_axis,
                  bool multimodal, float sm_scale, void *out, float *lse,
                  int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
                  size_t workspace_bytes, hipStream_t stream) {
    int rc = check_decode_args(desc, layer, num_qo_heads, batch, sm_scale, max_pages_per_req,
                               kv_chunk_pages);
    if (rc != PKV_OK)
        return rc;
    if (!(eps >= 0.0f) || !isfinite(eps) || !(rope_theta > 0.0f) || !isfinite(rope_theta))
        return PKV_ERR_BAD_SHAPE;
    if (!pkv::run_norm_rope_supported(desc.head_dim, num_qo_heads / desc.num_kv_heads))
        return PKV_ERR_UNSUPPORTED;
    uint32_t axis_bits[4] = {0, 0, 0, 0};
    if (multimodal) {
        if (!pair_axis)
            return PKV_ERR_NULL_PTR;
        for (int i = 0; i < desc.head_dim / 2; ++i) {
            if (pair_axis[i] > 2)
                return PKV_ERR_BAD_SHAPE;
            axis_bits[i / 16] |= (uint32_t)pair_axis[i] << (2 * (i % 16));
        }
    }
    if (batch == 0)
        return PKV_OK;
    if (!k_new || !v_new || !q_norm_weight || !k_norm_weight || !positions)
        return PKV_ERR_NULL_PTR;
    if (!aligned16(q_norm_weight) || !aligned16(k_norm_weight))
        return PKV_ERR_ALIGNMENT;
    RunLaunch r;
    rc = prepare_run(kv_cache, desc, layer, k_new, v_new, q, num_qo_heads, batch, sm_scale,
                     out, lse, max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes,
                     r);
    if (rc != PKV_OK)
        return rc;
    pkv::RunArgs &a = r.args;
    a.q_w = static_cast<const uint16_t *>(q_norm_weight);
    a.k_w = static_cast<const uint16_t *>(k_norm_weight);
    a.positions = positions;
    a.eps = eps;
    a.log2_theta = log2((double)rope_theta);
    a.pos_stride = multimodal ? 3 : 1;
    for (int i = 0; i < 4; ++i)
        a.axis_bits[i] = axis_bits[i];
    return launch_run(r, desc, stream);
}


// Host checks of a prefill launch (pkv_prefill and the prefill half of
// pkv_mixed_run); on success `a` is ready, and `any` says whether there is
// work (batch > 0).
int prepare_prefill(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
                    int32_t num_qo_heads, const int32_t *qo_indptr, const void *k_new,
                    const void *v_new, const int32_t *page_indptr, const int32_t *page_indices,
                    const int32_t *last_page_len, int32_t batch, int32_t max_q_rows,
                    float sm_scale, void *out, float *lse, pkv::PrefillArgs &a, bool &any) {
    any = false;
    int rc = check_desc(desc);
    if (rc != PKV_OK)
        return rc;
    if (layer < 0 || layer >= desc.num_layers || batch < 0 || num_qo_heads < 1 ||
        num_qo_heads > kMaxHeads || desc.num_kv_heads > kMaxHeads ||
        num_qo_heads % desc.num_kv_heads != 0 || max_q_rows < 1 || !isfinite(sm_scale))
        return PKV_ERR_BAD_SHAPE;
    if (!pkv::prefill_supported(desc.head_dim) || batch > 65535 ||
        2 * page_elems(desc) > (int64_t)UINT32_MAX)
        return PKV_ERR_UNSUPPORTED;
    if (batch == 0)
        return PKV_OK;
    const bool append = k_new != nullptr || v_new != nullptr;
    if (!kv_cache || !q || !qo_indptr || !page_indptr || !page_indices || !last_page_len ||
        !out || (append && (!k_new || !v_new)))
        return PKV_ERR_NULL_PTR;
    if (!aligned16(kv_cache) || !aligned16(q) || !aligned16(out) ||
        (append && (!aligned16(k_new) || !aligned16(v_new))))
        return PKV_ERR_ALIGNMENT;
    uint16_t *slab = static_cast<uint16_t *>(kv_cache) + (int64_t)layer * desc.num_pages * page_elems(desc);
    a.cache = slab;
    a.cache_w = append ? slab : nullptr;
    a.q = static_cast<const uint16_t *>(q);
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.qo_indptr = qo_indptr;
    a.indptr = page_indptr;
    a.indices = page_indices;
    a.last_len = last_page_len;
    a.page_stride = page_elems(desc);
    a.half_stride = desc.page_size * desc.num_kv_heads * desc.head_dim;
    a.row_stride = desc.num_kv_heads * desc.head_dim;
    a.num_pages = desc.num_pages;
    a.page_size = desc.page_size;
    a.num_qo_heads = num_qo_heads;
    a.num_kv_heads = desc.num_kv_heads;
    a.head_dim = desc.head_dim;
    a.batch = batch;
    a.max_rows = max_q_rows;
    const int64_t col_tiles = ((int64_t)max_q_rows * (num_qo_heads / desc.num_kv_heads) + 127) / 128;
    a.pair_tiles = (int32_t)((col_tiles + 1) / 2);
    a.skip_single = 0;
    a.list = nullptr;
    a.list_sig = 0;
    a.list_cap = 0;
    a.page_shift = 0;
    while ((1 << a.page_shift) < desc.page_size)
        ++a.page_shift;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    any = true;
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_last_hip_error(void) { return g_last_hip_error; }

const char *pkv_status_string(int status) {
    switch (status) {
    case PKV_OK: return "PKV_OK: success";
    case PKV_ERR_NULL_PTR: return "PKV_ERR_NULL_PTR: a required pointer is NULL";
    case PKV_ERR_BAD_SHAPE: return "PKV_ERR_BAD_SHAPE: a size, index or scale is out of range";
    case PKV_ERR_UNSUPPORTED:
        return "PKV_ERR_UNSUPPORTED: shape not built (head_dim, group, heads or page_size)";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: workspace missing or too small";
    case PKV_ERR_HIP: return "PKV_ERR_HIP: the HIP runtime refused a launch";
    case PKV_ERR_ALIGNMENT: return "PKV_ERR_ALIGNMENT: an array is not aligned as required";
    case PKV_ERR_BAD_TABLE: return "PKV_ERR_BAD_TABLE: the page table breaks a precondition";
    default: return "unknown pkv status";
    }
}

int pkv_append(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *k_new,
               const void *v_new, const int32_t *page_indptr, const int32_t *page_indices,
               const int32_t *last_page_len, int32_t batch, hipStream_t stream) {
    int rc = check_desc(desc);
    if (rc != PKV_OK)
        return rc;
    if (layer < 0 || layer >= desc.num_layers || batch < 0)
        return PKV_ERR_BAD_SHAPE;
    if (desc.head_dim % 8 != 0)
        return PKV_ERR_UNSUPPORTED;
    if (batch == 0)
        return PKV_OK;
    if (!kv_cache || !k_new || !v_new || !page_indptr || !page_indices || !last_page_len)
        return PKV_ERR_NULL_PTR;
    if (!aligned16(kv_cache) || !aligned16(k_new) || !aligned16(v_new))
        return PKV_ERR_ALIGNMENT;
    pkv::AppendArgs a;
    a.cache = static_cast<uint16_t *>(kv_cache) + (int64_t)layer * desc.num_pages * page_elems(desc);
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.indptr = page_indptr;
    a.indices = page_indices;
    a.last_len = last_page_len;
    a.page_stride = page_elems(desc);
    a.half_stride = desc.page_size * desc.num_kv_heads * desc.head_dim;
    a.row_elems = desc.num_kv_heads * desc.head_dim;
    a.num_pages = desc.num_pages;
    a.page_size = desc.page_size;
    return hip_status(pkv::launch_append(a, batch, stream));
}

int pkv_prefill(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
                int32_t num_qo_heads, const int32_t *qo_indptr, const void *k_new,
                const void *v_new, const int32_t *page_indptr, const int32_t *page_indices,
                const int32_t *last_page_len, int32_t batch, int32_t max_q_rows,
                float sm_scale, void *out, float *lse, hipStream_t stream) {
    pkv::PrefillArgs a;
    bool any = false;
    const int rc = prepare_prefill(kv_cache, desc, layer, q, num_qo_heads, qo_indptr, k_new,
                                   v_new, page_indptr, page_indices, last_page_len, batch,
                                   max_q_rows, sm_scale, out, lse, a, any);
    if (rc != PKV_OK || !any)
        return rc;
    return hip_status(pkv::launch_prefill(a, stream));
}

int pkv_plan_mixed(pkv_cache_desc_t desc, int32_t num_qo_heads, const int32_t *qo_indptr,
                   const int32_t *page_indptr, const int32_t *page_indices,
                   const int32_t *last_page_len, int32_t batch, int32_t total_rows,
                   int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    if (batch < 0 || total_rows < 0)
        return PKV_ERR_BAD_SHAPE;
    if (batch > 65535)
        return PKV_ERR_UNSUPPORTED;
    int rc = check_decode_args(desc, 0, num_qo_heads, total_rows, 1.f, max_pages_per_req,
                               kv_chunk_pages);
    if (rc != PKV_OK || total_rows == 0 || batch == 0)
        return rc;
    if (!qo_indptr)
        return PKV_ERR_NULL_PTR;
    pkv::PlanArgs a;
    rc = prepare_plan(desc, num_qo_heads, page_indptr, page_indices, last_page_len, total_rows,
                      max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes, a, true);
    if (rc != PKV_OK)
        return rc;
    a.qo_indptr = qo_indptr;
    a.num_entries = batch;
    return hip_status(pkv::launch_plan(a, stream));
}

int pkv_mixed_run(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
                  int32_t num_qo_heads, const int32_t *qo_indptr, const void *k_new,
                  const void *v_new, const int32_t *page_indptr, const int32_t *page_indices,
                  const int32_t *last_page_len, int32_t batch, int32_t total_rows,
                  int32_t max_q_rows, float sm_scale, void *out, float *lse,
                  int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
                  size_t workspace_bytes, hipStream_t stream) {
    if (total_rows < 0)
        return PKV_ERR_BAD_SHAPE;
    // every host check of both halves first
    pkv::PrefillArgs pa;
    bool any = false;
    int rc = prepare_prefill(kv_cache, desc, layer, q, num_qo_heads, qo_indptr, k_new, v_new,
                             page_indptr, page_indices, last_page_len, batch, max_q_rows,
                             sm_scale, out, lse, pa, any);
    if (rc != PKV_OK || !any || total_rows == 0)
        return rc;
    RunLaunch r;
    rc = prepare_run(kv_cache, desc, layer, k_new, v_new, q, num_qo_heads, total_rows, sm_scale,
                     out, lse, max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes, r,
                     true);
    if (rc != PKV_OK)
        return rc;
    rc = launch_run(r, desc, stream);
    if (rc != PKV_OK)
        return rc;
    // the prompts the plan listed; the decode rows went through the run above
    pa.skip_single = 1;
    pa.list = r.list;
    pa.list_sig = r.args.plan_sig;
    pa.list_cap = r.list_cap;
    return hip_status(pkv::launch_prefill(pa, stream));
}

}  // extern "C"

namespace {

// pkv_qk_norm_rope_append and its multimodal variant (pair_axis non-null:
// positions [batch, 3], pair i following component pair_axis[i]).
int norm_rope_append(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
                     int32_t num_qo_heads, const void *k_new, const void *v_new,
                     const void *q_norm_weight, const void *k_norm_weight, float eps,
                     float rope_theta, const int32_t *positions, const uint8_t *pair_axis,
                     bool multimodal, const int32_t *page_indptr, const int32_t *page_indices,
                     const int32_t *last_page_len, int32_t batch, void *q_out,
                     hipStream_t stream) {
    int rc = check_desc(desc);
    if (rc != PKV_OK)
        return rc;
    if (layer < 0 || layer >= desc.num_layers || batch < 0 || num_qo_heads < 1 ||
        num_qo_heads > kMaxHeads || desc.num_kv_heads > kMaxHeads ||
        !(eps >= 0.0f) || !isfinite(eps) || !(rope_theta > 0.0f) || !isfinite(rope_theta))
        return PKV_ERR_BAD_SHAPE;
    // one wave per (entry, head): the wave count is formed in 64 bits
    if ((int64_t)batch * ((int64_t)num_qo_heads + desc.num_kv_heads) > 0x7fffffffLL * 4)
        return PKV_ERR_BAD_SHAPE;
    if (!pkv::norm_rope_supported(desc.head_dim))
        return PKV_ERR_UNSUPPORTED;
    uint32_t axis_bits[4] = {0, 0, 0, 0};
    if (multimodal) {
        if (!pair_axis)
            return PKV_ERR_NULL_PTR;
        for (int i = 0; i < desc.head_dim / 2; ++i) {
            if (pair_axis[i] > 2)
                return PKV_ERR_BAD_SHAPE;
            axis_bits[i / 16] |= (uint32_t)pair_axis[i] << (2 * (i % 16));
        }
    }
    if (batch == 0)
        return PKV_OK;
    if (!kv_cache || !q || !k_new || !v_new || !q_norm_weight || !k_norm_weight ||
        !positions || !page_indptr || !page_indices || !last_page_len || !q_out)
        return PKV_ERR_NULL_PTR;
    if (!aligned16(kv_cache) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new) ||
        !aligned16(q_norm_weight) || !aligned16(k_norm_weight) || !aligned16(q_out))
        return PKV_ERR_ALIGNMENT;
    pkv::NormRopeArgs a;
    a.cache = static_cast<uint16_t *>(kv_cache) + (int64_t)layer * desc.num_pages * page_elems(desc);
    a.q = static_cast<const uint16_t *>(q);
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.q_w = static_cast<const uint16_t *>(q_norm_weight);
    a.k_w = static_cast<const uint16_t *>(k_norm_weight);
    a.q_out = static_cast<uint16_t *>(q_out);
    a.positions = positions;
    a.indptr = page_indptr;
    a.indices = page_indices;
    a.last_len = last_page_len;
    a.page_stride = page_elems(desc);
    a.half_stride = desc.page_size * desc.num_kv_heads * desc.head_dim;
    a.row_elems = desc.num_kv_heads * desc.head_dim;
    a.num_pages = desc.num_pages;
    a.page_size = desc.page_size;
    a.num_qo_heads = num_qo_heads;
    a.num_kv_heads = desc.num_kv_heads;
    a.head_dim = desc.head_dim;
    a.batch = batch;
    a.eps = eps;
    a.pos_stride = multimodal ? 3 : 1;
    for (int i = 0; i < 4; ++i)
        a.axis_bits[i] = axis_bits[i];
    for (int i = 0; i < 64; ++i)
        a.turns[i] = i < desc.head_dim / 2
                         ? pow((double)rope_theta, -2.0 * i / desc.head_dim) / (2.0 * M_PI)
                         : 0.0;
    return hip_status(pkv::launch_norm_rope(a, stream));
}

}  // namespace

extern "C" {

int pkv_qk_norm_rope_append(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                            const void *q, int32_t num_qo_heads, const void *k_new,
                            const void *v_new, const void *q_norm_weight,
                            const void *k_norm_weight, float eps, float rope_theta,
                            const int32_t *positions, const int32_t *page_indptr,
                            const int32_t *page_indices, const int32_t *last_page_len,
                            int32_t batch, void *q_out, hipStream_t stream) {
    return norm_rope_append(kv_cache, desc, layer, q, num_qo_heads, k_new, v_new,
                            q_norm_weight, k_norm_weight, eps, rope_theta, positions, nullptr,
                            false, page_indptr, page_indices, last_page_len, batch, q_out,
                            stream);
}

int pkv_qk_norm_mrope_append(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                             const void *q, int32_t num_qo_heads, const void *k_new,
                             const void *v_new, const void *q_norm_weight,
                             const void *k_norm_weight, float eps, float rope_theta,
                             const int32_t *positions, const uint8_t *pair_axis,
                             const int32_t *page_indptr, const int32_t *page_indices,
                             const int32_t *last_page_len, int32_t batch, void *q_out,
                             hipStream_t stream) {
    return norm_rope_append(kv_cache, desc, layer, q, num_qo_heads, k_new, v_new,
                            q_norm_weight, k_norm_weight, eps, rope_theta, positions, pair_axis,
                            true, page_indptr, page_indices, last_page_len, batch, q_out,
                            stream);
}

int pkv_run_qk_norm_rope(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                         const void *k_new, const void *v_new, const void *q,
                         int32_t num_qo_heads, int32_t batch, const void *q_norm_weight,
                         const void *k_norm_weight, float eps, float rope_theta,
                         const int32_t *positions, float sm_scale, void *out, float *lse,
                         int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return run_norm_rope(kv_cache, desc, layer, k_new, v_new, q, num_qo_heads, batch,
                         q_norm_weight, k_norm_weight, eps, rope_theta, positions, nullptr,
                         false, sm_scale, out, lse, max_pages_per_req, kv_chunk_pages,
                         workspace, workspace_bytes, stream);
}

int pkv_run_qk_norm_mrope(void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                          const void *k_new, const void *v_new, const void *q,
                          int32_t num_qo_heads, int32_t batch, const void *q_norm_weight,
                          const void *k_norm_weight, float eps, float rope_theta,
                          const int32_t *positions, const uint8_t *pair_axis, float sm_scale,
                          void *out, float *lse, int32_t max_pages_per_req,
                          int32_t kv_chunk_pages, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return run_norm_rope(kv_cache, desc, layer, k_new, v_new, q, num_qo_heads, batch,
                         q_norm_weight, k_norm_weight, eps, rope_theta, positions, pair_axis,
                         true, sm_scale, out, lse, max_pages_per_req, kv_chunk_pages,
                         workspace, workspace_bytes, stream);
}

size_t pkv_decode_workspace_size(pkv_cache_desc_t desc, int32_t num_qo_heads, int32_t batch,
                                 int32_t max_pages_per_req, int32_t kv_chunk_pages) {
    if (check_desc(desc) != PKV_OK || batch <= 0 || num_qo_heads <= 0 ||
        max_pages_per_req <= 0 || kv_chunk_pages < 0)
        return 0;
    return (size_t)make_layout(desc, num_qo_heads, batch, max_pages_per_req, kv_chunk_pages)
        .ws_bytes;
}

int pkv_plan(pkv_cache_desc_t desc, int32_t num_qo_heads, const int32_t *page_indptr,
             const int32_t *page_indices, const int32_t *last_page_len, int32_t batch,
             int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
             size_t workspace_bytes, hipStream_t stream) {
    int rc = check_decode_args(desc, 0, num_qo_heads, batch, 1.f, max_pages_per_req,
                               kv_chunk_pages);
    if (rc != PKV_OK || batch == 0)
        return rc;
    pkv::PlanArgs a;
    rc = prepare_plan(desc, num_qo_heads, page_indptr, page_indices, last_page_len, batch,
                      max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes, a);
    if (rc != PKV_OK)
        return rc;
    return hip_status(pkv::launch_plan(a, stream));
}

int pkv_run(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *k_new,
            const void *v_new, const void *q, int32_t num_qo_heads, int32_t batch,
            float sm_scale, void *out, float *lse, int32_t max_pages_per_req,
            int32_t kv_chunk_pages, void *workspace, size_t workspace_bytes,
            hipStream_t stream) {
    int rc = check_decode_args(desc, layer, num_qo_heads, batch, sm_scale, max_pages_per_req,
                               kv_chunk_pages);
    if (rc != PKV_OK || batch == 0)
        return rc;
    RunLaunch r;
    rc = prepare_run(kv_cache, desc, layer, k_new, v_new, q, num_qo_heads, batch, sm_scale,
                     out, lse, max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes,
                     r);
    if (rc != PKV_OK)
        return rc;
    return launch_run(r, desc, stream);
}

int pkv_decode(const void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
               int32_t num_qo_heads, const int32_t *page_indptr, const int32_t *page_indices,
               const int32_t *last_page_len, int32_t batch, float sm_scale, void *out,
               float *lse, int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
               size_t workspace_bytes, hipStream_t stream) {
    return plan_and_run(const_cast<void *>(kv_cache), desc, layer, nullptr, nullptr, q,
                        num_qo_heads, page_indptr, page_indices, last_page_len, batch,
                        sm_scale, out, lse, max_pages_per_req, kv_chunk_pages, workspace,
                        workspace_bytes, stream);
}

int pkv_append_decode(void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *k_new,
                      const void *v_new, const void *q, int32_t num_qo_heads,
                      const int32_t *page_indptr, const int32_t *page_indices,
                      const int32_t *last_page_len, int32_t batch, float sm_scale, void *out,
                      float *lse, int32_t max_pages_per_req, int32_t kv_chunk_pages,
                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const int rc = check_decode_args(desc, layer, num_qo_heads, batch, sm_scale,
                                     max_pages_per_req, kv_chunk_pages);
    if (rc != PKV_OK || batch == 0)
        return rc;
    if (k_new == nullptr || v_new == nullptr)
        return PKV_ERR_NULL_PTR;
    return plan_and_run(kv_cache, desc, layer, k_new, v_new, q, num_qo_heads, page_indptr,
                        page_indices, last_page_len, batch, sm_scale, out, lse,
                        max_pages_per_req, kv_chunk_pages, workspace, workspace_bytes, stream);
}

int pkv_decode_static(const void *kv_cache, pkv_cache_desc_t desc, int32_t layer,
                      const void *q, int32_t num_qo_heads, const int32_t *page_indptr,
                      const int32_t *page_indices, const int32_t *last_page_len,
                      int32_t batch, float sm_scale, void *out, float *lse,
                      int32_t max_pages_per_req, int32_t kv_chunk_pages, hipStream_t stream) {
    const int rc = check_decode_args(desc, layer, num_qo_heads, batch, sm_scale,
                                     max_pages_per_req, kv_chunk_pages);
    if (rc != PKV_OK || batch == 0)
        return rc;
    // the size check is host arithmetic only: nothing reaches the device for
    // a call the array cannot hold
    const Layout lay = make_layout(desc, num_qo_heads, batch, max_pages_per_req,
                                   kv_chunk_pages);
    if ((uint64_t)lay.ws_bytes > (uint64_t)pkv::kStaticScratchBytes)
        return PKV_ERR_WORKSPACE;
    void *scratch = nullptr;
    const int hrc = hip_status(pkv::static_scratch(&scratch));
    if (hrc != PKV_OK)
        return hrc;
    return plan_and_run(const_cast<void *>(kv_cache), desc, layer, nullptr, nullptr, q,
                        num_qo_heads, page_indptr, page_indices, last_page_len, batch,
                        sm_scale, out, lse, max_pages_per_req, kv_chunk_pages, scratch,
                        pkv::kStaticScratchBytes, stream);
}

int pkv_validate_page_table(const int32_t *page_indptr, const int32_t *page_indices,
                            const int32_t *last_page_len, int32_t batch, int32_t num_pages,
                            int32_t page_size, int32_t max_pages_per_req, int32_t *bad_entry) {
    if (bad_entry)
        *bad_entry = -1;
    if (batch < 0 || num_pages < 1 || page_size < 1)
        return PKV_ERR_BAD_SHAPE;
    if (batch == 0)
        return PKV_OK;
    if (!page_indptr || !page_indices || !last_page_len)
        return PKV_ERR_NULL_PTR;
    if (page_indptr[0] != 0)
        return PKV_ERR_BAD_TABLE;
    // which entry appends into each real page (tail pages only)
    int32_t *owner = static_cast<int32_t *>(malloc(sizeof(int32_t) * (size_t)num_pages));
    if (!owner)
        return PKV_ERR_BAD_SHAPE;
    for (int32_t p = 0; p < num_pages; ++p)
        owner[p] = -1;
    int status = PKV_OK;
    for (int32_t b = 0; b < batch && status == PKV_OK; ++b) {
        const int64_t n = (int64_t)page_indptr[b + 1] - page_indptr[b];
        const int32_t last = last_page_len[b];
        bool ok = n >= 1 && (max_pages_per_req <= 0 || n <= max_pages_per_req) && last >= 1 &&
                  last <= page_size;
        bool uses_zero = false;
        for (int64_t i = 0; ok && i < n; ++i) {
            const int32_t p = page_indices[page_indptr[b] + i];
            ok = p >= 0 && p < num_pages;
            uses_zero |= ok && p == 0;
        }
        if (ok && uses_zero)
            ok = n == 1 && last == 1;   // a padding entry
        if (ok && !uses_zero) {
            // the append target is (tail page, last - 1); a real table never
            // lets two entries share a tail page, so any repeat is reported
            const int32_t tail = page_indices[page_indptr[b + 1] - 1];
            ok = owner[tail] < 0;
            owner[tail] = b;
        }
        if (!ok) {
            status = PKV_ERR_BAD_TABLE;
            if (bad_entry)
                *bad_entry = b;
        }
    }
    free(owner);
    return status;
}

}  // extern "C"
