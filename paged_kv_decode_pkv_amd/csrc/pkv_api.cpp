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

int log2_int(int32_t x) {
    int r = 0;
    while ((1 << r) < x)
        ++r;
    return r;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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

int32_t effective_chunk(int32_t kv_chunk_pages) {
    return kv_chunk_pages == 0 ? pkv::kDefaultChunkPages : kv_chunk_pages;
}

}  // namespace

extern "C" {

int32_t pkv_default_chunk_pages(void) { return pkv::kDefaultChunkPages; }

int pkv_last_hip_error(void) { return g_last_hip_error; }

const char *pkv_status_string(int status) {
    switch (status) {
    case PKV_OK: return "PKV_OK: success";
    case PKV_ERR_NULL_PTR: return "PKV_ERR_NULL_PTR: a required pointer is NULL";
    case PKV_ERR_BAD_SHAPE: return "PKV_ERR_BAD_SHAPE: a size, index or scale is out of range";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: shape not built (head_dim, group or page_size)";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: workspace missing or too small";
    case PKV_ERR_HIP: return "PKV_ERR_HIP: the HIP runtime refused a launch";
    case PKV_ERR_ALIGNMENT: return "PKV_ERR_ALIGNMENT: a bf16 array is not 16-byte aligned";
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

size_t pkv_decode_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t head_dim,
                                 int32_t max_pages_per_req, int32_t kv_chunk_pages) {
    const int32_t k = effective_chunk(kv_chunk_pages);
    if (batch <= 0 || num_qo_heads <= 0 || head_dim <= 0 || max_pages_per_req <= 0 || k <= 0)
        return 0;
    const int64_t chunks = (max_pages_per_req + (int64_t)k - 1) / k;
    if (chunks <= 1)
        return 0;
    const int64_t rows = (int64_t)batch * chunks * num_qo_heads;
    const int64_t bytes = rows * head_dim * 4 + rows * 4 + 256;
    return (size_t)((bytes + 255) / 256 * 256);
}

int pkv_decode(const void *kv_cache, pkv_cache_desc_t desc, int32_t layer, const void *q,
               int32_t num_qo_heads, const int32_t *page_indptr, const int32_t *page_indices,
               const int32_t *last_page_len, int32_t batch, float sm_scale, void *out,
               float *lse, int32_t max_pages_per_req, int32_t kv_chunk_pages, void *workspace,
               size_t workspace_bytes, hipStream_t stream) {
    int rc = check_desc(desc);
    if (rc != PKV_OK)
        return rc;
    if (layer < 0 || layer >= desc.num_layers || batch < 0 || num_qo_heads < 1 ||
        num_qo_heads % desc.num_kv_heads != 0 || !isfinite(sm_scale) ||
        max_pages_per_req < 1 || kv_chunk_pages < 0)
        return PKV_ERR_BAD_SHAPE;
    const int32_t chunk = effective_chunk(kv_chunk_pages);
    if (chunk > pkv::kMaxChunkPages)
        return PKV_ERR_UNSUPPORTED;
    const int group = num_qo_heads / desc.num_kv_heads;
    if ((desc.head_dim != 64 && desc.head_dim != 128) || group > 8)
        return PKV_ERR_UNSUPPORTED;
    if (batch == 0)
        return PKV_OK;
    if (!kv_cache || !q || !page_indptr || !page_indices || !last_page_len || !out)
        return PKV_ERR_NULL_PTR;
    if (!aligned16(kv_cache) || !aligned16(q) || !aligned16(out))
        return PKV_ERR_ALIGNMENT;
    const int64_t max_chunks = (max_pages_per_req + (int64_t)chunk - 1) / chunk;
    if ((int64_t)desc.num_kv_heads * max_chunks * batch > 0x7fffffffLL)
        return PKV_ERR_BAD_SHAPE;
    const size_t need = pkv_decode_workspace_size(batch, num_qo_heads, desc.head_dim,
                                                  max_pages_per_req, kv_chunk_pages);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return PKV_ERR_WORKSPACE;
    if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return PKV_ERR_ALIGNMENT;

    pkv::DecodeArgs a;
    a.cache = static_cast<const uint16_t *>(kv_cache) +
              (int64_t)layer * desc.num_pages * page_elems(desc);
    a.q = static_cast<const uint16_t *>(q);
    a.indptr = page_indptr;
    a.indices = page_indices;
    a.last_len = last_page_len;
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    const int64_t rows = (int64_t)batch * max_chunks * num_qo_heads;
    a.part_o = need ? static_cast<float *>(workspace) : nullptr;
    a.part_lse = need ? static_cast<float *>(workspace) + rows * desc.head_dim : nullptr;
    a.page_stride = page_elems(desc);
    a.half_stride = desc.page_size * desc.num_kv_heads * desc.head_dim;
    a.row_stride = desc.num_kv_heads * desc.head_dim;
    a.num_qo_heads = num_qo_heads;
    a.num_kv_heads = desc.num_kv_heads;
    a.num_pages = desc.num_pages;
    a.max_chunks = (int32_t)max_chunks;
    a.chunk_pages = chunk;
    a.page_size = desc.page_size;
    a.log2_page = log2_int(desc.page_size);
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    return hip_status(pkv::launch_decode(a, desc.head_dim, group, batch, stream));
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
    // slot owner per (page, slot) of real pages, to catch two appends landing
    // on one slot; sized on demand
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
            const int32_t tail = page_indices[page_indptr[b + 1] - 1];
            // the append target is (tail, last - 1); two entries may share a
            // tail page only at different slots, which a real table never
            // does, so any repeat of a tail page is reported
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
