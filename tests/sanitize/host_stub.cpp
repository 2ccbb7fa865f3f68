// host_stub.cpp -- test infrastructure: host-only stand-ins for the kernel
// launches of libpkv, so that the C ABI's host code (argument checks,
// workspace layout, plan signatures, page-table validation) can be built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven on a
// machine without a GPU.  Nothing here runs on a device.  Each stand-in
// checks the arguments the host code hands it for internal consistency and
// returns hipSuccess, or hipErrorInvalidValue when they are inconsistent (the
// driver then sees PKV_ERR_HIP and fails).  The support predicates answer as
// the gfx950 build does.
#include <stdint.h>

#include "pkv_launch.h"

namespace pkv {

namespace {
bool ordered(const void *a, const void *b) {
    return reinterpret_cast<uintptr_t>(a) < reinterpret_cast<uintptr_t>(b);
}
}  // namespace

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t) {
    if (!a.cache || !a.k_new || !a.v_new || batch < 1 || a.row_elems < 8 ||
        a.half_stride != a.row_elems * a.page_size || a.page_stride != 2LL * a.half_stride)
        return hipErrorInvalidValue;
    return hipSuccess;
}

bool prefill_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t) {
    if (!a.q || !a.out || ((a.k_new != nullptr) != (a.cache_w != nullptr)) || a.max_rows < 1 ||
        a.pair_tiles < 1 || a.num_qo_heads % a.num_kv_heads != 0 ||
        a.row_stride != a.num_kv_heads * a.head_dim)
        return hipErrorInvalidValue;
    return hipSuccess;
}

bool norm_rope_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_norm_rope(const NormRopeArgs &a, hipStream_t) {
    if (!a.q || !a.q_out || a.batch < 1 || (a.pos_stride != 1 && a.pos_stride != 3) ||
        a.turns[0] != 1.0 / (2.0 * 3.14159265358979323846) ||
        (a.head_dim == 64 && a.turns[32] != 0.0))
        return hipErrorInvalidValue;
    return hipSuccess;
}

hipError_t balanced_blocks(int head_dim, int group, int num_kv_heads, int *blocks) {
    if (!run_supported(head_dim, group))
        return hipErrorInvalidValue;
    // 256 compute units holding one workgroup each, shared by the head groups
    const int waves = group_waves(num_kv_heads);
    *blocks = (256 + num_kv_heads / waves - 1) / (num_kv_heads / waves);
    return hipSuccess;
}

bool run_supported(int head_dim, int group) {
    return (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 8;
}

bool run_norm_rope_supported(int head_dim, int group) {
    return head_dim == 128 && group >= 1 && group <= 4;
}

hipError_t launch_plan(const PlanArgs &a, hipStream_t) {
    // workspace regions in layout order: counters, entries, block records
    if (!ordered(a.cnt, a.ent) || !ordered(a.ent, a.blocks) || a.num_blocks < 1 ||
        a.block_stride < 2 || (a.plan_sig & 1) == 0 || a.max_pages < 1)
        return hipErrorInvalidValue;
    return hipSuccess;
}

hipError_t launch_run(const RunArgs &a, const int32_t *blocks, const int32_t *ent,
                      int num_blocks, int head_dim, int group, hipStream_t) {
    const char *po = reinterpret_cast<const char *>(a.part_o);
    const char *pl = reinterpret_cast<const char *>(a.part_lse);
    if (!ordered(a.cnt, ent) || !ordered(ent, blocks) || !ordered(blocks, a.part_o) ||
        po + a.part_o_bytes != pl || a.part_lse_bytes < 8 || num_blocks < 1 ||
        !run_supported(head_dim, group) || (a.plan_sig & 1) == 0 ||
        a.num_qo_heads != group * a.num_kv_heads || (a.cache_w && a.cache_w != a.cache))
        return hipErrorInvalidValue;
    return hipSuccess;
}

hipError_t static_scratch(void **ptr) {
    // a stand-in device address (never dereferenced), 256-byte aligned
    *ptr = reinterpret_cast<void *>(static_cast<uintptr_t>(0x7f0000000000ULL));
    return hipSuccess;
}

}  // namespace pkv
