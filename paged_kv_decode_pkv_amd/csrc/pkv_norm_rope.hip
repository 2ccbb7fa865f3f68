// pkv_norm_rope.hip -- fused q/k RMSNorm, rotary embedding and KV write for
// gfx950 (MI355X).
//
// The step that feeds the paged decode on Qwen3-style attention: each layer's
// q/k norm, RoPE and KV write run as one kernel, in fp32 throughout and
// rounded to bf16 once ("Supported Models", M* docs, Qwen3-Omni and Qwen3-TTS
// notes).  Per head of D values x at the entry's position p:
//   y = x / sqrt(mean(x^2) + eps) * w          (RMSNorm over the head)
//   z_i       = y_i cos a_i - y_{i+D/2} sin a_i,    a_i = p * theta^(-2i/D)
//   z_{i+D/2} = y_{i+D/2} cos a_i + y_i sin a_i      (rotate-half pairing)
// q heads go to q_out; k heads go to the K slot that the append fills, and
// the same wave copies the entry's V row, bit for bit, to the V slot.
//
// One wave per (entry, head) over the Hq query heads and then the Hkv key
// heads of every entry.  Lane l holds elements 2l and 2l + 1 of the row (one
// 4-byte word, so a row is one coalesced 256-byte access at D = 128); the
// element D/2 away sits in lane l ^ (D/4), and one lane swap brings it over.
// The angle is formed in turns and reduced to [-1/2, 1/2] of a turn in fp64
// (positions reach tens of thousands, where an fp32 product would already be
// off by a few thousandths of a radian; the fp64 product is off by about
// 1e-12 of a turn, and taking the nearest whole turn off is exact), then the
// sine and cosine and the rotation run in fp32.  The rates per pair come with the arguments,
// computed on the host.  Multimodal RoPE (the Qwen3-Omni Thinker's variant) gives
// each entry a (t, h, w) position and each pair the component it follows; the
// rest is the same.  The work is a few KiB per entry: the launch is bound
// by latency, not by HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_launch.h"

namespace pkv {
namespace {

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t float_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u | ((u >> 16) & 0x8000u);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int D, bool MR>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeArgs a) {
    constexpr int kLanes = D / 2;   // lanes holding a word of the row
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int heads = a.num_qo_heads + a.num_kv_heads;
    if (wave >= (int64_t)a.batch * heads)
        return;   // whole waves: the lane swaps below stay within live waves
    const int b = (int)(wave / heads);
    const int head = (int)(wave - (int64_t)b * heads);
    const bool is_q = head < a.num_qo_heads;
    const int h = is_q ? head : head - a.num_qo_heads;
    const bool live = lane < kLanes;

    const uint32_t *src = reinterpret_cast<const uint32_t *>(
        is_q ? a.q + ((int64_t)b * a.num_qo_heads + h) * D
             : a.k_new + ((int64_t)b * a.num_kv_heads + h) * D);
    const uint32_t *wsrc = reinterpret_cast<const uint32_t *>(is_q ? a.q_w : a.k_w);
    const uint32_t xw = live ? src[lane] : 0u;
    const uint32_t ww = live ? wsrc[lane] : 0u;
    const float x0 = bf16_to_float(xw & 0xFFFFu), x1 = bf16_to_float(xw >> 16);

    // RMSNorm: the row's sum of squares over the wave
    float ss = x0 * x0 + x1 * x1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        ss += __shfl_xor(ss, o, 64);
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
    const float y0 = x0 * inv * bf16_to_float(ww & 0xFFFFu);
    const float y1 = x1 * inv * bf16_to_float(ww >> 16);

    // rotation partner: the lane holding the elements D/2 away
    const float p0 = __shfl_xor(y0, D / 4, 64);
    const float p1 = __shfl_xor(y1, D / 4, 64);
    const bool upper = lane >= D / 4;   // holds elements of the second half
    const double pos = (double)a.positions[(int64_t)b * a.pos_stride];
    float z[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = (2 * lane + j) % (D / 2);   // pair index of the element
        double pp = pos;   // the position this pair follows
        if constexpr (MR) {
            const int q4 = i >> 4;
            const uint32_t word = q4 == 0   ? a.axis_bits[0]
                                  : q4 == 1 ? a.axis_bits[1]
                                  : q4 == 2 ? a.axis_bits[2]
                                            : a.axis_bits[3];
            const int ax = (int)((word >> (2 * (i & 15))) & 3u);
            pp = (double)a.positions[(int64_t)b * 3 + ax];
        }
        const double turns = pp * a.turns[i];
        const float ang = (float)(turns - rint(turns)) * 6.2831853071795865f;
        float s, c;
        sincosf(ang, &s, &c);
        const float y = j == 0 ? y0 : y1;
        const float p = j == 0 ? p0 : p1;
        z[j] = upper ? y * c + p * s : y * c - p * s;
    }
    const uint32_t out = float_to_bf16(z[0]) | (float_to_bf16(z[1]) << 16);

    if (is_q) {
        if (live)
            reinterpret_cast<uint32_t *>(a.q_out + ((int64_t)b * a.num_qo_heads + h) * D)[lane] =
                out;
        return;
    }
    // KV write: the slot the append fills (entries with a malformed table row
    // write nothing, as the append does)
    const int end = a.indptr[b + 1];
    if (end - a.indptr[b] < 1)
        return;
    const int page = a.indices[end - 1];
    const int slot = a.last_len[b] - 1;
    if (page < 0 || page >= a.num_pages || slot < 0 || slot >= a.page_size)
        return;
    uint16_t *dst = a.cache + (int64_t)page * a.page_stride + (int64_t)slot * a.row_elems +
                    (int64_t)h * D;
    if (live) {
        reinterpret_cast<uint32_t *>(dst)[lane] = out;
        const uint32_t *vs = reinterpret_cast<const uint32_t *>(
            a.v_new + ((int64_t)b * a.num_kv_heads + h) * D);
        reinterpret_cast<uint32_t *>(dst + a.half_stride)[lane] = vs[lane];
    }
}

}  // namespace

bool norm_rope_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_norm_rope(const NormRopeArgs &a, hipStream_t stream) {
    NormRopeArgs args = a;
    void *params[] = {&args};
    const int64_t waves = (int64_t)a.batch * (a.num_qo_heads + a.num_kv_heads);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const void *k = nullptr;
    const bool mr = a.pos_stride == 3;
    if (a.head_dim == 128)
        k = mr ? reinterpret_cast<const void *>(&norm_rope_kernel<128, true>)
               : reinterpret_cast<const void *>(&norm_rope_kernel<128, false>);
    else if (a.head_dim == 64)
        k = mr ? reinterpret_cast<const void *>(&norm_rope_kernel<64, true>)
               : reinterpret_cast<const void *>(&norm_rope_kernel<64, false>);
    else
        return hipErrorInvalidValue;
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), params, 0, stream);
}

}  // namespace pkv
