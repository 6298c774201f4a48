// Combine: the log-sum-exp reduce phase of the 3-phase flash decode
// ("Qwen MoE BringUp", "Architecture Diagram - Qwen3-30B-A3B (Extern Dispatch,
// 75 tok/s)", Paged Attention block).  For each query row, over the live
// chunks c of its sequence (those starting before seq_pos + q_len):
//     M = max_c m_c,  w_c = 2^(m_c - M)  (0 for a chunk the row saw nothing of)
//     out = (sum_c w_c acc_c) / (sum_c w_c l_c)
// rounded to nearest-even into the 16-bit output type.
//
// One wave per (sequence, KV head, query row); each lane owns two dims, so a
// chunk's 512-byte partial is one coalesced load per wave.
#include "da_internal.h"

#include <math.h>

namespace da {

template <bool F16>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnParams p, uint16_t *out) {
    const int r = blockIdx.x % p.rows;
    const int bh = blockIdx.x / p.rows;
    const int b = bh / p.n_kv_heads;
    const int h = bh - b * p.n_kv_heads;
    const int i = r / p.group, g = r - i * p.group;
    const int lane = threadIdx.x;
    uint32_t *o = reinterpret_cast<uint32_t *>(
                      out + (((size_t)b * p.q_len + i) * p.n_q_heads + (size_t)h * p.group + g) * kHeadDim) +
                  lane;
    const int sp = p.seq_pos[b];
    if (sp < 0 || sp > p.max_seq - p.q_len) {  // broken contract: flag the rows with NaN
        const uint32_t nan16 = F16 ? 0x7e00u : 0x7fc0u;
        *o = nan16 | (nan16 << 16);
        return;
    }
    const int n_live = (sp + p.q_len + p.chunk - 1) / p.chunk;
    const size_t cstride_ml = (size_t)p.rows * 2;
    const size_t cstride_acc = (size_t)p.rows * kHeadDim;
    const float *ml = p.ws_ml + ((size_t)bh * p.n_chunks * p.rows + r) * 2;
    const float *acc = p.ws_acc + ((size_t)bh * p.n_chunks * p.rows + r) * kHeadDim + 2 * lane;

    float M = -INFINITY;
    for (int c = 0; c < n_live; ++c) M = fmaxf(M, ml[c * cstride_ml]);
    float L = 0.f, a0 = 0.f, a1 = 0.f;
    for (int c = 0; c < n_live; ++c) {
        const float m = ml[c * cstride_ml];
        const float w = (m == -INFINITY) ? 0.f : exp2_fast(m - M);
        L = fmaf(w, ml[c * cstride_ml + 1], L);
        const float2 v = *reinterpret_cast<const float2 *>(acc + c * cstride_acc);
        a0 = fmaf(w, v.x, a0);
        a1 = fmaf(w, v.y, a1);
    }
    *o = (uint32_t)round16<F16>(a0 / L) | ((uint32_t)round16<F16>(a1 / L) << 16);
}

hipError_t launch_attn_combine(const AttnParams &p, bool fp16, void *out, hipStream_t s) {
    const int grid = p.batch * p.n_kv_heads * p.rows;
    if (fp16)
        hipLaunchKernelGGL(attn_combine_kernel<true>, dim3(grid), dim3(64), 0, s, p, (uint16_t *)out);
    else
        hipLaunchKernelGGL(attn_combine_kernel<false>, dim3(grid), dim3(64), 0, s, p, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace da
