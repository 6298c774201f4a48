// Combine: the log-sum-exp reduce phase of the 3-phase flash decode
// ("Qwen MoE BringUp", "Architecture Diagram - Qwen3-30B-A3B (Extern Dispatch,
// 75 tok/s)", Paged Attention block).  For each query row, over the live
// chunks c of its sequence (those starting before seq_pos + q_len):
//     M = max_c m_c,  w_c = 2^(m_c - M)  (0 for a chunk the row saw nothing of)
//     out = (sum_c w_c acc_c) / (sum_c w_c l_c)
// rounded to nearest-even into the 16-bit output type.
//
// One 256-lane workgroup per (sequence, KV head, query row).  Lane c computes
// chunk c's weight (a block-wide max first), then the four waves split the
// chunks, each lane owning two dims so a chunk's 512-byte partial is one
// coalesced load per wave; the four wave sums are added in a fixed order.
#include "da_internal.h"

#include <math.h>

namespace da {

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxChunks = 2048;  // whole weight table in LDS

template <bool F16>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnParams p, uint16_t *out) {
    __shared__ float wts[kCombineMaxChunks];
    __shared__ float red[4][2 * 64];
    __shared__ float wmax[4], wsum[4];

    const int r = blockIdx.x % p.rows;
    const int bh = blockIdx.x / p.rows;
    const int b = bh / p.n_kv_heads;
    const int h = bh - b * p.n_kv_heads;
    const int i = r / p.group, g = r - i * p.group;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t *o = reinterpret_cast<uint32_t *>(
                      out + (((size_t)b * p.q_len + i) * p.n_q_heads + (size_t)h * p.group + g) * kHeadDim) +
                  lane;
    const SeqChunks sc = seq_chunks(p, b, p.fixed_chunk > 0 ? p.fixed_chunk : balanced_chunk(p));
    if (sc.n == 0) {  // seq_pos breaks the contract: flag the rows with NaN
        if (wave == 0) {
            const uint32_t nan16 = F16 ? 0x7e00u : 0x7fc0u;
            *o = nan16 | (nan16 << 16);
        }
        return;
    }
    const int n_live = sc.n;
    const size_t cstride_ml = (size_t)p.rows * 2;
    const size_t cstride_acc = (size_t)p.rows * kHeadDim;
    const float *ml = p.ws_ml + ((size_t)bh * p.n_chunks * p.rows + r) * 2;
    const float *acc = p.ws_acc + ((size_t)bh * p.n_chunks * p.rows + r) * kHeadDim + 2 * lane;

    // M = max over live chunks
    float m = -INFINITY;
    for (int c = tid; c < n_live; c += kCombineThreads) m = fmaxf(m, ml[c * cstride_ml]);
    m = wave_max(m);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

    // chunk weights and L = sum_c w_c l_c
    float l = 0.f;
    for (int c = tid; c < n_live; c += kCombineThreads) {
        const float mc = ml[c * cstride_ml];
        const float w = (mc == -INFINITY) ? 0.f : exp2_fast(mc - M);
        wts[c] = w;
        l = fmaf(w, ml[c * cstride_ml + 1], l);
    }
    l = wave_sum(l);
    if (lane == 0) wsum[wave] = l;
    __syncthreads();
    const float L = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);

    // weighted sum of the partial V sums: wave w takes chunks w, w+4, ...
    float a0 = 0.f, a1 = 0.f;
    int c = wave;
    for (; c + 12 < n_live; c += 16) {  // four loads in flight per lane
        const float2 v0 = *reinterpret_cast<const float2 *>(acc + (size_t)c * cstride_acc);
        const float2 v1 = *reinterpret_cast<const float2 *>(acc + (size_t)(c + 4) * cstride_acc);
        const float2 v2 = *reinterpret_cast<const float2 *>(acc + (size_t)(c + 8) * cstride_acc);
        const float2 v3 = *reinterpret_cast<const float2 *>(acc + (size_t)(c + 12) * cstride_acc);
        a0 = fmaf(wts[c], v0.x, a0);
        a1 = fmaf(wts[c], v0.y, a1);
        a0 = fmaf(wts[c + 4], v1.x, a0);
        a1 = fmaf(wts[c + 4], v1.y, a1);
        a0 = fmaf(wts[c + 8], v2.x, a0);
        a1 = fmaf(wts[c + 8], v2.y, a1);
        a0 = fmaf(wts[c + 12], v3.x, a0);
        a1 = fmaf(wts[c + 12], v3.y, a1);
    }
    for (; c < n_live; c += 4) {
        const float2 v = *reinterpret_cast<const float2 *>(acc + (size_t)c * cstride_acc);
        a0 = fmaf(wts[c], v.x, a0);
        a1 = fmaf(wts[c], v.y, a1);
    }
    red[wave][2 * lane] = a0;
    red[wave][2 * lane + 1] = a1;
    __syncthreads();
    if (wave == 0) {
        const float s0 = (red[0][2 * lane] + red[1][2 * lane]) + (red[2][2 * lane] + red[3][2 * lane]);
        const float s1 =
            (red[0][2 * lane + 1] + red[1][2 * lane + 1]) + (red[2][2 * lane + 1] + red[3][2 * lane + 1]);
        *o = (uint32_t)round16<F16>(s0 / L) | ((uint32_t)round16<F16>(s1 / L) << 16);
    }
}

hipError_t launch_attn_combine(const AttnParams &p, bool fp16, void *out, hipStream_t s) {
    const int grid = p.batch * p.n_kv_heads * p.rows;
    if (fp16)
        hipLaunchKernelGGL(attn_combine_kernel<true>, dim3(grid), dim3(kCombineThreads), 0, s, p,
                           (uint16_t *)out);
    else
        hipLaunchKernelGGL(attn_combine_kernel<false>, dim3(grid), dim3(kCombineThreads), 0, s, p,
                           (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace da
