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
// chunks, each lane owning D/64 dims so a chunk's partial is one coalesced load
// per wave; the four wave sums are added in a fixed order.  Each wave's first
// four partial sums are loaded before the (m, l) pairs, since they do not
// depend on the weights (steps by graph replay, 4-token verify 38.6 -> 38.0 us,
// head_dim-256 layers 478.6 -> 476.9 us for 10; same sums in the same order).  With an output gate
// the result is multiplied by sigmoid(gate) before rounding.
#include "da_internal.h"

#include <math.h>

namespace da {

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxChunks = 2048;  // whole weight table in LDS

template <bool F16, int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const int32_t *__restrict__ seq_pos,
                                                                         int32_t batch, AttnParams p, uint16_t *out) {
    const int sp_first = first_seq_pos(seq_pos, batch, threadIdx.x & 63);
    constexpr int NV = D / 64;  // dims per lane
    __shared__ float wts[kCombineMaxChunks];
    __shared__ float red[4][D];
    __shared__ float wmax[4], wsum[4];

    const int r = blockIdx.x % p.rows;
    const int bh = blockIdx.x / p.rows;
    const int b = bh / p.n_kv_heads;
    const int h = bh - b * p.n_kv_heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t o_off = out_row_off(p, b, h, r) + NV * lane;
    const int T = p.fixed_chunk > 0 ? p.fixed_chunk : balanced_chunk_wave(p, seq_pos, batch, sp_first, lane);
    const SeqChunks sc = seq_chunks_at(p, b < 64 ? __builtin_amdgcn_readlane(sp_first, b) : seq_pos[b], T);
    if (sc.n == 0) {  // seq_pos breaks the contract: flag the rows with NaN
        if (wave == 0) {
            const uint16_t nan16 = F16 ? 0x7e00u : 0x7fc0u;
#pragma unroll
            for (int k = 0; k < NV; ++k) out[o_off + k] = nan16;
        }
        return;
    }
    const int n_live = sc.n;
    const size_t cstride_ml = (size_t)p.rows * 2;
    const size_t cstride_acc = (size_t)p.rows * D;
    const float *ml = p.ws_ml + ((size_t)bh * p.n_chunks * p.rows + r) * 2;
    const float *acc = p.ws_acc + ((size_t)bh * p.n_chunks * p.rows + r) * D + NV * lane;

    auto ld = [&](int c, float (&v)[NV]) {
        if constexpr (NV == 2) {
            const float2 x = *reinterpret_cast<const float2 *>(acc + (size_t)c * cstride_acc);
            v[0] = x.x;
            v[1] = x.y;
        } else {
            const float4 x = *reinterpret_cast<const float4 *>(acc + (size_t)c * cstride_acc);
            v[0] = x.x;
            v[1] = x.y;
            v[2] = x.z;
            v[3] = x.w;
        }
    };
    // The partial sums of this wave's first four chunks (w, w + 4, w + 8, w + 12)
    // do not depend on the weights: issued now, they arrive with the (m, l) pairs.
    float v0[4][NV];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (wave + 4 * u < n_live) {
            ld(wave + 4 * u, v0[u]);
        } else {
#pragma unroll
            for (int k = 0; k < NV; ++k) v0[u][k] = 0.f;
        }
    }

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
    float a[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) a[k] = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (wave + 4 * u < n_live) {
#pragma unroll
            for (int k = 0; k < NV; ++k) a[k] = fmaf(wts[wave + 4 * u], v0[u][k], a[k]);
        }
    int c = wave + 16;
    for (; c + 12 < n_live; c += 16) {  // four loads in flight per lane
        float v[4][NV];
#pragma unroll
        for (int u = 0; u < 4; ++u) ld(c + 4 * u, v[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < NV; ++k) a[k] = fmaf(wts[c + 4 * u], v[u][k], a[k]);
    }
    for (; c < n_live; c += 4) {
        float v[NV];
        ld(c, v);
#pragma unroll
        for (int k = 0; k < NV; ++k) a[k] = fmaf(wts[c], v[k], a[k]);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) red[wave][NV * lane + k] = a[k];
    __syncthreads();
    if (wave == 0) {
        float o[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int d = NV * lane + k;
            o[k] = ((red[0][d] + red[1][d]) + (red[2][d] + red[3][d])) / L;
        }
        store_out<F16, NV>(p, out, o_off, o);
    }
}

hipError_t launch_attn_combine(const AttnParams &p, bool fp16, void *out, hipStream_t s) {
    const int grid = p.batch * p.n_kv_heads * p.rows;
    uint16_t *o = (uint16_t *)out;
    if (p.head_dim == 256) {
        if (fp16)
            hipLaunchKernelGGL((attn_combine_kernel<true, 256>), dim3(grid), dim3(kCombineThreads), 0, s, p.seq_pos, p.batch, p, o);
        else
            hipLaunchKernelGGL((attn_combine_kernel<false, 256>), dim3(grid), dim3(kCombineThreads), 0, s, p.seq_pos, p.batch, p, o);
    } else {
        if (fp16)
            hipLaunchKernelGGL((attn_combine_kernel<true, 128>), dim3(grid), dim3(kCombineThreads), 0, s, p.seq_pos, p.batch, p, o);
        else
            hipLaunchKernelGGL((attn_combine_kernel<false, 128>), dim3(grid), dim3(kCombineThreads), 0, s, p.seq_pos, p.batch, p, o);
    }
    return hipGetLastError();
}

}  // namespace da
