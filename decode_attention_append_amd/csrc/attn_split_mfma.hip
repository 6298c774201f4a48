// Split-context attention partials on the matrix cores, for problems with 16
// to 32 query rows per KV head (e.g. a 4-token speculative verify with 8 query
// heads per KV head).  With that many rows sharing each key, Q K^T and P V
// are real small matrix products, so they run as bf16/fp16 MFMA with fp32
// accumulation ("Architecture Diagram - Qwen3-30B-A3B", paged attention: fp16
// in, fp32 accumulate; "Attention Computation" for what is computed).
//
// Same contract as the vector-ALU kernel: per (sequence b, KV head h, chunk c)
// and query row r, (m, l, acc) with scores in log2 units, written to the
// workspace for the combine kernel.
//
// Mapping on gfx950 (wave64, v_mfma_f32_32x32x16_{bf16,f16}):
//  - a workgroup of 4 waves owns one (b, h, chunk); wave w takes 32-key tiles
//    w, w+4, ...
//  - scores are produced transposed, S^T[key][row] = K q^T, so a lane ends up
//    holding 16 scores of ONE query row (row = lane % 32).  The row's running
//    max/sum and its rescale factor then live in that lane, and the scores
//    feed the P V product as its B operand without leaving registers;
//  - the output is produced transposed too, O^T[dim][row] = V^T P^T.  V^T's
//    A operand needs 8 keys of one dim per lane: each lane loads 8 bytes (four
//    dims) of each of its 8 keys and regroups 16-bit halves with v_perm, so
//    MFMA o (0..3) covers dims 4*i + o;
//  - the running max uses the standard online rescale, applied only when some
//    row's max grew;
//  - P is rounded to the input's 16-bit type for the P V product, and the
//    fp32 sum l adds those same rounded weights, so the output is an exact
//    convex combination of the value rows up to fp32 rounding.
//  - one MFMA applies a value row to all 32 query rows at once, so a later
//    draft token's value row meets the earlier draft tokens' rows with weight
//    exactly 0: finite values contribute nothing, as the mask requires, but a
//    non-finite value there (inf/NaN input) would reach them as 0 * inf.  Rows
//    past the context are never read into a product.
#include "da_internal.h"

#include <math.h>

namespace da {

template <bool F16>
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
    return (uint32_t)round16<F16>(lo) | ((uint32_t)round16<F16>(hi) << 16);
}

constexpr int kObufStride = kHeadDim + 1;  // pad: lanes of one dim hit distinct banks

template <bool F16>
__global__ __launch_bounds__(256) void attn_split_mfma_kernel(AttnParams p) {
    __shared__ float obuf[2 * 32 * kObufStride];
    __shared__ float wave_m[4][32], wave_l[4][32];

    const int n_chunks = p.n_chunks;
    const int c = blockIdx.x % n_chunks;
    const int bh = blockIdx.x / n_chunks;
    const int b = bh / p.n_kv_heads;
    const int h = bh - b * p.n_kv_heads;
    const int sp = p.seq_pos[b];
    if (sp < 0 || sp > p.max_seq - p.q_len) return;
    const int ctx = sp + p.q_len;
    const int t0 = c * p.chunk;
    if (t0 >= ctx) return;
    const int n_tok = min(p.chunk, ctx - t0);
    const int last = n_tok - 1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

    // B operand of S^T = K q^T: lane holds q[row l32][dims 16s + 8hf .. +8), s = 0..7
    u32x4_t qop[8];
    int vis_row = 0;  // exclusive local key limit of row l32
    if (l32 < p.rows) {
        const int i = l32 / p.group, g = l32 - i * p.group;
        const uint8_t *qp =
            p.q + (((size_t)b * p.q_len + i) * p.n_q_heads + (size_t)h * p.group + g) * kRowBytes + 16 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) qop[s] = ld16(qp + 32 * s);
        vis_row = min(sp + i + 1 - t0, n_tok);
    } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) qop[s] = u32x4_t{0u, 0u, 0u, 0u};
    }

    const size_t head_off = ((size_t)bh * p.max_seq + t0) * kRowBytes;
    const uint8_t *kb = p.k_cache + head_off;
    const uint8_t *vb = p.v_cache + head_off;

    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t oacc[4];
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[o][v] = 0.f;

    const int n_tile = (n_tok + 31) >> 5;
    for (int tt = wave; tt < n_tile; tt += 4) {
        const int tb = tt * 32;
        // A operand of S^T: key tb + l32, dims 16s + 8hf .. +8
        u32x4_t kop[8];
        const uint8_t *kr = kb + (size_t)min(tb + l32, last) * kRowBytes + 16 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) kop[s] = ld16(kr + 32 * s);
        // V rows for the P V product: key-block kb2 (16 keys), slot u of this half:
        // key 16*kb2 + 8*(u/4) + 4*hf + u%4, dims 4*l32 .. 4*l32+3
        u32x2_t vx[2][8];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int key = tb + 16 * kb2 + 8 * (u >> 2) + 4 * hf + (u & 3);
                vx[kb2][u] = ld8(vb + (size_t)min(key, last) * kRowBytes + 8 * l32);
            }

        f32x16_t st;
#pragma unroll
        for (int v = 0; v < 16; ++v) st[v] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) st = mfma32<F16>(kop[s], qop[s], st);

        // lane holds row l32's scores for keys tb + 8*(v/4) + 4*hf + v%4
        float s2[16];
        float mt = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = tb + 8 * (v >> 2) + 4 * hf + (v & 3);
            s2[v] = key < vis_row ? st[v] * p.scale_log2 : -INFINITY;
            mt = fmaxf(mt, s2[v]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
        float pv[16];
        float psum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            // the weight as the P V product will see it, so that l sums exactly
            // the weights applied to the value rows
            pv[v] = (m_new == -INFINITY) ? 0.f : round_trip16<F16>(exp2_fast(s2[v] - m_new));
            psum += pv[v];
        }
        if (__any(m_new != m_run)) {
#pragma unroll
            for (int o = 0; o < 4; ++o)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[o][v] *= alpha;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // Keys past the context were loaded as copies of the last row; their weight
        // is zero for every row, and zeroing their value rows keeps a non-finite
        // last row from reaching the others as 0 * inf.
        const bool padded = tb + 31 > last;

#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            u32x4_t pop;
#pragma unroll
            for (int j = 0; j < 4; ++j) pop[j] = pack16<F16>(pv[8 * kb2 + 2 * j], pv[8 * kb2 + 2 * j + 1]);
            if (padded) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int key = tb + 16 * kb2 + 8 * (u >> 2) + 4 * hf + (u & 3);
                    if (key > last) vx[kb2][u] = u32x2_t{0u, 0u};
                }
            }
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const int word = o >> 1;
                const uint32_t sel = (o & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t vop;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vop[j] = __builtin_amdgcn_perm(vx[kb2][2 * j + 1][word], vx[kb2][2 * j][word], sel);
                oacc[o] = mfma32<F16>(vop, pop, oacc[o]);
            }
        }
    }

    // ---- merge the four waves' (m, l, O) in a fixed order ------------------------
    // Waves 0 and 1 store their rescaled O^T into two LDS slices, waves 2 and 3
    // then add theirs into slice 0 and 1 respectively, and the write-out sums the
    // slices: (w0 + w2) + (w1 + w3), the same order on every run.
    l_run += __shfl_xor(l_run, 32);
    if (hf == 0) {
        wave_m[wave][l32] = m_run;
        wave_l[wave][l32] = l_run;
    }
    __syncthreads();
    const float m_fin = fmaxf(fmaxf(wave_m[0][l32], wave_m[1][l32]), fmaxf(wave_m[2][l32], wave_m[3][l32]));
    const float f = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_fin);
    float *slice = obuf + (wave & 1) * (32 * kObufStride);
    if (wave < 2) {
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                slice[l32 * kObufStride + 4 * (8 * (v >> 2) + 4 * hf + (v & 3)) + o] = oacc[o][v] * f;
    }
    __syncthreads();
    if (wave >= 2) {
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                slice[l32 * kObufStride + 4 * (8 * (v >> 2) + 4 * hf + (v & 3)) + o] += oacc[o][v] * f;
    }
    __syncthreads();

    const size_t part = (size_t)bh * n_chunks + c;
    float *wa = p.ws_acc + part * p.rows * kHeadDim;
    for (int idx = tid; idx < p.rows * kHeadDim; idx += 256) {
        const int r = idx >> 7, d = idx & (kHeadDim - 1);
        wa[idx] = obuf[r * kObufStride + d] + obuf[32 * kObufStride + r * kObufStride + d];
    }
    if (tid < p.rows) {
        const int r = tid;
        const float mf = fmaxf(fmaxf(wave_m[0][r], wave_m[1][r]), fmaxf(wave_m[2][r], wave_m[3][r]));
        float lf = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (wave_m[w][r] != -INFINITY) lf += exp2_fast(wave_m[w][r] - mf) * wave_l[w][r];
        p.ws_ml[(part * p.rows + r) * 2 + 0] = mf;
        p.ws_ml[(part * p.rows + r) * 2 + 1] = lf;
    }
}

hipError_t launch_attn_mfma(const AttnParams &p, bool fp16, hipStream_t s) {
    const int grid = p.batch * p.n_kv_heads * p.n_chunks;
    if (fp16)
        hipLaunchKernelGGL(attn_split_mfma_kernel<true>, dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(attn_split_mfma_kernel<false>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace da
