// Split-context attention partials on the matrix cores.  With many query
// rows sharing each key (e.g. a 4-token speculative verify with 8 query heads
// per KV head: 32 rows), Q K^T and P V are real small matrix products, so they
// run as bf16/fp16 MFMA with fp32 accumulation ("Architecture Diagram -
// Qwen3-30B-A3B", paged attention: fp16 in, fp32 accumulate; "Attention
// Computation" for what is computed).
//
// Same contract as the vector-ALU kernel: per (sequence b, KV head h, chunk c)
// and query row r, (m, l, acc) with scores in log2 units, written to the
// workspace for the combine kernel.
//
// Mapping on gfx950 (wave64, v_mfma_f32_16x16x32_{bf16,f16}; RB blocks of 16
// query rows, RB = 1 or 2):
//  - a workgroup of 4 waves owns one (b, h, chunk); wave w takes 32-key tiles
//    w, w+4, ... and loads tile t+4 while it computes tile t;
//  - scores come out transposed, S^T[key][row] = K q^T, so lane l holds 8
//    scores of ONE query row (row = l % 16) and that row's running max, sum
//    and rescale factor stay in the lane; the scores then feed P V as its B
//    operand without leaving registers;
//  - the output is transposed too, O^T[dim][row] = V^T P^T.  V^T's A operand
//    wants 8 keys of one dim per lane: lane (i, q) loads 16 bytes (dims
//    8i..8i+7) of each of its 8 keys -- four whole rows per load instruction --
//    and v_perm regroups 16-bit halves, so MFMA o (0..7) covers dims 8i + o;
//  - P is rounded to the input's 16-bit type for P V, and the fp32 sum l adds
//    those same rounded weights, so the result is a convex combination of the
//    value rows up to fp32 rounding;
//  - one MFMA applies a value row to 16 query rows at once, so a later draft
//    token's value row meets earlier draft tokens' rows with weight exactly 0:
//    finite values contribute nothing, as the mask requires, but an inf/NaN
//    value there would reach them as 0 * inf.  Slots past the context are
//    never read into a product.
#include "da_internal.h"

#include <math.h>

namespace da {

template <bool F16>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
    return (uint32_t)round16<F16>(lo) | ((uint32_t)round16<F16>(hi) << 16);
}

constexpr int kObufStride = kHeadDim + 4;

// Key of slot u (0..7) of lane group q inside a 32-key tile, in the order the
// P V product consumes them: keys 4q..4q+3, then 16+4q..16+4q+3.
__device__ __forceinline__ int pv_key(int q, int u) { return (u < 4 ? 4 * q + u : 16 + 4 * q + (u - 4)); }

struct Tile {
    u32x4_t k[2][4];  // K: key block kb (16 keys), k-step s (32 dims)
    u32x4_t v[8];     // V: slot u, dims 8i .. 8i+7
};

__device__ __forceinline__ void load_tile(Tile &t, const uint8_t *kb, const uint8_t *vb, int tb, int last,
                                          int l16, int q) {
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk) {
        const uint8_t *kr = kb + (size_t)min(tb + 16 * kblk + l16, last) * kRowBytes + 16 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) t.k[kblk][s] = ld16(kr + 64 * s);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) t.v[u] = ld16(vb + (size_t)min(tb + pv_key(q, u), last) * kRowBytes + 16 * l16);
}

template <bool F16, int RB>
__global__ __launch_bounds__(256) void attn_split_mfma_kernel(AttnParams p) {
    __shared__ float obuf[2][16 * RB * kObufStride];
    __shared__ float wave_m[4][16 * RB], wave_l[4][16 * RB];

    const int n_chunks = p.n_chunks;
    int b, h, c;
    SeqChunks sc;
    if (!locate(p, blockIdx.x, b, h, c, sc)) return;  // past the last chunk of the launch
    const int bh = b * p.n_kv_heads + h;
    const int sp = p.seq_pos[b];
    const int ctx = sc.ctx;
    const int t0 = c * sc.len;
    const int n_tok = min(sc.len, ctx - t0);
    const int last = n_tok - 1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q = lane >> 4;

    // B operand of S^T = K q^T: lane holds q[row][dims 64s + 16q .. +16 bytes), s = 0..3
    u32x4_t qop[RB][4];
    int vis[RB];  // exclusive local key limit of this lane's row in each row block
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 16 + l16;
        if (row < p.rows) {
            const int i = row / p.group, g = row - i * p.group;
            const uint8_t *qp =
                p.q + (((size_t)b * p.q_len + i) * p.n_q_heads + (size_t)h * p.group + g) * kRowBytes + 16 * q;
#pragma unroll
            for (int s = 0; s < 4; ++s) qop[rb][s] = ld16(qp + 64 * s);
            vis[rb] = min(sp + i + 1 - t0, n_tok);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) qop[rb][s] = u32x4_t{0u, 0u, 0u, 0u};
            vis[rb] = 0;
        }
    }

    const size_t head_off = ((size_t)bh * p.max_seq + t0) * kRowBytes;
    const uint8_t *kb = p.k_cache + head_off;
    const uint8_t *vb = p.v_cache + head_off;

    float m_run[RB], l_run[RB];
    f32x4_t oacc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
#pragma unroll
        for (int o = 0; o < 8; ++o) oacc[rb][o] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const int n_tile = (n_tok + 31) >> 5;
    Tile cur, nxt;
    load_tile(cur, kb, vb, min(wave, n_tile - 1) * 32, last, l16, q);
    for (int tt = wave; tt < n_tile; tt += 4) {
        const int tb = tt * 32;
        // prefetch the wave's next tile (or re-read this one, already in cache)
        load_tile(nxt, kb, vb, (tt + 4 < n_tile ? tt + 4 : tt) * 32, last, l16, q);

        // zero value rows past the context (copies of the last row) so a
        // non-finite last row cannot reach the other rows as 0 * inf
        if (tb + 31 > last) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (tb + pv_key(q, u) > last) cur.v[u] = u32x4_t{0u, 0u, 0u, 0u};
        }

#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            // S^T for the two 16-key blocks: lane holds keys tb + 16*kblk + 4q + v of row l16
            f32x4_t st[2];
#pragma unroll
            for (int kblk = 0; kblk < 2; ++kblk) {
                st[kblk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) st[kblk] = mfma16<F16>(cur.k[kblk][s], qop[rb][s], st[kblk]);
            }
            float s2[8];
            float mt = -INFINITY;
#pragma unroll
            for (int kblk = 0; kblk < 2; ++kblk)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int key = tb + 16 * kblk + 4 * q + v;
                    const float x = key < vis[rb] ? st[kblk][v] * p.scale_log2 : -INFINITY;
                    s2[4 * kblk + v] = x;
                    mt = fmaxf(mt, x);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run[rb], mt);
            const float alpha = (m_run[rb] == -INFINITY) ? 0.f : exp2_fast(m_run[rb] - m_new);
            float pv[8];
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                pv[u] = (m_new == -INFINITY) ? 0.f : round_trip16<F16>(exp2_fast(s2[u] - m_new));
                psum += pv[u];
            }
            if (__any(m_new != m_run[rb])) {
#pragma unroll
                for (int o = 0; o < 8; ++o) oacc[rb][o] *= alpha;
            }
            l_run[rb] = l_run[rb] * alpha + psum;
            m_run[rb] = m_new;

            // B operand of O^T: P^T, slot u <-> key pv_key(q, u) = s2 index u
            u32x4_t pop;
#pragma unroll
            for (int j = 0; j < 4; ++j) pop[j] = pack16<F16>(pv[2 * j], pv[2 * j + 1]);
#pragma unroll
            for (int o = 0; o < 8; ++o) {
                const int word = o >> 1;
                const uint32_t sel = (o & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t vop;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vop[j] = __builtin_amdgcn_perm(cur.v[2 * j + 1][word], cur.v[2 * j][word], sel);
                oacc[rb][o] = mfma16<F16>(vop, pop, oacc[rb][o]);
            }
        }
        cur = nxt;
    }

    // ---- merge the four waves' (m, l, O) in a fixed order ------------------------
    // Waves 0 and 1 store their rescaled O^T into two LDS slices, waves 2 and 3
    // add theirs into slice 0 and 1, and the write-out sums the two slices:
    // (w0 + w2) + (w1 + w3), the same order on every run.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        l_run[rb] += __shfl_xor(l_run[rb], 16);
        l_run[rb] += __shfl_xor(l_run[rb], 32);
        if (q == 0) {
            wave_m[wave][rb * 16 + l16] = m_run[rb];
            wave_l[wave][rb * 16 + l16] = l_run[rb];
        }
    }
    __syncthreads();
    float f[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 16 + l16;
        const float m_fin =
            fmaxf(fmaxf(wave_m[0][row], wave_m[1][row]), fmaxf(wave_m[2][row], wave_m[3][row]));
        f[rb] = (m_run[rb] == -INFINITY) ? 0.f : exp2_fast(m_run[rb] - m_fin);
    }
    float *slice = obuf[wave & 1];
    if (wave < 2) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int o = 0; o < 8; ++o)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    slice[(rb * 16 + l16) * kObufStride + 8 * (4 * q + v) + o] = oacc[rb][o][v] * f[rb];
    }
    __syncthreads();
    if (wave >= 2) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int o = 0; o < 8; ++o)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    slice[(rb * 16 + l16) * kObufStride + 8 * (4 * q + v) + o] += oacc[rb][o][v] * f[rb];
    }
    __syncthreads();

    const size_t part = (size_t)bh * n_chunks + c;
    float *wa = p.ws_acc + part * p.rows * kHeadDim;
    for (int idx = tid; idx < p.rows * kHeadDim; idx += 256) {
        const int r = idx >> 7, d = idx & (kHeadDim - 1);
        wa[idx] = obuf[0][r * kObufStride + d] + obuf[1][r * kObufStride + d];
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

template <bool F16>
static hipError_t launch_dtype(const AttnParams &p, int grid, hipStream_t s) {
    if (p.rows <= 16)
        hipLaunchKernelGGL((attn_split_mfma_kernel<F16, 1>), dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((attn_split_mfma_kernel<F16, 2>), dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnParams &p, int grid, bool fp16, hipStream_t s) {
    return fp16 ? launch_dtype<true>(p, grid, s) : launch_dtype<false>(p, grid, s);
}

}  // namespace da
