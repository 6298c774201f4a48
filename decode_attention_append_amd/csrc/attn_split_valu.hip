// Split-context attention partials on the vector ALU, for problems with at
// most 16 query rows per KV head (Hq/Hkv * q_len; chosen automatically below 8).
//
// What is computed ("Qwen MoE BringUp", Per-Layer IR Patterns, "Attention
// Computation", split as in the split-KV phase of the 3-phase flash decode in
// "Architecture Diagram - Qwen3-30B-A3B (Extern Dispatch, 75 tok/s)"): for one
// (sequence b, KV head h, chunk c of the context) and each query row r of
// that KV head,
//     s_j  = (q_r . k_j) * scale * log2(e)          visible keys j of the chunk
//     m    = max_j s_j,  p_j = 2^(s_j - m),  l = sum_j p_j
//     acc  = sum_j p_j v_j                          (fp32 throughout)
// and (m, l, acc) is written to the workspace.  The combine kernel merges the
// chunks.  A key j is visible to query token i iff j <= seq_pos + i.
//
// Mapping on gfx950: one workgroup of 4 waves per (b, h, chunk), serving every
// query row of KV head h, so each K/V byte is read once; chunks of up to 2048
// keys (1024 at 16 rows), or of up to 8192 (one workgroup per compute unit)
// for up to 2 rows per KV head and at least 128 (b, h) pairs.  Sixteen lanes hold
// one 256-byte row (16 bytes each): a wave's 128-bit load covers four
// consecutive keys, 1 KiB contiguous.  Q.K partial dots use the packed
// dot2 (bf16/fp16 pair -> fp32) instruction, then a 16-lane DPP butterfly.
// The chunk's scores go to LDS; the chunk is two-pass (all scores, then the
// maximum, then P.V), so no running rescale is needed inside a chunk.  Each
// wave streams its 16-key slabs through two register buffers in turn, so the
// next slab is in flight while the current one is computed.
#include "da_internal.h"

#include <math.h>

namespace da {

// Sum of f(0) .. f(NW-1) as a fixed pairwise tree: ((0 + 1) + (2 + 3)) + ...
template <int NW, typename F>
__device__ __forceinline__ float tree_sum(F &&f) {
    float v[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) v[w] = f(w);
#pragma unroll
    for (int st = 1; st < NW; st *= 2)
#pragma unroll
        for (int w = 0; w < NW; w += 2 * st) v[w] = v[w] + v[w + st];
    return v[0];
}

// The one-launch step's merge of every query row of (b, h) over its n chunks,
// by the whole workgroup of NW waves.  With at most 16 chunks, or 4 rows or
// more, each wave merges whole rows (r = wave, wave + NW, ...); otherwise the
// waves split each row's chunks into NW consecutive ranges and their merge
// states are combined in LDS in a fixed order.  `red` is LDS of at least
// NW * 128 + 2 * NW floats.  Uniform across the workgroup (it has barriers).
template <bool F16, int NW>
__device__ void merge_rows_block(const AttnParams &p, float *red, int bh, int b, int h, int n, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    if (n <= 16 || p.rows >= 4) {
        for (int r = wave; r < p.rows; r += NW) merge_row_wave<F16, kHeadDim>(p, p.out, bh, b, h, r, n, lane);
        return;
    }
    float *wm = red + NW * kHeadDim, *wl = wm + NW;
    const int c_lo = wave * n / NW, c_hi = (wave + 1) * n / NW;
    for (int r = 0; r < p.rows; ++r) {
        const MergeState<kHeadDim> s = merge_range<kHeadDim>(p, (size_t)bh * p.n_chunks * p.rows + r, c_lo, c_hi, lane);
        red[wave * kHeadDim + 2 * lane] = s.a[0];
        red[wave * kHeadDim + 2 * lane + 1] = s.a[1];
        if (lane == 0) {
            wm[wave] = s.m;
            wl[wave] = s.l;
        }
        __syncthreads();
        if (wave == 0) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w]);
            float f[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) f[w] = wm[w] == -INFINITY ? 0.f : exp2_fast(wm[w] - M);
            const float L = tree_sum<NW>([&](int w) { return f[w] * wl[w]; });
            float o[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int d = 2 * lane + k;
                o[k] = tree_sum<NW>([&](int w) { return f[w] * red[w * kHeadDim + d]; }) / L;
            }
            store_out<F16, 2>(p, p.out, out_row_off(p, b, h, r) + 2 * lane, o);
        }
        __syncthreads();
    }
}

// The one-launch step's append and merge, and the rotary embedding of q, are
// compiled for up to 8 rows; the 16-row kernel (only used when the vector-ALU
// kernel is forced) has no registers to spare for them: the launcher runs that
// step as three launches and refuses it a rotary table.
constexpr int kValuOneLaunchRows = 8;

// Waves per workgroup.
constexpr int kValuWaves = 4;

// ROPE: the problem has a rotary table (a separate instantiation, so that the
// rotation's registers never weigh on the kernel without one).
template <bool F16, int RP, bool ROPE>
__global__ __launch_bounds__(64 * kValuWaves) void attn_split_valu_kernel(const int32_t *__restrict__ seq_pos, int32_t batch, AttnParams p) {
    constexpr int NW = kValuWaves;
    const int sp_first = first_seq_pos(seq_pos, batch, threadIdx.x & 63);
    constexpr bool kOneLaunch = RP <= kValuOneLaunchRows;
    static_assert(!ROPE || kOneLaunch, "the rotary embedding is compiled up to 8 rows");
    extern __shared__ float lds[];  // scores [chunk][RP], later the wave sums [NW][RP][128]
    __shared__ float row_m[RP], row_l[RP];

    const int n_chunks = p.n_chunks;
    int b, h, c;
    SeqChunks sc;
    int item = blockIdx.x;
    int sp;
    if (!locate_wave(p, seq_pos, batch, sp_first, item, b, h, c, sc, sp, threadIdx.x & 63)) {  // past the last chunk of the launch
        if (kOneLaunch && p.out && item < p.batch && !seq_pos_ok(p, p.seq_pos[item]))
            flag_sequence_nan<F16>(p, item, threadIdx.x, 64 * NW);
        return;
    }
    const int bh = b * p.n_kv_heads + h;
    const int ctx = sc.ctx;
    const int t0 = c * sc.len;
    const int n_tok = min(sc.len, ctx - t0);
    const int n_slab = (n_tok + 15) >> 4;  // 16-key slabs; a wave does one per step

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int gq = lane >> 4;  // which of the 4 keys of a 1 KiB load
    const int cq = lane & 15;  // 16-byte column: dims 8*cq .. 8*cq+7

    // Paged caches: the pool page of every 16-token block of the chunk is read
    // once, at most two entries per thread (a chunk has at most 512 blocks),
    // issued before the query loads and kept in LDS.  A block-table load per
    // slab would be a vector load whose wait also waits for the slabs in flight.
    const int lp0 = t0 / kPageTokens;
    const bool paged = p.layout.block_table != nullptr;
    constexpr int kTabPerThread = kValuLongChunk / kPageTokens / (64 * NW);
    __shared__ int pg_tab[kValuLongChunk / kPageTokens];
    int pg_mine[kTabPerThread];  // checked against the pool when stored, after the query loads are issued
#pragma unroll
    for (int j = 0; j < kTabPerThread; ++j) {
        const int s_ = tid + j * 64 * NW;
        pg_mine[j] = paged && s_ < n_slab ? p.layout.block_table[(size_t)b * p.layout.pages_per_seq + lp0 + s_] : 0;
    }

    // Query rows: r = i * group + g is query token i of query head h*group + g.
    uint32_t qr[RP][4];
    int vis[RP];  // exclusive limit of the visible local key indices of row r
    // Every row's load is issued unconditionally (no branch between them and
    // the first cache loads, so none waits for another): rows past p.rows
    // re-read the last row; their keys are all hidden (vis 0) and nothing of
    // theirs is stored.
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int rr = min(r, p.rows - 1);
        const int i = div_small(rr, p.group), g = rr - i * p.group;
        const uint8_t *qp =
            p.q + (((size_t)b * p.q_len + i) * p.n_q_heads + (size_t)h * p.group + g) * kRowBytes + cq * 16;
        const u32x4_t v = ld16(qp);
        qr[r][0] = v[0];
        qr[r][1] = v[1];
        qr[r][2] = v[2];
        qr[r][3] = v[3];
        vis[r] = r < p.rows ? min(sp + i + 1 - t0, n_tok) : 0;
    }
    if (ROPE) {  // rotary embedding of the query rows at seq_pos + i
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            u32x4_t v = {qr[r][0], qr[r][1], qr[r][2], qr[r][3]};
            rope_row<F16>(v, cq, p.rope_dim, sp + div_small(r, p.group), p.rope_freqs, r < p.rows);
            qr[r][0] = v[0];
            qr[r][1] = v[1];
            qr[r][2] = v[2];
            qr[r][3] = v[3];
        }
    }

    if (paged) {
#pragma unroll
        for (int j = 0; j < kTabPerThread; ++j) {
            const int s_ = tid + j * 64 * NW;
            if (s_ < n_slab) pg_tab[s_] = (unsigned)pg_mine[j] < (unsigned)p.layout.n_pages ? pg_mine[j] : -1;
        }
        __syncthreads();
    }

    const int last = n_tok - 1;  // loads past the context re-read the last row (masked)
    // Cache addresses of this lane's 16-byte column (contiguous or paged caches).
    // Chunks start on multiples of 32 keys, so slab s (keys t0 + 16 s ..) is one
    // 16-token block: one page of a paged cache.  A block-table entry outside
    // the pool (-1) reads page 0 and drops writes.
    auto block_off = [&](int s_) {
        if (paged) {
            const int pg = pg_tab[s_];
            return ((size_t)(pg < 0 ? 0 : pg) * p.n_kv_heads + h) * kPageTokens * kRowBytes;
        }
        return kv_block_off(p.layout, b, h, p.n_kv_heads, p.max_seq, lp0 + s_);
    };
    auto row_off = [&](int t) { return block_off(t >> 4) + (size_t)(t & 15) * kRowBytes + cq * 16; };
    auto slab_ptr = [&](const uint8_t *cache, int s_) { return cache + block_off(s_) + cq * 16; };
    auto row_ptr = [&](const uint8_t *cache, int t) { return cache + row_off(t); };
    auto row_writable = [&](int t) { return !paged || pg_tab[t >> 4] >= 0; };

    // Slab loads: four 128-bit loads per lane cover 16 keys (1 KiB each).
    //  - Fast slabs (full, and below this step's new rows) use one base address
    //    and immediate offsets; a wave streams them through two register buffers
    //    used in turn, with no copy between iterations, so it waits only for the
    //    older slab.
    //  - The rest, at most the chunk's last couple of slabs, go row by row: keys
    //    past the chunk re-read row `last` (masked later), and in the one-launch
    //    step the new rows (local keys from new_first on) are read from k_new /
    //    v_new, rotated in the K pass when there is a rotary table, and stored
    //    into the cache (no other chunk touches them).
    const bool fused_append = kOneLaunch && p.k_new != nullptr;
    const int new_first = fused_append ? sp - t0 : n_tok;
    const int n_fast = min(n_tok >> 4, max(new_first, 0) >> 4);
    const size_t new_stride = (size_t)p.n_kv_heads * kRowBytes;
    const size_t new_off = ((size_t)b * p.q_len * p.n_kv_heads + h) * kRowBytes + cq * 16;
    auto load_fast = [&](u32x4_t (&buf)[4], const uint8_t *base, int s_) {
        const uint8_t *r0 = slab_ptr(base, s_) + (size_t)gq * kRowBytes;
#pragma unroll
        for (int u = 0; u < 4; ++u) buf[u] = ld16_stream(r0 + u * 4 * kRowBytes);
    };
    auto load_rows = [&](u32x4_t (&buf)[4], const uint8_t *base, const uint8_t *nbase, uint8_t *wbase, bool rot,
                         int s_) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = min(s_ * 16 + u * 4 + gq, last);
            buf[u] = ld16(t >= new_first ? nbase + (size_t)(t - new_first) * new_stride : row_ptr(base, t));
        }
        if (ROPE && rot) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = min(s_ * 16 + u * 4 + gq, last);
                rope_row<F16>(buf[u], cq, p.rope_dim, t0 + t, p.rope_freqs, t >= new_first);
            }
        }
        if (fused_append) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = s_ * 16 + u * 4 + gq;
                if (t >= new_first && t <= last && row_writable(t))
                    *reinterpret_cast<u32x4_t *>(wbase + row_off(t)) = buf[u];
            }
        }
    };
    // This wave's slabs are wave, wave + NW, ...
    const int nf = wave < n_fast ? (n_fast - 1 - wave) / NW + 1 : 0;
    const int first_slow = n_fast + (((wave - n_fast) % NW) + NW) % NW;
    // b0 holds the wave's first fast slab when `preloaded` (issued early by the caller).
    auto pass = [&](const uint8_t *base, const uint8_t *nbase, uint8_t *wbase, bool rot, u32x4_t (&b0)[4],
                    bool preloaded, auto &&body) {
        if (nf > 0) {
            u32x4_t b1[4];
            if (!preloaded) load_fast(b0, base, wave);
            int i = 0;
            for (; i + 2 <= nf; i += 2) {
                load_fast(b1, base, wave + (i + 1) * NW);
                body(b0, wave + i * NW);
                load_fast(b0, base, wave + min(i + 2, nf - 1) * NW);
                body(b1, wave + (i + 1) * NW);
            }
            if (i < nf) body(b0, wave + i * NW);
        }
        for (int s_ = first_slow; s_ < n_slab; s_ += NW) {
            u32x4_t b0[4];
            load_rows(b0, base, nbase, wbase, rot, s_);
            body(b0, s_);
        }
    };

    // ---- pass 1: scores of the chunk into LDS ----------------------------------
    const uint8_t *knb = fused_append ? p.k_new + new_off : nullptr;
    const uint8_t *vnb = fused_append ? p.v_new + new_off : nullptr;
    uint8_t *kwb = fused_append ? p.k_cache_w : nullptr;
    uint8_t *vwb = fused_append ? p.v_cache_w : nullptr;
    u32x4_t kb0[4], vb0[4];
    auto score_slab = [&](u32x4_t (&cur)[4], int s_) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tl = s_ * 16 + u * 4 + gq;
            float score[RP];
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                float a = dot2<F16>(qr[r][0], cur[u][0], 0.f);
                a = dot2<F16>(qr[r][1], cur[u][1], a);
                a = dot2<F16>(qr[r][2], cur[u][2], a);
                a = dot2<F16>(qr[r][3], cur[u][3], a);
                score[r] = row16_sum(a);
            }
            if (cq == 0) {
#pragma unroll
                for (int r = 0; r < RP; ++r)
                    lds[tl * RP + r] = tl < vis[r] ? score[r] * p.scale_log2 : -INFINITY;
            }
        }
    };
    pass(p.k_cache, knb, kwb, fused_append, kb0, false, score_slab);
    // The V pass's first slab does not depend on the weights: issue it now, so
    // its latency overlaps the other waves' last K slabs and the softmax.
    if (nf > 0) load_fast(vb0, p.v_cache, wave);
    __syncthreads();

    // ---- chunk maximum and weights p = 2^(s - m), sum l ------------------------
    const int n_pad = n_slab * 16;
    // Both loops over a row's scores take them eight at a time while eight remain,
    // every LDS read of the eight issued before any is used, so a lane waits for
    // one LDS round trip per eight scores instead of one per score (a long chunk's
    // 8192 scores per row are 128 per lane of the row's wave; read one at a time,
    // 16 per lane over 8 waves took about 3 us between the passes); the rest go
    // one at a time, as a short chunk's single score does.  The max and the sum keep the order t = t0, t0 + stride, ... of
    // every lane.
    constexpr int kBatch = 8;
    auto row_max = [&](int r, int t0, int stride) {
        float m = -INFINITY;
        int tb = t0;
        for (; tb + (kBatch - 1) * stride < n_pad; tb += kBatch * stride) {
            float x[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) x[j] = lds[(tb + j * stride) * RP + r];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) m = fmaxf(m, x[j]);
        }
        for (; tb < n_pad; tb += stride) m = fmaxf(m, lds[tb * RP + r]);
        return m;
    };
    // p = 2^(s - m) written over the scores, and their sum
    auto row_exp = [&](int r, int t0, int stride, float m) {
        float l = 0.f;
        auto weigh = [&](int t, float x) {
            const float e = (m == -INFINITY) ? 0.f : exp2_fast(x - m);
            lds[t * RP + r] = e;
            l += e;
        };
        int tb = t0;
        for (; tb + (kBatch - 1) * stride < n_pad; tb += kBatch * stride) {
            float x[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) x[j] = lds[(tb + j * stride) * RP + r];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) weigh(tb + j * stride, x[j]);
        }
        for (; tb < n_pad; tb += stride) weigh(tb, lds[tb * RP + r]);
        return l;
    };
    // A wave per row; with fewer rows than waves and at least 1024 keys, every
    // wave takes keys wave*64 + lane, + NW*64, ... of every row instead, and the
    // waves' maxima and sums meet in LDS (a fixed-order sum): on 8192-key chunks
    // of 2 rows (batch 32, 8 KV heads) 152.9 against 153.7 us a launch, where a
    // wave per row left two waves idle.
    if (RP >= NW || n_pad < 1024) {
        for (int r = wave; r < RP; r += NW) {
            const float m = wave_max(row_max(r, lane, 64));
            const float l = wave_sum(row_exp(r, lane, 64, m));
            if (lane == 0) {
                row_m[r] = m;
                row_l[r] = l;
            }
        }
    } else {
        __shared__ float wpart[NW][RP];  // the waves' maxima, then their sums
        float mr[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const float m = wave_max(row_max(r, wave * 64 + lane, NW * 64));
            if (lane == 0) wpart[wave][r] = m;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            float m = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) m = fmaxf(m, wpart[w][r]);
            mr[r] = m;
        }
        __syncthreads();  // every wave has read the maxima
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const float l = wave_sum(row_exp(r, wave * 64 + lane, NW * 64, mr[r]));
            if (lane == 0) wpart[wave][r] = l;
        }
        __syncthreads();
        if (tid < RP) {
            row_m[tid] = mr[tid];
            row_l[tid] = tree_sum<NW>([&](int w) { return wpart[w][tid]; });
        }
    }
    __syncthreads();

    // ---- pass 2: acc = sum_j p_j v_j ----------------------------------------------
    float acc[RP][8];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[r][d] = 0.f;
    const int first_draft = sp - t0;  // local keys above this may be hidden from some rows
    pass(p.v_cache, vnb, vwb, false, vb0, true, [&](u32x4_t (&cur)[4], int s_) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tl = s_ * 16 + u * 4 + gq;
            float pr[RP];
#pragma unroll
            for (int r = 0; r < RP; ++r) pr[r] = lds[tl * RP + r];
            float vf[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) unpack2<F16>(cur[u][k], vf[2 * k], vf[2 * k + 1]);
            if (tl > first_draft) {
                // a later draft token (or padding past the context): rows that
                // cannot see it must not touch its value row, even NaN * 0
#pragma unroll
                for (int r = 0; r < RP; ++r)
                    if (pr[r] != 0.f) {
#pragma unroll
                        for (int d = 0; d < 8; ++d) acc[r][d] = fmaf(pr[r], vf[d], acc[r][d]);
                    }
            } else {
#pragma unroll
                for (int r = 0; r < RP; ++r)
#pragma unroll
                    for (int d = 0; d < 8; ++d) acc[r][d] = fmaf(pr[r], vf[d], acc[r][d]);
            }
        }
    });

    // ---- reduce the four key slots of a wave, then the four waves ---------------
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            acc[r][d] = xor32(xor16(acc[r][d], FAdd{}), FAdd{});
        }
    __syncthreads();  // every wave is done with the scores
    float *red = lds;  // [NW][RP][128]
    if (gq == 0) {
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int d = 0; d < 8; ++d) red[(wave * RP + r) * kHeadDim + cq * 8 + d] = acc[r][d];
    }
    __syncthreads();

    auto wave_sum_of = [&](int r, int d) {
        return tree_sum<NW>([&](int w) { return red[(w * RP + r) * kHeadDim + d]; });
    };

    // One-launch step, a sequence whose context is this one chunk: the output
    // rows are this chunk's acc / l (what the merge would compute from one
    // partial), written here; no partial, no arrival.
    if (kOneLaunch && p.counters && sc.n == 1) {
        for (int idx = tid; idx < p.rows * (kHeadDim / 2); idx += 64 * NW) {
            const int r = idx / (kHeadDim / 2), d = 2 * (idx - r * (kHeadDim / 2));
            const float x[2] = {wave_sum_of(r, d) / row_l[r], wave_sum_of(r, d + 1) / row_l[r]};
            store_out<F16, 2>(p, p.out, out_row_off(p, b, h, r) + d, x);
        }
        return;
    }

    const size_t part = (size_t)bh * n_chunks + c;
    float *wa = p.ws_acc + part * p.rows * kHeadDim;
    // device-scope stores: the one-launch step's merge may read them from another XCD
    for (int idx = tid; idx < p.rows * kHeadDim; idx += 64 * NW) {
        const int r = idx >> 7, d = idx & (kHeadDim - 1);
        st_dev(wa + idx, wave_sum_of(r, d));
    }
    if (tid < p.rows) {
        st_dev(p.ws_ml + (part * p.rows + tid) * 2 + 0, row_m[tid]);
        st_dev(p.ws_ml + (part * p.rows + tid) * 2 + 1, row_l[tid]);
    }

    // One-launch step: the workgroup that stores the last partial of (b, h)
    // merges all its rows and resets the arrival counter for the next call.
    if (kOneLaunch && p.counters) {
        __shared__ int s_last;
        wait_mem();       // this wave's partial stores are complete
        __syncthreads();  // and so are the other waves'
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&p.counters[bh * kCounterStride], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == sc.n - 1;
        __syncthreads();
        if (s_last) {
            merge_rows_block<F16, NW>(p, lds, bh, b, h, sc.n, tid);
            if (tid == 0) p.counters[bh * kCounterStride] = 0;
        }
    }
}

// LDS: the scores of the longest chunk, and at least the wave sums
// [NW][RP][128] and the fused merge's NW * 128 + 2 * NW floats.
template <int RP, int NW>
static size_t lds_bytes_of(const AttnParams &p) {
    size_t f = (size_t)RP * p.max_chunk;
    const size_t sums = (size_t)NW * RP * kHeadDim, merge = (size_t)NW * kHeadDim + 2 * NW;
    if (f < sums) f = sums;
    if (f < merge) f = merge;
    return f * sizeof(float);
}

template <bool F16, int RP>
static hipError_t launch_rp(const AttnParams &p, int grid, hipStream_t s) {
    const size_t lds = lds_bytes_of<RP, kValuWaves>(p);
    const dim3 block(64 * kValuWaves);
    if constexpr (RP <= kValuOneLaunchRows) {
        if (p.rope_freqs) {
            hipLaunchKernelGGL((attn_split_valu_kernel<F16, RP, true>), dim3(grid), block, lds, s, p.seq_pos, p.batch, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attn_split_valu_kernel<F16, RP, false>), dim3(grid), block, lds, s, p.seq_pos, p.batch, p);
    return hipGetLastError();
}

template <bool F16>
static hipError_t launch_dtype(const AttnParams &p, int grid, hipStream_t s) {
    if (p.rows <= 1) return launch_rp<F16, 1>(p, grid, s);
    if (p.rows <= 2) return launch_rp<F16, 2>(p, grid, s);
    if (p.rows <= 4) return launch_rp<F16, 4>(p, grid, s);
    if (p.rows <= 8) return launch_rp<F16, 8>(p, grid, s);
    return launch_rp<F16, 16>(p, grid, s);
}

hipError_t launch_attn_valu(const AttnParams &p, int grid, bool fp16, hipStream_t s) {
    return fp16 ? launch_dtype<true>(p, grid, s) : launch_dtype<false>(p, grid, s);
}

}  // namespace da
