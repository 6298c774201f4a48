// Split-context attention partials on the matrix cores.  With many query
// rows sharing each key (8 query heads per KV head, or a 4-token speculative
// verify with 8 query heads per KV head: 32 rows), Q K^T and P V are real small
// matrix products, so they run as bf16/fp16 MFMA with fp32 accumulation ("Architecture Diagram -
// Qwen3-30B-A3B", paged attention: fp16 in, fp32 accumulate; "Attention
// Computation" for what is computed).
//
// Same contract as the vector-ALU kernel: per (sequence b, KV head h, chunk c)
// and query row r, (m, l, acc) with scores in log2 units, written to the
// workspace for the combine kernel.
//
// Mapping on gfx950 (wave64, v_mfma_f32_16x16x32_{bf16,f16}):
//  - a 4-wave workgroup owns one (b, h, chunk); its waves take the chunk's
//    32-key tiles in turn (tile i by wave i mod 4), each streaming its tiles
//    through two register buffers so its next tile is in flight while it
//    computes the current one.  Every wave computes every query row of the
//    KV head: rows come in blocks of 16 (one block up to 16 rows, held in
//    registers; two up to 32, whose q rows sit in LDS), so each tile is read
//    from memory once.  At
//    the end the waves' (m, l, acc) are merged through LDS in a fixed order
//    and one partial per chunk is stored;
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
//  - one MFMA applies a value row to 16 query rows at once, so a key hidden
//    from some of them would reach those rows as 0 * v, which is NaN for a
//    non-finite v.  The only such keys are this step's later draft tokens
//    (positions past seq_pos, at most q_len - 1 of them, in the chunk's last
//    tiles): their value rows are zeroed in the MFMA operand and added on the
//    vector ALU only to the rows that see them.  Slots past the context are
//    never read into a product.
#include "da_internal.h"

#include <math.h>

#include <type_traits>

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

// Key of slot u (0..7) of lane group q inside a 32-key tile, in the order the
// P V product consumes them: keys 4q..4q+3, then 16+4q..16+4q+3.
__device__ __forceinline__ int pv_key(int q, int u) { return (u < 4 ? 4 * q + u : 16 + 4 * q + (u - 4)); }

// Rotary embedding of one row held as this lane's four 16-byte pieces, dims
// 8q + 32s .. +7 (s = 0..3): with the first R dims rotating (pairs j, j + R/2),
// piece s < R/64 pairs with piece s + R/64 of the same lane.
// The frequencies those pieces use, freqs[8q .. 8q+7] and, when R = 128,
// freqs[32+8q .. 32+8q+7], loaded ahead of the rotation.
__device__ __forceinline__ void piece_freqs(f32x4_t (&f)[4], int R, const float *freqs, int q) {
    f[0] = *reinterpret_cast<const f32x4_t *>(freqs + 8 * q);
    f[1] = *reinterpret_cast<const f32x4_t *>(freqs + 8 * q + 4);
    if (R == 128) {
        f[2] = *reinterpret_cast<const f32x4_t *>(freqs + 32 + 8 * q);
        f[3] = *reinterpret_cast<const f32x4_t *>(freqs + 36 + 8 * q);
    } else {
        f[2] = f[3] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
}
template <bool F16>
__device__ __forceinline__ void rope_pieces_with(u32x4_t (&x)[4], int R, int pos, const f32x4_t (&f)[4]) {
    if (R == 128) {
        rope8_with<F16>(x[0], x[2], pos, f[0], f[1]);
        rope8_with<F16>(x[1], x[3], pos, f[2], f[3]);
    } else {  // R == 64
        rope8_with<F16>(x[0], x[1], pos, f[0], f[1]);
    }
}
template <bool F16>
__device__ __forceinline__ void rope_pieces(u32x4_t (&x)[4], int R, int pos, const float *freqs, int q) {
    f32x4_t f[4];
    piece_freqs(f, R, freqs, q);
    rope_pieces_with<F16>(x, R, pos, f);
}

struct Tile {
    u32x4_t k[2][4];  // K: key block kb (16 keys), k-step s (32 dims)
    u32x4_t v[8];     // V: slot u, dims 8i .. 8i+7
};

// A whole 32-key tile inside the chunk: two block bases, immediate offsets.
__device__ __forceinline__ void load_full(Tile &t, const CacheView &cv, int tb, int l16, int q) {
    const size_t blk[2] = {cv.block(tb / kPageTokens), cv.block(tb / kPageTokens + 1)};
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk) {
        const uint8_t *kr = cv.k + blk[kblk] + (size_t)l16 * kRowBytes + 16 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) t.k[kblk][s] = ld16_stream(kr + 64 * s);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint8_t *v0 = cv.v + blk[half] + (size_t)(4 * q) * kRowBytes + 16 * l16;
#pragma unroll
        for (int u = 0; u < 4; ++u) t.v[4 * half + u] = ld16_stream(v0 + u * kRowBytes);
    }
}

// Where a tile's rows come from when they are not all plain cache rows: the
// chunk's partial last tile (keys past `last` re-read row `last`, their scores
// are masked and their value rows zeroed so a non-finite last row cannot reach
// other rows as 0 * inf), and in the one-launch step the tiles holding this
// step's new rows (local keys from `new_first` on), which are read from
// k_new / v_new and, by `store`, appended to the cache.
struct RowSource {
    const uint8_t *knew, *vnew;  // new rows of (b, h), row i at + i * stride
    size_t stride;
    int new_first;
    int t0;             // absolute position of local key 0
    const float *rope;  // rotary table: new K rows are rotated at t0 + key first
    int rope_dim;
    bool store;
};

template <bool F16>
__device__ __forceinline__ void load_rows(Tile &t, const CacheView &cv, int tb, int last, int l16, int q,
                                          const RowSource &rs) {
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk) {
        const int key = min(tb + 16 * kblk + l16, last);
        const uint8_t *kr = key >= rs.new_first ? rs.knew + (size_t)(key - rs.new_first) * rs.stride + 16 * q
                                                : cv.k + cv.row(key) + 16 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) t.k[kblk][s] = ld16(kr + 64 * s);
        if (rs.rope && key >= rs.new_first) rope_pieces<F16>(t.k[kblk], rs.rope_dim, rs.t0 + key, rs.rope, q);
        if (rs.store && key >= rs.new_first && tb + 16 * kblk + l16 <= last && cv.writable(key)) {
            uint8_t *kw = cv.kw + cv.row(key) + 16 * q;
#pragma unroll
            for (int s = 0; s < 4; ++s) *reinterpret_cast<u32x4_t *>(kw + 64 * s) = t.k[kblk][s];
        }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int k_raw = tb + pv_key(q, u);
        const int key = min(k_raw, last);
        t.v[u] = ld16(key >= rs.new_first ? rs.vnew + (size_t)(key - rs.new_first) * rs.stride + 16 * l16
                                          : cv.v + cv.row(key) + 16 * l16);
        if (k_raw > last) t.v[u] = u32x4_t{0u, 0u, 0u, 0u};
        else if (rs.store && key >= rs.new_first && cv.writable(key))
            *reinterpret_cast<u32x4_t *>(cv.vw + cv.row(key) + 16 * l16) = t.v[u];
    }
}

constexpr int kMfmaWaves = 4;  // waves per workgroup, all on one chunk

template <bool F16, int RB, bool ROPE>
__global__ __launch_bounds__(64 * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_split_mfma_kernel(const int32_t *__restrict__ seq_pos, int32_t batch, AttnParams p) {
    const int sp_first = first_seq_pos(seq_pos, batch, threadIdx.x & 63);
    constexpr int KS = kMfmaWaves;  // waves taking the chunk's tiles in turn
    const int tid = threadIdx.x, lane = tid & 63;
    const int kw = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches

    int b, h, c;
    SeqChunks sc;
    int rest = blockIdx.x;
    int sp;
    if (!locate_wave(p, seq_pos, batch, sp_first, rest, b, h, c, sc, sp, lane)) {  // past the last chunk of the launch
        if (p.out && rest < p.batch && !seq_pos_ok(p, p.seq_pos[rest]))
            flag_sequence_nan<F16>(p, rest, tid, 64 * kMfmaWaves);
        return;
    }
    const int bh = b * p.n_kv_heads + h;
    const int t0 = c * sc.len;
    const int n_tok = min(sc.len, sc.ctx - t0);
    const int last = n_tok - 1;
    const int l16 = lane & 15, q = lane >> 4;

    // Paged caches: the chunk's pool pages, one per thread (chunks have at most
    // 4096 keys, 256 blocks), issued before the query loads and kept in LDS, so
    // that no tile waits on a block-table load.
    static_assert(4096 / kPageTokens <= 64 * kMfmaWaves, "one block-table entry per thread");
    __shared__ int pg_tab[64 * kMfmaWaves];

    CacheView cv;
    cv.k = p.k_cache;
    cv.v = p.v_cache;
    cv.kw = p.k_cache_w;
    cv.vw = p.v_cache_w;
    cv.L = p.layout;
    cv.b = b;
    cv.h = h;
    cv.n_kv_heads = p.n_kv_heads;
    cv.max_seq = p.max_seq;
    cv.t0 = t0;
    cv.pg_tab = pg_tab;

    // Tiles 0 .. nt-1 hold old cache rows only and load whole; this wave takes
    // tiles kw, kw + KS, ... of them.
    const int new_first = p.k_new ? sp - t0 : n_tok;
    const int n_all = (n_tok + 31) >> 5;
    // keys past draft_first (this step's later draft tokens) are hidden from some
    // rows: they never sit in a whole tile (the per-row path handles them)
    const int draft_first = sp - t0;
    const int nt = min(n_tok >> 5, max(min(new_first, draft_first + 1), 0) >> 5);
    const int nj = kw < nt ? (nt - kw + KS - 1) / KS : 0;

    // B operand of S^T = K q^T for row block rb: q[rb*16 + l16][dims 32s + 8q .. +7],
    // s = 0..3.  One row block stays in this wave's registers; two live in LDS,
    // shared by the four waves (row stride padded by 16 bytes against bank
    // conflicts): wave rb loads and rotates row block rb, and every tile reads
    // them back.
    int vis[RB];  // exclusive local key limit of this lane's row in each row block
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 16 + l16;
        const int i = row / p.group;
        vis[rb] = row < p.rows ? min(sp + i + 1 - t0, n_tok) : 0;
    }
    // Rows past p.rows re-read the last row (no branch between these loads and
    // the first tile's): all their keys are hidden (vis 0) and nothing of
    // theirs is stored.
    auto issue_q = [&](u32x4_t (&qop)[4], int rb) {
        const int row = min(rb * 16 + l16, p.rows - 1);
        const int i = row / p.group, g = row - i * p.group;
        const uint8_t *qp =
            p.q + (((size_t)b * p.q_len + i) * p.n_q_heads + (size_t)h * p.group + g) * kRowBytes + 16 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) qop[s] = ld16(qp + 64 * s);
    };
    // q (and its rotation's frequencies) are issued first.  With one row block
    // the wave's first tile follows at once and q is rotated after it: the
    // tile's loads are in flight while q arrives.  The rotation is a separate
    // instantiation, so that without a table no conditional load sits between
    // the two.
    u32x4_t qreg[4];
    __shared__ u32x4_t qsh[RB > 1 ? RB : 1][16][17];
    const bool loads_q = RB == 1 || kw < RB;
    if (loads_q) issue_q(qreg, RB == 1 ? 0 : kw);
    if (p.layout.block_table) {  // the load and its use in one branch: no load left pending past it
        store_chunk_page(p.layout, pg_tab, load_chunk_page(p.layout, b, t0, n_tok, tid), n_tok, tid);
        __syncthreads();
    }
    f32x4_t qfreq[4];
    if (ROPE && loads_q) piece_freqs(qfreq, p.rope_dim, p.rope_freqs, q);
    auto rotate_q = [&](u32x4_t (&qop)[4], int rb) {
        const int row = rb * 16 + l16;
        if (ROPE && row < p.rows) rope_pieces_with<F16>(qop, p.rope_dim, sp + row / p.group, qfreq);
    };
    Tile ta, tb_;
    if constexpr (RB > 1) {
        // The row blocks are stored before the wave's first tile is issued.
        // Stored after it, the store (on one side of a branch) made the compiler
        // wait for the tile's loads too, and the first compute then waited for
        // the whole tile instead of its first quarter: 1.1 us more on the
        // 32-row verify workload.
        if (kw < RB) {
            rotate_q(qreg, kw);
#pragma unroll
            for (int s = 0; s < 4; ++s) qsh[kw][l16][4 * s + q] = qreg[s];
        }
        if (nj > 0) load_full(ta, cv, kw * 32, l16, q);
        __syncthreads();
    } else {
        if (nj > 0) load_full(ta, cv, kw * 32, l16, q);
        rotate_q(qreg, 0);
    }
    auto qpiece = [&](int rb, int s) -> u32x4_t {
        if constexpr (RB == 1)
            return qreg[s];
        else
            return qsh[rb][l16][4 * s + q];
    };

    float m_run[RB], l_run[RB];
    f32x4_t oacc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
#pragma unroll
        for (int o = 0; o < 8; ++o) oacc[rb][o] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // One 32-key tile: S^T and the online softmax of every row block, then
    // O^T += V^T P^T with each V operand serving every row block.
    // On the tiles of the per-row path (kTail), this step's later draft keys
    // (local keys past draft_first) are hidden from some rows, which meet them
    // in the P V product with weight 0: exact for finite value rows.  If one of
    // their value rows holds an inf or NaN, they are left out of the product
    // and added on the vector ALU instead: for each such key k (wave-uniform) a
    // lane takes its row's rounded weight of k from the lane that holds it and,
    // if that weight is not 0, adds weight * v_k to its 32 dims, which it
    // gathers from the tile's V operand of the four lanes that hold them.
    auto compute = [&](Tile &t, int tt, auto tail) {
        constexpr bool kTail = decltype(tail)::value;
        const int tb = tt * 32;
        if constexpr (RB > 1) asm volatile("" ::: "memory");  // keep the q reads inside the loop
        u32x4_t pop[RB];
        float pvs[RB][8];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            // S^T for the two 16-key blocks: lane holds keys tb + 16*kblk + 4q + v of its row
            f32x4_t st[2];
#pragma unroll
            for (int kblk = 0; kblk < 2; ++kblk) {
                st[kblk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) st[kblk] = mfma16<F16>(t.k[kblk][s], qpiece(rb, s), st[kblk]);
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
            mt = xor32(xor16(mt, FMax{}), FMax{});
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
#pragma unroll
            for (int j = 0; j < 4; ++j) pop[rb][j] = pack16<F16>(pv[2 * j], pv[2 * j + 1]);
            if constexpr (kTail) {
#pragma unroll
                for (int u = 0; u < 8; ++u) pvs[rb][u] = pv[u];
            }
        }
        bool split = false;  // kTail: a later draft key's value row is not finite
        if constexpr (kTail) {
            bool bad = false;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (tb + pv_key(q, u) > draft_first) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) bad |= nonfinite2<F16>(t.v[u][w]);
                }
            split = __any(bad);
        }
        u32x4_t tv[8];  // the V operand, without the later draft keys when split
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            tv[u] = t.v[u];
            if constexpr (kTail) {
                if (split && tb + pv_key(q, u) > draft_first) tv[u] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int o = 0; o < 8; ++o) {
            const int word = o >> 1;
            const uint32_t sel = (o & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t vop;
#pragma unroll
            for (int j = 0; j < 4; ++j) vop[j] = __builtin_amdgcn_perm(tv[2 * j + 1][word], tv[2 * j][word], sel);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) oacc[rb][o] = mfma16<F16>(vop, pop[rb], oacc[rb][o]);
        }
        if constexpr (kTail) {
            const int k_hi = split ? min(tb + 31, last) : -1;
            for (int k = max(tb, draft_first + 1); k <= k_hi; ++k) {
                const int kk = k - tb, qk = (kk & 15) >> 2;
                const int uk = 4 * (kk >> 4) + (kk & 3);  // slot of key k in the lanes with q == qk
                // v_k dims 8i .. 8i + 7 sit in slot uk of lane (i, qk); this lane
                // wants dims 32q .. 32q + 31, from lanes (4q + v, qk), v = 0..3
                u32x4_t vk;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t x = 0;
#pragma unroll
                    for (int u = 0; u < 8; ++u) x = u == uk ? t.v[u][w] : x;
                    vk[w] = x;
                }
                u32x4_t vr[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int w = 0; w < 4; ++w) vr[v][w] = (uint32_t)__shfl((int)vk[w], 4 * q + v + 16 * qk);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    float pk = 0.f;
#pragma unroll
                    for (int u = 0; u < 8; ++u) pk = u == uk ? pvs[rb][u] : pk;
                    pk = __shfl(pk, l16 + 16 * qk);
                    if (pk != 0.f) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                float lo, hi;
                                unpack2<F16>(vr[v][w], lo, hi);
                                oacc[rb][2 * w][v] = fmaf(pk, lo, oacc[rb][2 * w][v]);
                                oacc[rb][2 * w + 1][v] = fmaf(pk, hi, oacc[rb][2 * w + 1][v]);
                            }
                    }
                }
            }
        }
    };

    // Full tiles: with one row block through two register buffers used in
    // turn, with no copy between them, so the wave waits only for the older
    // tile while the newer one is in flight; with two row blocks (whose second
    // accumulator takes the registers of the second buffer) one tile at a time,
    // the workgroup's other waves keeping the compute unit's loads in flight.
    if constexpr (RB == 1) {
        if (nj > 0) {
            int j = 0;
            for (; j + 2 <= nj; j += 2) {
                load_full(tb_, cv, (kw + KS * (j + 1)) * 32, l16, q);
                compute(ta, kw + KS * j, std::false_type{});
                if (j + 2 < nj) load_full(ta, cv, (kw + KS * (j + 2)) * 32, l16, q);
                compute(tb_, kw + KS * (j + 1), std::false_type{});
            }
            if (j < nj) compute(ta, kw + KS * j, std::false_type{});
        }
    } else {
        for (int j = 0; j < nj; ++j) {
            if (j > 0) load_full(ta, cv, (kw + KS * j) * 32, l16, q);
            compute(ta, kw + KS * j, std::false_type{});
        }
    }

    // The tiles that hold new rows or run past the chunk take the per-row path,
    // tile i by wave i mod KS (which also appends its new rows).
    RowSource rs;
    rs.new_first = new_first;
    rs.t0 = t0;
    rs.rope = ROPE && p.k_new ? p.rope_freqs : nullptr;
    rs.rope_dim = p.rope_dim;
    rs.store = p.k_new != nullptr;
    rs.stride = (size_t)p.n_kv_heads * kRowBytes;
    if (p.k_new) {
        const size_t noff = ((size_t)b * p.q_len * p.n_kv_heads + h) * kRowBytes;
        rs.knew = p.k_new + noff;
        rs.vnew = p.v_new + noff;
    } else {
        rs.knew = rs.vnew = nullptr;
    }
    for (int i = nt; i < n_all; ++i) {
        if (i % KS != kw) continue;
        Tile tt_;
        load_rows<F16>(tt_, cv, i * 32, last, l16, q, rs);
        compute(tt_, i, std::true_type{});
    }

    // ---- merge of the four waves, then one partial per chunk --------------------
    // lane: row rb*16 + l16, dims 8 (4q + v) + o in oacc[rb][o][v]
    __shared__ float mlsh[kMfmaWaves][RB][16][2];
    __shared__ f32x4_t red[kMfmaWaves][RB][8][64];  // one slot per wave, lane-private layout
    __shared__ int s_last;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        l_run[rb] = xor32(xor16(l_run[rb], FAdd{}), FAdd{});
        if (q == 0) {
            mlsh[kw][rb][l16][0] = m_run[rb];
            mlsh[kw][rb][l16][1] = l_run[rb];
        }
    }
    __syncthreads();
    float M[RB], L[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        M[rb] = -INFINITY;
#pragma unroll
        for (int k = 0; k < KS; ++k) M[rb] = fmaxf(M[rb], mlsh[k][rb][l16][0]);
        L[rb] = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const float mk = mlsh[k][rb][l16][0];
            L[rb] += mk == -INFINITY ? 0.f : exp2_fast(mk - M[rb]) * mlsh[k][rb][l16][1];
        }
        const float f = m_run[rb] == -INFINITY ? 0.f : exp2_fast(m_run[rb] - M[rb]);
#pragma unroll
        for (int o = 0; o < 8; ++o) oacc[rb][o] *= f;
    }
    // Every wave writes its rescaled sums; after one barrier wave w adds output
    // slots o = 2w, 2w + 1 of all four in a fixed order, (0 + 1) + (2 + 3), and
    // stores them, so the adds and the stores are shared by the four waves.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int o = 0; o < 8; ++o) red[kw][rb][o][lane] = oacc[rb][o];
    __syncthreads();

    // When the one-launch step merges in this launch, device-scope stores (the
    // merge may read them from another XCD); else plain stores, which the L2
    // gathers into whole lines (a lane's 8-byte pieces are scattered).
    {
        const bool dev = p.counters != nullptr;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            f32x4_t sum[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int o = 2 * kw + j;
                sum[j] = (red[0][rb][o][lane] + red[1][rb][o][lane]) + (red[2][rb][o][lane] + red[3][rb][o][lane]);
            }
            const int row = rb * 16 + l16;
            if (row >= p.rows) continue;
            const size_t part = ((size_t)bh * p.n_chunks + c) * p.rows + row;
            float *wa = p.ws_acc + part * kHeadDim;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                // dims 8*(4q+v) + 2w and + 1: two consecutive floats of this lane
                float *dst = wa + 8 * (4 * q + v) + 2 * kw;
                if (dev) {
                    __hip_atomic_store(reinterpret_cast<uint64_t *>(dst),
                                       (uint64_t)__float_as_uint(sum[0][v]) |
                                           ((uint64_t)__float_as_uint(sum[1][v]) << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    *reinterpret_cast<float2 *>(dst) = make_float2(sum[0][v], sum[1][v]);
                }
            }
            if (kw == 0 && q == 0) {
                if (dev) {
                    st_dev(p.ws_ml + part * 2 + 0, M[rb]);
                    st_dev(p.ws_ml + part * 2 + 1, L[rb]);
                } else {
                    p.ws_ml[part * 2 + 0] = M[rb];
                    p.ws_ml[part * 2 + 1] = L[rb];
                }
            }
        }
    }

    // One-launch step: the workgroup that stores the last partial of (b, h)
    // merges its rows (wave w takes rows w, w + 4, ..., two at a time) and
    // resets the arrival counter for the next call.
    if (p.counters) {
        wait_mem();       // this wave's partial stores are complete
        __syncthreads();  // and so are the other waves'
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&p.counters[bh * kCounterStride], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == sc.n - 1;
        __syncthreads();
        if (s_last) {
            if (sc.n <= 16) {
                for (int r = kw; r < p.rows; r += 2 * kMfmaWaves)
                    merge_two_rows_wave<F16, kHeadDim>(p, bh, b, h, r, kMfmaWaves, sc.n, lane);
            } else {
                for (int r = kw; r < p.rows; r += kMfmaWaves)
                    merge_row_wave<F16, kHeadDim>(p, p.out, bh, b, h, r, sc.n, lane);
            }
            if (tid == 0) p.counters[bh * kCounterStride] = 0;
        }
    }
}

// `items` = chunks in the launch (an upper bound), one workgroup each: four
// waves over the chunk's tiles, each computing every row (one 16-row block up
// to 16 rows, two up to 32).
template <bool F16>
static hipError_t launch_dtype(const AttnParams &p, int items, hipStream_t s) {
    const dim3 grid(items), block(64 * kMfmaWaves);
    if (p.rope_freqs) {
        if (p.rows <= 16)
            hipLaunchKernelGGL((attn_split_mfma_kernel<F16, 1, true>), grid, block, 0, s, p.seq_pos, p.batch, p);
        else
            hipLaunchKernelGGL((attn_split_mfma_kernel<F16, 2, true>), grid, block, 0, s, p.seq_pos, p.batch, p);
    } else {
        if (p.rows <= 16)
            hipLaunchKernelGGL((attn_split_mfma_kernel<F16, 1, false>), grid, block, 0, s, p.seq_pos, p.batch, p);
        else
            hipLaunchKernelGGL((attn_split_mfma_kernel<F16, 2, false>), grid, block, 0, s, p.seq_pos, p.batch, p);
    }
    return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnParams &p, int grid, bool fp16, hipStream_t s) {
    if (p.head_dim != kHeadDim) return launch_attn_mfma256(p, grid, fp16, s);
    return fp16 ? launch_dtype<true>(p, grid, s) : launch_dtype<false>(p, grid, s);
}

}  // namespace da
