// Split-context attention partials on the matrix cores for head_dim 256: the
// full-SDPA layers of "Architecture Diagram - Qwen3.5-35B-A3B" on the "Qwen MoE
// BringUp" page (GQA 16Q:2KV, head_dim 256; "Attention Computation" of the same
// page for what is computed).  Same contract and output as the head_dim-128
// kernel: per (sequence b, KV head h, chunk c) and query row r, the fp32
// partial (m, l, acc[256]) with scores in log2 units.
//
// Mapping on gfx950 (wave64).  A 256-dim key row is twice the bytes of a
// 128-dim one, so a tile holds 16 keys instead of 32 and the registers per tile
// stay the same:
//  - S^T = K q^T with v_mfma_f32_16x16x32: 16 keys x 16 query rows, eight
//    k-steps of 32 dims.  Lane (row l16, group q) holds q[row][32s + 8q .. +7]
//    for s = 0..7, and the key tile the same pieces of key l16.  The result
//    gives lane (l16, q) the scores of keys 4q .. 4q+3 of row l16;
//  - O^T += V^T P^T with v_mfma_f32_16x16x16 (k = 16 keys).  The B operand is
//    exactly those four weights of the lane (rounded to the 16-bit type, as on
//    the 128 kernel); the A operand wants keys 4q .. 4q+3 of one dim per lane:
//    lane (i, q) loads 16 bytes (dims 128 hh + 8i .. +7) of each of keys
//    4q .. 4q+3, and v_perm pairs their 16-bit halves, so MFMA (hh, o) produces
//    dims 128 hh + 8 (4q + v) + o of every row;
//  - one 4-wave workgroup per chunk.  Up to 16 query rows every wave computes
//    every row and the four waves take the chunk's tiles in turn (tile i by
//    wave i mod 4); above 16 rows the waves form two pairs, one per 16-row
//    group, and the two waves of a pair take the tiles in turn, so each tile
//    is read once per row group;
//  - everything else follows the head_dim-128 kernel: two tile buffers used
//    in turn, the per-row path for the chunk's last tile and this step's new
//    rows, the fused append, rotary embedding, paged caches and the in-launch
//    merge.
#include "da_internal.h"

#include <math.h>

#include <type_traits>

namespace da {
namespace {

constexpr int kD = 256;
constexpr int kRow = kD * 2;  // bytes per row
constexpr int kWaves = 4;     // waves per workgroup

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h16x4_t __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ f32x4_t mfma_k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ f32x4_t mfma_k16(u32x2_t a, u32x2_t b, f32x4_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h16x4_t, a),
                                                     __builtin_bit_cast(h16x4_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                         __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)round16<F16>(lo) | ((uint32_t)round16<F16>(hi) << 16);
}

// Rotary embedding of a row held as this lane's eight pieces (dims 32s + 8q ..
// +7): with the first R dims rotating, piece s < R/64 pairs with s + R/64.
// f0, f1 are freqs[8q .. 8q+7], which every R uses, loaded ahead by the caller.
template <bool F16>
__device__ __forceinline__ void rope_pieces8(u32x4_t (&x)[8], int R, int pos, const float *freqs, int q, f32x4_t f0,
                                             f32x4_t f1) {
    if (R == 256) {
        rope8_with<F16>(x[0], x[4], pos, f0, f1);
#pragma unroll
        for (int s = 1; s < 4; ++s) rope8<F16>(x[s], x[s + 4], pos, freqs, 32 * s + 8 * q);
    } else if (R == 128) {
        rope8_with<F16>(x[0], x[2], pos, f0, f1);
        rope8<F16>(x[1], x[3], pos, freqs, 32 + 8 * q);
    } else {  // R == 64
        rope8_with<F16>(x[0], x[1], pos, f0, f1);
    }
}
template <bool F16>
__device__ __forceinline__ void rope_pieces8(u32x4_t (&x)[8], int R, int pos, const float *freqs, int q) {
    rope_pieces8<F16>(x, R, pos, freqs, q, *reinterpret_cast<const f32x4_t *>(freqs + 8 * q),
                      *reinterpret_cast<const f32x4_t *>(freqs + 8 * q + 4));
}

struct Tile16 {
    u32x4_t k[8];     // K of key l16: dims 32s + 8q .. +7
    u32x4_t v[2][4];  // V of key 4q + u: dims 128 hh + 8 l16 .. +7
};

// A whole 16-key tile: one 16-token block (one page of a paged cache).
__device__ __forceinline__ void load_full16(Tile16 &t, const CacheView &cv, int tb, int l16, int q) {
    const size_t blk = cv.block(tb / kPageTokens);
    const uint8_t *kr = cv.k + blk + (size_t)l16 * kRow + 16 * q;
#pragma unroll
    for (int s = 0; s < 8; ++s) t.k[s] = ld16_stream(kr + 64 * s);
    const uint8_t *vr = cv.v + blk + (size_t)(4 * q) * kRow + 16 * l16;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int u = 0; u < 4; ++u) t.v[hh][u] = ld16_stream(vr + u * kRow + 256 * hh);
}

// Where rows come from when a tile is not all plain cache rows: keys past
// `last` re-read row `last` (scores masked, value rows zeroed), and this step's
// new rows (local keys from new_first on) come from k_new / v_new, rotated (K)
// and, by `store`, appended to the cache.
struct RowSource16 {
    const uint8_t *knew, *vnew;  // new rows of (b, h), row i at + i * stride
    size_t stride;
    int new_first;
    int t0;
    const float *rope;
    int rope_dim;
    bool store;
};

template <bool F16>
__device__ __forceinline__ void load_rows16(Tile16 &t, const CacheView &cv, int tb, int last, int l16, int q,
                                            const RowSource16 &rs) {
    {
        const int key = min(tb + l16, last);
        const uint8_t *kr = key >= rs.new_first ? rs.knew + (size_t)(key - rs.new_first) * rs.stride + 16 * q
                                                : cv.k + cv.row(key) + 16 * q;
#pragma unroll
        for (int s = 0; s < 8; ++s) t.k[s] = ld16(kr + 64 * s);
        if (rs.rope && key >= rs.new_first) rope_pieces8<F16>(t.k, rs.rope_dim, rs.t0 + key, rs.rope, q);
        if (rs.store && key >= rs.new_first && tb + l16 <= last && cv.writable(key)) {
            uint8_t *kw = cv.kw + cv.row(key) + 16 * q;
#pragma unroll
            for (int s = 0; s < 8; ++s) *reinterpret_cast<u32x4_t *>(kw + 64 * s) = t.k[s];
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int k_raw = tb + 4 * q + u;
        const int key = min(k_raw, last);
        const bool fresh = key >= rs.new_first;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            t.v[hh][u] = ld16(fresh ? rs.vnew + (size_t)(key - rs.new_first) * rs.stride + 256 * hh + 16 * l16
                                    : cv.v + cv.row(key) + 256 * hh + 16 * l16);
            if (k_raw > last) t.v[hh][u] = u32x4_t{0u, 0u, 0u, 0u};
            else if (rs.store && fresh && cv.writable(key))
                *reinterpret_cast<u32x4_t *>(cv.vw + cv.row(key) + 256 * hh + 16 * l16) = t.v[hh][u];
        }
    }
}

template <bool F16, int RG, bool ROPE>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_split_mfma256_kernel(const int32_t *__restrict__ seq_pos, int32_t batch, AttnParams p) {
    const int sp_first = first_seq_pos(seq_pos, batch, threadIdx.x & 63);
    constexpr int KS = kWaves / RG;  // waves sharing one row group's tiles
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave % RG, kw = wave / RG;

    int b, h, c;
    SeqChunks sc;
    int rest = blockIdx.x;
    int sp;
    if (!locate_wave(p, seq_pos, batch, sp_first, rest, b, h, c, sc, sp, lane)) {  // past the last chunk of the launch
        if (p.out && rest < p.batch && !seq_pos_ok(p, p.seq_pos[rest])) flag_sequence_nan<F16>(p, rest, tid, 64 * kWaves);
        return;
    }
    const int bh = b * p.n_kv_heads + h;
    const int t0 = c * sc.len;
    const int n_tok = min(sc.len, sc.ctx - t0);
    const int last = n_tok - 1;
    const int l16 = lane & 15, q = lane >> 4;

    // Paged caches: the chunk's pool pages, one per thread (chunks have at most
    // 4096 keys, 256 blocks), issued before the query loads and kept in LDS.
    static_assert(4096 / kPageTokens <= 64 * kWaves, "one block-table entry per thread");
    __shared__ int pg_tab[64 * kWaves];

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
    const int n_all = (n_tok + 15) >> 4;
    // keys past draft_first (this step's later draft tokens) are hidden from some
    // rows: they never sit in a whole tile (the per-row path handles them)
    const int draft_first = sp - t0;
    const int nt = min(n_tok >> 4, max(min(new_first, draft_first + 1), 0) >> 4);
    const int nj = kw < nt ? (nt - kw + KS - 1) / KS : 0;

    // B operand of S^T = K q^T: q[row][32s + 8q .. +7] for s = 0..7.  The 16 rows
    // live in this wave's LDS slice (row stride padded by 16 bytes against bank
    // conflicts) rather than in 32 registers the key tiles need; each tile reads
    // them back.  After the last tile the same memory serves the waves' merge.
    //
    // q (and the first rotation frequencies) are issued first, with no branch,
    // then the wave's first tile; the rotation and the LDS store follow, so the
    // tile's loads are in flight while q arrives.  Rows past p.rows re-read the
    // last row: all their keys are hidden (vis 0) and nothing of theirs is stored.
    // q rows while the tiles stream; then the same memory holds the four waves'
    // sums for the merge (16 rows x 256 floats each)
    __shared__ f32x4_t lds_q_red[kWaves * 16 * 64];
    static_assert(sizeof(u32x4_t) * kWaves * 16 * 33 <= sizeof(lds_q_red), "q rows fit the merge slots");
    auto &qsh = *reinterpret_cast<u32x4_t (*)[kWaves][16][33]>(lds_q_red);
    __shared__ float mlsh[kWaves][16][2];
    __shared__ int s_last;
    const int row = rg * 16 + l16;
    const int qrow = min(row, p.rows - 1);
    const int qi = div_small(qrow, p.group), qg = qrow - qi * p.group;
    const int vis = row < p.rows ? min(sp + qi + 1 - t0, n_tok) : 0;  // exclusive local key limit of this row
    u32x4_t qop[8];
    {
        const uint8_t *qp =
            p.q + (((size_t)b * p.q_len + qi) * p.n_q_heads + (size_t)h * p.group + qg) * kRow + 16 * q;
#pragma unroll
        for (int s = 0; s < 8; ++s) qop[s] = ld16(qp + 64 * s);
    }
    f32x4_t qf0, qf1;
    if (ROPE) {
        qf0 = *reinterpret_cast<const f32x4_t *>(p.rope_freqs + 8 * q);
        qf1 = *reinterpret_cast<const f32x4_t *>(p.rope_freqs + 8 * q + 4);
    }
    if (p.layout.block_table) {  // the load and its use in one branch: no load left pending past it
        store_chunk_page(p.layout, pg_tab, load_chunk_page(p.layout, b, t0, n_tok, tid), n_tok, tid);
        __syncthreads();
    }
    Tile16 ta, tb_;
    if (nj > 0) load_full16(ta, cv, kw * 16, l16, q);
    if (ROPE && row < p.rows) rope_pieces8<F16>(qop, p.rope_dim, sp + qi, p.rope_freqs, q, qf0, qf1);
#pragma unroll
    for (int s = 0; s < 8; ++s) qsh[wave][l16][4 * s + q] = qop[s];
    // the wave reads back what other lanes of it wrote
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t oacc[2][8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int o = 0; o < 8; ++o) oacc[hh][o] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One 16-key tile: S^T, online softmax, O^T += V^T P^T.  On the tiles of
    // the per-row path (kTail), this step's later draft keys (local keys past
    // draft_first) are hidden from some rows, which meet them in the P V
    // product with weight 0: exact for finite value rows.  If one of their value
    // rows holds an inf or NaN, they are left out of the product and added on
    // the vector ALU instead: for each such key k (wave-uniform) a lane takes its
    // row's rounded weight of k from the lane that holds it and, if that weight
    // is not 0, adds weight * v_k to its 64 dims, gathered from the tile's V
    // operand of the four lanes that hold them.
    auto compute = [&](Tile16 &t, int tt, auto tail) {
        constexpr bool kTail = decltype(tail)::value;
        const int tb = tt * 16;
        asm volatile("" ::: "memory");  // keep the q reads inside the loop (no hoisting into registers)
        f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) st = mfma_k32<F16>(t.k[s], qsh[wave][l16][4 * s + q], st);
        float x[4];
        float mt = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            x[v] = tb + 4 * q + v < vis ? st[v] * p.scale_log2 : -INFINITY;
            mt = fmaxf(mt, x[v]);
        }
        mt = xor32(xor16(mt, FMax{}), FMax{});
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
        float pw[4];
        float psum = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            pw[v] = (m_new == -INFINITY) ? 0.f : round_trip16<F16>(exp2_fast(x[v] - m_new));
            psum += pw[v];
        }
        if (__any(m_new != m_run)) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int o = 0; o < 8; ++o) oacc[hh][o] *= alpha;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        const u32x2_t pop = {pack2<F16>(pw[0], pw[1]), pack2<F16>(pw[2], pw[3])};
        bool split = false;  // kTail: a later draft key's value row is not finite
        if constexpr (kTail) {
            bool bad = false;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (tb + 4 * q + u > draft_first) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) bad |= nonfinite2<F16>(t.v[hh][u][w]);
                    }
            split = __any(bad);
        }
        u32x4_t tv[2][4];  // the V operand, without the later draft keys when split
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                tv[hh][u] = t.v[hh][u];
                if constexpr (kTail) {
                    if (split && tb + 4 * q + u > draft_first) tv[hh][u] = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int o = 0; o < 8; ++o) {
                const int w = o >> 1;
                const uint32_t sel = (o & 1) ? 0x07060302u : 0x05040100u;
                const u32x2_t vop = {__builtin_amdgcn_perm(tv[hh][1][w], tv[hh][0][w], sel),
                                     __builtin_amdgcn_perm(tv[hh][3][w], tv[hh][2][w], sel)};
                oacc[hh][o] = mfma_k16<F16>(vop, pop, oacc[hh][o]);
            }
        if constexpr (kTail) {
            const int k_hi = split ? min(tb + 15, last) : -1;
            for (int k = max(tb, draft_first + 1); k <= k_hi; ++k) {
                const int qk = (k - tb) >> 2, uk = (k - tb) & 3;  // lanes with q == qk hold key k in slot uk
                float pk = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) pk = v == uk ? pw[v] : pk;
                pk = __shfl(pk, l16 + 16 * qk);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    // v_k dims 128 hh + 8i .. + 7 sit in slot uk of lane (i, qk);
                    // this lane wants dims 128 hh + 32q .. + 31, from lanes (4q + v, qk)
                    u32x4_t vk;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        uint32_t x = 0;
#pragma unroll
                        for (int u = 0; u < 4; ++u) x = u == uk ? t.v[hh][u][w] : x;
                        vk[w] = x;
                    }
                    u32x4_t vr[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
#pragma unroll
                        for (int w = 0; w < 4; ++w) vr[v][w] = (uint32_t)__shfl((int)vk[w], 4 * q + v + 16 * qk);
                    if (pk != 0.f) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                float lo, hi;
                                unpack2<F16>(vr[v][w], lo, hi);
                                oacc[hh][2 * w][v] = fmaf(pk, lo, oacc[hh][2 * w][v]);
                                oacc[hh][2 * w + 1][v] = fmaf(pk, hi, oacc[hh][2 * w + 1][v]);
                            }
                    }
                }
            }
        }
    };

    // full tiles through two buffers used in turn
    if (nj > 0) {
        int j = 0;
        for (; j + 2 <= nj; j += 2) {
            load_full16(tb_, cv, (kw + KS * (j + 1)) * 16, l16, q);
            compute(ta, kw + KS * j, std::false_type{});
            if (j + 2 < nj) load_full16(ta, cv, (kw + KS * (j + 2)) * 16, l16, q);
            compute(tb_, kw + KS * (j + 1), std::false_type{});
        }
        if (j < nj) compute(ta, kw + KS * j, std::false_type{});
    }

    // the rest row by row (the chunk's last partial tile, this step's new rows),
    // tile i by wave i mod KS of the row group
    RowSource16 rs;
    rs.new_first = new_first;
    rs.t0 = t0;
    rs.rope = ROPE && p.k_new ? p.rope_freqs : nullptr;
    rs.rope_dim = p.rope_dim;
    rs.store = p.k_new != nullptr && rg == 0;
    rs.stride = (size_t)p.n_kv_heads * kRow;
    if (p.k_new) {
        const size_t noff = ((size_t)b * p.q_len * p.n_kv_heads + h) * kRow;
        rs.knew = p.k_new + noff;
        rs.vnew = p.v_new + noff;
    } else {
        rs.knew = rs.vnew = nullptr;
    }
    for (int i = nt; i < n_all; ++i) {
        if (i % KS != kw) continue;
        Tile16 tt_;
        load_rows16<F16>(tt_, cv, i * 16, last, l16, q, rs);
        compute(tt_, i, std::true_type{});
    }

    // ---- merge of the KS waves of a row group, then one partial per chunk ------
    // rows l16: dims 128 hh + 8 (4q + v) + o in oacc[hh][o][v]
    l_run = xor32(xor16(l_run, FAdd{}), FAdd{});
    if (q == 0) {
        mlsh[wave][l16][0] = m_run;
        mlsh[wave][l16][1] = l_run;
    }
    __syncthreads();  // every wave is past its last tile: qsh is free
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < KS; ++k) M = fmaxf(M, mlsh[rg + RG * k][l16][0]);
    float L = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const float mk = mlsh[rg + RG * k][l16][0];
        L += mk == -INFINITY ? 0.f : exp2_fast(mk - M) * mlsh[rg + RG * k][l16][1];
    }
    {
        const float f = m_run == -INFINITY ? 0.f : exp2_fast(m_run - M);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int o = 0; o < 8; ++o) oacc[hh][o] *= f;
    }
    // Every wave writes its sums to its own slot (16 rows x 256 floats in the q
    // memory, lane-private layout); after one barrier the waves of a row group
    // split the output slots and add the group's sums in a fixed order, with
    // four waves per group (0 + 2) + (1 + 3), and store them.
    f32x4_t *red = lds_q_red;
#pragma unroll
    for (int e = 0; e < 16; ++e) red[(wave * 16 + e) * 64 + lane] = oacc[e >> 3][e & 7];
    __syncthreads();
    constexpr int kE = 16 / KS;  // output slots per wave: hh = e / 8, o = e % 8
    const int e0 = kw * kE;
    f32x4_t sum[kE];
#pragma unroll
    for (int j = 0; j < kE; ++j) {
        const int e = e0 + j;
        auto slot = [&](int k) { return red[((rg + RG * k) * 16 + e) * 64 + lane]; };
        if constexpr (KS == 4)
            sum[j] = (slot(0) + slot(2)) + (slot(1) + slot(3));
        else
            sum[j] = slot(0) + slot(1);
    }

    if (row < p.rows) {
        const size_t part = ((size_t)bh * p.n_chunks + c) * p.rows + row;
        float *wa = p.ws_acc + part * kD;
        const bool dev = p.counters != nullptr;
#pragma unroll
        for (int j = 0; j < kE; j += 4) {
            const int hh = (e0 + j) >> 3, o = (e0 + j) & 7;  // four consecutive o of one hh
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float *dst = wa + 128 * hh + 8 * (4 * q + v) + o;
                if (dev) {
                    st_dev4(dst, sum[j][v], sum[j + 1][v], sum[j + 2][v], sum[j + 3][v]);
                } else {
                    *reinterpret_cast<float4 *>(dst) = make_float4(sum[j][v], sum[j + 1][v], sum[j + 2][v], sum[j + 3][v]);
                }
            }
        }
        if (kw == 0 && q == 0) {
            if (dev) {
                st_dev(p.ws_ml + part * 2 + 0, M);
                st_dev(p.ws_ml + part * 2 + 1, L);
            } else {
                p.ws_ml[part * 2 + 0] = M;
                p.ws_ml[part * 2 + 1] = L;
            }
        }
    }

    // One-launch step: the workgroup that stores the last partial of (b, h)
    // merges its rows (wave w takes rows w, w + 4, ..., two at a time) and
    // resets the arrival counter.
    if (p.counters) {
        wait_mem();       // this wave's partial stores are complete
        __syncthreads();  // and so are the other waves'
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&p.counters[bh * kCounterStride], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == sc.n - 1;
        __syncthreads();
        if (s_last) {
            if (sc.n <= 16) {
                for (int r = wave; r < p.rows; r += 2 * kWaves) merge_two_rows_wave<F16, kD>(p, bh, b, h, r, kWaves, sc.n, lane);
            } else {
                for (int r = wave; r < p.rows; r += kWaves) merge_row_wave<F16, kD>(p, p.out, bh, b, h, r, sc.n, lane);
            }
            if (tid == 0) p.counters[bh * kCounterStride] = 0;
        }
    }
}

// `items` = chunks in the launch (an upper bound), one workgroup each: four
// waves over the chunk's tiles (up to 16 rows), or two pairs (17..32 rows).
template <bool F16>
hipError_t launch_dtype256(const AttnParams &p, int items, hipStream_t s) {
    const dim3 grid(items), block(64 * kWaves);
    if (p.rope_freqs) {
        if (p.rows <= 16)
            hipLaunchKernelGGL((attn_split_mfma256_kernel<F16, 1, true>), grid, block, 0, s, p.seq_pos, p.batch, p);
        else
            hipLaunchKernelGGL((attn_split_mfma256_kernel<F16, 2, true>), grid, block, 0, s, p.seq_pos, p.batch, p);
    } else {
        if (p.rows <= 16)
            hipLaunchKernelGGL((attn_split_mfma256_kernel<F16, 1, false>), grid, block, 0, s, p.seq_pos, p.batch, p);
        else
            hipLaunchKernelGGL((attn_split_mfma256_kernel<F16, 2, false>), grid, block, 0, s, p.seq_pos, p.batch, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma256(const AttnParams &p, int items, bool fp16, hipStream_t s) {
    return fp16 ? launch_dtype256<true>(p, items, s) : launch_dtype256<false>(p, items, s);
}

}  // namespace da
