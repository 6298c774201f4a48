// Internal declarations shared by the HIP translation units of libdecode_attn.
// Device helpers for gfx950 (CDNA4, wave64) and the parameter blocks the host
// launcher hands to each kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace da {

constexpr int kHeadDim = 128;     // head_dim of the vector-ALU kernel and the 128 MFMA kernel
constexpr int kRowBytes = kHeadDim * 2;
constexpr int kMaxHeadDim = 256;  // the MFMA kernel also takes 256
constexpr int kMaxRows = 32;      // (Hq/Hkv) * q_len limit
constexpr int kMaxQLen = 8;
constexpr int kTokenTile = 64;    // chunk sizes are multiples of this
constexpr int kMaxChunk = 2048;  // longest fixed chunk (chunk_tokens); balanced chunks go up to 4096 / 8192
constexpr int kValuLongChunk = 8192;  // the vector-ALU kernel's long chunks (at most 2 rows)
// int32s between two (sequence, KV head) arrival counters of the one-launch step:
// one 128-byte line each, so the arrivals of different heads do not contend for
// one line (batch-1 MHA at 4k, 16 chunks per head: 14.15 -> 13.6 us a layer).
constexpr int kCounterStride = 32;

// ---- cache layout -----------------------------------------------------------
// Contiguous: [B][Hkv][max_seq][D].  Paged ("Architecture Diagram - Qwen3-30B-A3B",
// Paged Attention: a page pool [pages][KV heads][16 tokens][D]): token t of
// sequence b is in pool page block_table[b][t / 16], slot t % 16, and max_seq =
// pages_per_seq * 16.
struct KvLayout {
    const int32_t *block_table;  // [B][pages_per_seq], null for the contiguous layout
    int32_t pages_per_seq, n_pages;
    int32_t row_bytes;           // head_dim * 2
};

constexpr int kPageTokens = 16;

// Pool page of logical page `lp` of sequence b; a block-table entry outside the
// pool gives -1 (the caller's contract is broken: reads use page 0, writes are
// dropped, so nothing outside the pool is touched).
__device__ __forceinline__ int kv_page(const KvLayout &L, int b, int lp) {
    const int pg = L.block_table[(size_t)b * L.pages_per_seq + lp];
    return (unsigned)pg < (unsigned)L.n_pages ? pg : -1;
}

// Byte offset of the 16-token block holding tokens 16 * lp .. 16 * lp + 15 of
// (b, h), and of token t.  Contiguous caches have no pages, but the same
// arithmetic (blocks of 16 consecutive rows) applies.
__device__ __forceinline__ size_t kv_block_off(const KvLayout &L, int b, int h, int n_kv_heads, int max_seq,
                                               int lp) {
    if (!L.block_table)
        return (((size_t)b * n_kv_heads + h) * max_seq + (size_t)lp * kPageTokens) * L.row_bytes;
    const int pg = kv_page(L, b, lp);
    return ((size_t)(pg < 0 ? 0 : pg) * n_kv_heads + h) * kPageTokens * L.row_bytes;
}
__device__ __forceinline__ size_t kv_row_off(const KvLayout &L, int b, int h, int n_kv_heads, int max_seq, int t) {
    return kv_block_off(L, b, h, n_kv_heads, max_seq, t / kPageTokens) + (size_t)(t % kPageTokens) * L.row_bytes;
}
__device__ __forceinline__ bool kv_row_writable(const KvLayout &L, int b, int t) {
    return !L.block_table || kv_page(L, b, t / kPageTokens) >= 0;
}

// The caches of one (sequence b, KV head h) seen from a chunk starting at key t0
// (a multiple of 32): contiguous, or paged through the block table.  A 16-token
// block is one page of a paged cache.
struct CacheView {
    const uint8_t *k, *v;  // whole caches / pools
    uint8_t *kw, *vw;      // the same, writable (one-launch step), or null
    KvLayout L;
    int b, h, n_kv_heads, max_seq, t0;
    const int *pg_tab;  // paged: the pool page of the chunk's block j (-1 outside the pool), in LDS
    // byte offset of the chunk's 16-token block j; a page outside the pool reads page 0
    __device__ __forceinline__ size_t block_of_page(int pg) const {
        return ((size_t)(pg < 0 ? 0 : pg) * n_kv_heads + h) * kPageTokens * L.row_bytes;
    }
    __device__ __forceinline__ size_t block(int j) const {  // j wave-uniform
        if (!L.block_table) return kv_block_off(L, b, h, n_kv_heads, max_seq, t0 / kPageTokens + j);
        return block_of_page(__builtin_amdgcn_readfirstlane(pg_tab[j]));
    }
    __device__ __forceinline__ size_t row(int key) const {  // key may differ per lane
        if (!L.block_table) return kv_row_off(L, b, h, n_kv_heads, max_seq, t0 + key);
        return block_of_page(pg_tab[key / kPageTokens]) + (size_t)(key % kPageTokens) * L.row_bytes;
    }
    __device__ __forceinline__ bool writable(int key) const {
        return !L.block_table || pg_tab[key / kPageTokens] >= 0;
    }
};

// Paged caches: the pool pages of a chunk's 16-token blocks, one per thread of a
// workgroup (a chunk has at most `n_threads` blocks).  load_chunk_pages issues the
// raw block-table load early; store_chunk_pages checks it against the pool and
// writes it to `tab` in LDS (the caller then synchronises the workgroup).
__device__ __forceinline__ int load_chunk_page(const KvLayout &L, int b, int t0, int n_tok, int tid) {
    int pg = 0;
    if (L.block_table && tid < (n_tok + kPageTokens - 1) / kPageTokens)
        pg = L.block_table[(size_t)b * L.pages_per_seq + t0 / kPageTokens + tid];
    return pg;
}
__device__ __forceinline__ void store_chunk_page(const KvLayout &L, int *tab, int pg, int n_tok, int tid) {
    if (tid < (n_tok + kPageTokens - 1) / kPageTokens) tab[tid] = (unsigned)pg < (unsigned)L.n_pages ? pg : -1;
}

// ---- parameter blocks ------------------------------------------------------

struct AppendParams {
    uint8_t *k_cache;
    uint8_t *v_cache;
    const uint8_t *k_new;
    const uint8_t *v_new;
    const int32_t *seq_pos;
    const float *rope_freqs;   // rope_dim/2 rotary frequencies, or null: k_new is copied as is
    KvLayout layout;
    int32_t batch, q_len, n_kv_heads, max_seq;
    int32_t head_dim, rope_dim;
};

struct AttnParams {
    const uint8_t *q;
    const uint8_t *k_cache;
    const uint8_t *v_cache;
    const int32_t *seq_pos;
    float *ws_acc;  // [B*Hkv][n_chunks][rows][head_dim] unnormalised weighted V sums
    float *ws_ml;   // [B*Hkv][n_chunks][rows][2]  (running max in log2 units, sum)
    int32_t batch, q_len, n_q_heads, n_kv_heads, max_seq;
    int32_t head_dim;  // 128 or 256 (256: MFMA kernel only)
    int32_t group;  // Hq / Hkv
    int32_t rows;   // group * q_len
    int32_t n_chunks;      // chunk slots per (sequence, KV head) in the workspace
    int32_t fixed_chunk;   // > 0: every chunk has this many keys; 0: balanced chunks
    int32_t target_wg;     // balanced: chunks to aim for over the whole launch
    int32_t alt_target_wg; // balanced: the target for contexts too uneven for target_wg's
                           //   long chunks (0: none; see balanced_chunk)
    int32_t min_chunk;     // balanced: smallest chunk (multiple of 32)
    int32_t max_chunk;     // largest chunk the kernel accepts (multiple of 32)
    float scale_log2;      // softmax scale * log2(e): scores are kept in log2 units
    const float *rope_freqs;  // rope_dim/2 rotary frequencies, or null: q (and fused-appended
                              //   k_new rows) are used as given
    int32_t rope_dim;         // rotated dims (the first rope_dim of each row)
    KvLayout layout;          // contiguous or paged caches
    const uint16_t *out_gate; // [B][q_len][Hq][D] sigmoid output gate, or null
    int32_t seq_chunk_cap; // balanced: at most this many chunks per sequence unless its
                           //   length needs more of max_chunk keys (0: no cap)
    int32_t chunk_align;   // balanced: a sequence whose chunks would be at least 3/4
                           //   this long gets lengths rounded up to a multiple of it
                           //   (a multiple of 32; 32: no effect)

    // One-launch step (all null for the separate entry points):
    uint8_t *k_cache_w;        // k_cache as writable: the fused append stores new rows here
    uint8_t *v_cache_w;
    const uint8_t *k_new;      // [B][q_len][Hkv][D]: the chunk holding a sequence's new
    const uint8_t *v_new;      //   positions reads them from here and appends them
    int32_t *counters;         // [B*Hkv] chunk arrivals, kCounterStride apart, for the fused combine (0 between calls)
    uint16_t *out;             // output written by the fused combine
};

// ---- split-context chunk plan, computed identically by every kernel ---------
//
// Balanced mode: the chunk length aims at an equal share of all visible keys
// per chunk, T = ceil32(Hkv * sum_b ctx_b / target_wg) clamped to
// [min_chunk, max_chunk]; sequence b gets n_b = max(round(ctx_b / T),
// ceil(ctx_b / max_chunk)) chunks of ceil32(ctx_b / n_b) keys, so chunks of
// one sequence are equal and all chunks are close to T.  With alt_target_wg
// (the vector-ALU kernel's long chunks, about one per compute unit), when the
// longest chunk of that plan is more than 5/4 of the equal share the contexts
// are too uneven for one chunk per compute unit, whose longest chunk then sets
// the launch's time, and T comes from alt_target_wg instead (more, shorter
// chunks, which the dispatcher balances over the compute units).  With seq_chunk_cap,
// round(ctx_b / T) is first capped at it (fewer, longer chunks).  Fixed mode: chunks of
// fixed_chunk keys.  A sequence whose seq_pos breaks the contract has no
// chunks.  Work items (chunks) are laid out sequence-major: for b, for h, for c.

struct SeqChunks {
    int n;      // chunks of this sequence (0 if its seq_pos is out of range)
    int len;    // keys per chunk (the last may be shorter)
    int ctx;    // visible keys
};

// a / b for 0 <= a <= 2^22 and 1 <= b (every quotient of the chunk plan:
// contexts are at most 2^21 keys).  On the device the float quotient
// a * rcp(b) is within 0.75 of a / b at these sizes (rcp is within one ulp,
// the product within half an ulp: 1.5 * 2^-23 relative), so its truncation is
// the integer quotient or one off either way, and the remainder's sign and
// size correct it: about ten instructions where the generic division takes
// some thirty.  The chunk plan runs at the start of every workgroup, before
// its first cache load, so it is kept short and free of branches.
__host__ __device__ inline int div_small(int a, int b) {
#ifdef __HIP_DEVICE_COMPILE__
    int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
    const int r = a - q * b;
    return q + (r >= b) - (r < 0);
#else
    return a / b;
#endif
}
__host__ __device__ inline int ceil_small(int a, int b) { return div_small(a + b - 1, b); }
__host__ __device__ inline int round_up32(int a) { return (a + 31) & ~31; }
__host__ __device__ inline bool pow2(int a) { return a > 0 && (a & (a - 1)) == 0; }

__host__ __device__ inline bool seq_pos_ok(const AttnParams &p, int sp) {
    return sp >= 0 && sp <= p.max_seq - p.q_len;
}

// Balanced chunk length for `total` visible keys over all sequences and
// `target` chunks.
__host__ __device__ inline int balanced_len(const AttnParams &p, int64_t total, int target) {
    // ceil(total * Hkv / target) clamped to max_chunk, with a 32-bit division
    // whenever the clamp does not decide it (a 64-bit division is a long
    // instruction sequence on this GPU)
    const int64_t x = total * p.n_kv_heads;
    int t;
    if (x >= (int64_t)target * p.max_chunk)
        t = p.max_chunk;
    else if (__builtin_expect(pow2(target), 1))  // the automatic targets: a shift
        t = (int)((x + target - 1) >> __builtin_ctz((unsigned)target));
    else if (x + target <= (int64_t)0xffffffffu)
        t = (int)(((uint32_t)x + (uint32_t)target - 1u) / (uint32_t)target);
    else
        t = (int)((x + target - 1) / target);
    t = round_up32(t);
    return t < p.min_chunk ? p.min_chunk : (t > p.max_chunk ? p.max_chunk : t);
}

// Chunks of a sequence whose first new token sits at `sp`, for chunk length T
// (straight-line code: an out-of-range sp runs on a one-key context and is
// zeroed at the end).
__host__ __device__ inline SeqChunks seq_chunks_at(const AttnParams &p, int sp, int T) {
    const bool ok = seq_pos_ok(p, sp);
    const int ctx = ok ? sp + p.q_len : 1;
    int len;
    if (p.fixed_chunk > 0) {
        len = p.fixed_chunk;
    } else {
        int n = div_small(ctx + (T >> 1), T);  // round(ctx / T); T is a multiple of 32
        if (p.seq_chunk_cap > 0 && n > p.seq_chunk_cap) n = p.seq_chunk_cap;
        n = max(n, ceil_small(ctx, p.max_chunk));
        n = min(max(n, 1), p.n_chunks);
        const int raw = round_up32(ceil_small(ctx, n));
        const int a = p.chunk_align;
        len = a > 32 && 4 * raw >= 3 * a ? ceil_small(raw, a) * a : raw;
        len = min(len, p.max_chunk);  // raw <= max_chunk: no chunk is shorter than raw
    }
    // rounding the length up may leave the last chunk empty: n from the length
    return ok ? SeqChunks{ceil_small(ctx, len), len, ctx} : SeqChunks{0, 0, 0};
}

__host__ __device__ inline SeqChunks seq_chunks(const AttnParams &p, int b, int T) {
    return seq_chunks_at(p, p.seq_pos[b], T);
}

// True when the longest chunk of target_wg's plan (`longest` keys) exceeds 5/4
// of the equal share ceil(Hkv * total / target_wg): then alt_target_wg's plan
// is used.  Measured on the vector-ALU kernel's long chunks (batch 32, 8 KV
// heads, 8 layers, steps by eager launches, target_wg / alt_target_wg):
// contexts 7k-8k 1209 / 1222 us and 6k-8k 1159 / 1299 us (longest at most
// 1.14 share), 4k-8k 1084 / 966 us, 2k-8k 1053 / 977 us and 1k-8k 1014 / 824
// us (1.33 share and more); batch 16 MHA 16 heads at 4k-8k 1028 / 979 us;
// with two (sequence, KV head) pairs per compute unit, batch 64 at 2k-4k
// (longest 0.67 share), 1024 / 1064 us.
__host__ __device__ inline bool long_plan_uneven(const AttnParams &p, int64_t total, int longest) {
    return (int64_t)4 * longest * p.target_wg > (int64_t)5 * p.n_kv_heads * total;
}

__host__ __device__ inline int balanced_chunk(const AttnParams &p) {
    int64_t total = 0;
    for (int b = 0; b < p.batch; ++b) {
        const int sp = p.seq_pos[b];
        if (seq_pos_ok(p, sp)) total += sp + p.q_len;
    }
    const int T = balanced_len(p, total, p.target_wg);
    // no chunk exceeds max_chunk: when that is even, the plan stands unchecked
    if (p.alt_target_wg <= 0 || !long_plan_uneven(p, total, p.max_chunk)) return T;
    int longest = 0;
    for (int b = 0; b < p.batch; ++b) longest = max(longest, seq_chunks(p, b, T).len);
    return long_plan_uneven(p, total, longest) ? balanced_len(p, total, p.alt_target_wg) : T;
}

// Which (b, h, c) work item `w` is; false if w is past the last chunk, and then
// `w` is left as the item's index counted from the first item past the chunks.
__host__ __device__ inline bool locate(const AttnParams &p, int &w, int &b, int &h, int &c, SeqChunks &sc) {
    const int T = p.fixed_chunk > 0 ? p.fixed_chunk : balanced_chunk(p);
    for (b = 0; b < p.batch; ++b) {
        sc = seq_chunks(p, b, T);
        const int here = sc.n * p.n_kv_heads;
        if (w < here) {
            h = w / sc.n;
            c = w - h * sc.n;
            return true;
        }
        w -= here;
    }
    return false;
}

// Workspace carving, shared by the attention and the combine.
inline size_t ws_acc_floats(int32_t bh, int32_t n_chunks, int32_t rows, int32_t head_dim) {
    return (size_t)bh * n_chunks * rows * head_dim;
}
inline size_t ws_ml_floats(int32_t bh, int32_t n_chunks, int32_t rows) {
    return (size_t)bh * n_chunks * rows * 2;
}

// ---- host-side launch entry points (one per translation unit) ---------------

hipError_t launch_kv_append(const AppendParams &p, int threads_total, bool fp16, hipStream_t s);
hipError_t launch_fill_zero(int32_t *x, int n, hipStream_t s);
hipError_t launch_attn_valu(const AttnParams &p, int items, bool fp16, hipStream_t s);
hipError_t launch_attn_mfma(const AttnParams &p, int items, bool fp16, hipStream_t s);
hipError_t launch_attn_mfma256(const AttnParams &p, int items, bool fp16, hipStream_t s);
hipError_t launch_attn_combine(const AttnParams &p, bool fp16, void *out, hipStream_t s);

// ---- device helpers --------------------------------------------------------

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte global load of a read-only stream.
__device__ __forceinline__ u32x4_t ld16(const uint8_t *p) {
    return *reinterpret_cast<const u32x4_t *>(p);
}

// 16-byte load of the bulk K/V cache stream (whole tiles and slabs), which a
// launch reads exactly once: a non-temporal load (`global_load_dwordx4 ... nt`),
// so the stream neither allocates in nor evicts from the caches on its way.  On
// gfx950 a plain 2 GiB read streams at 6.0-6.2 TB/s and a non-temporal one at
// 6.9-7.2 TB/s (same lanes and depths); on the attention kernels it took the
// one-launch layer of batch 32, 16:8 heads at 8192 keys from 179.8 to 161.8 us
// and GQA-8 long context's attention launch from 43.8 to 41.1 us.  The per-row
// loads (partial tiles, new rows) and the query rows keep plain loads: with
// every load non-temporal the 512-context layer lost 0.6 us.
__device__ __forceinline__ u32x4_t ld16_stream(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

// fp32 sum of a.lo*b.lo + a.hi*b.hi + c over packed 16-bit pairs.
template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The two 16-bit elements of a packed pair as fp32 (exact).
template <bool F16>
__device__ __forceinline__ void unpack2(uint32_t x, float &lo, float &hi) {
    if constexpr (F16) {
        f16x2_t h = __builtin_bit_cast(f16x2_t, x);
        lo = (float)h.x;
        hi = (float)h.y;
    } else {
        lo = __uint_as_float(x << 16);
        hi = __uint_as_float(x & 0xffff0000u);
    }
}

// Whether either 16-bit element of a packed pair is inf or NaN (all exponent
// bits set).
template <bool F16>
__device__ __forceinline__ bool nonfinite2(uint32_t x) {
    constexpr uint32_t e = F16 ? 0x7c00u : 0x7f80u;
    return (x & e) == e || ((x >> 16) & e) == e;
}

// fp32 -> 16-bit element, round to nearest even.
template <bool F16>
__device__ __forceinline__ uint16_t round16(float x) {
    if constexpr (F16)
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    else
        return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// fp32 value rounded to the 16-bit type (nearest even) and widened back, exactly.
template <bool F16>
__device__ __forceinline__ float round_trip16(float x) {
    if constexpr (F16)
        return (float)(_Float16)x;
    else
        return __uint_as_float((uint32_t)round16<false>(x) << 16);
}

// ---- rotary embedding ("Qwen MoE BringUp", Per-Layer IR Patterns, RoPE) -----
// A row at position pos rotates each pair (x at dim j, y at dim j + D/2) by the
// angle a_j = pos * freqs[j], formed as a float32 product like the page's f32
// MatMul:  x' = x cos a - y sin a,  y' = y cos a + x sin a, in fp32 with one
// rounding back to 16 bits.  The angle is reduced in double precision to a
// fraction of a turn, a / 2pi - rint(a / 2pi) (exact to about 1e-10 turns for
// the largest positions), and the hardware sine and cosine take that fraction
// (v_sin_f32 / v_cos_f32 work in turns).
__device__ __forceinline__ void rope_pair(float &x, float &y, int pos, float freq) {
    const float a = __fmul_rn((float)pos, freq);
    const double turns = (double)a * 0.15915494309189533577;  // 1 / (2 pi)
    const float fr = (float)(turns - rint(turns));
    const float sn = __builtin_amdgcn_sinf(fr);
    const float cs = __builtin_amdgcn_cosf(fr);
    const float nx = fmaf(x, cs, -(y * sn));
    const float ny = fmaf(y, cs, x * sn);
    x = nx;
    y = ny;
}

// Rotates eight pairs held as 16-bit elements: `lo` holds dims j0 .. j0+7, `hi`
// dims j0+64 .. j0+71 (head_dim 128).
// rope8_with takes the eight frequencies already loaded (f0, f1 = freqs[j0 ..
// j0+7]), so a caller can issue their loads early.
template <bool F16>
__device__ __forceinline__ void rope8_with(u32x4_t &lo, u32x4_t &hi, int pos, f32x4_t f0, f32x4_t f1) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float x0, x1, y0, y1;
        unpack2<F16>(lo[w], x0, x1);
        unpack2<F16>(hi[w], y0, y1);
        const float fa = w < 2 ? f0[2 * w] : f1[2 * w - 4];
        const float fb = w < 2 ? f0[2 * w + 1] : f1[2 * w - 3];
        rope_pair(x0, y0, pos, fa);
        rope_pair(x1, y1, pos, fb);
        lo[w] = (uint32_t)round16<F16>(x0) | ((uint32_t)round16<F16>(x1) << 16);
        hi[w] = (uint32_t)round16<F16>(y0) | ((uint32_t)round16<F16>(y1) << 16);
        // one word at a time: interleaving all eight pairs' double-precision
        // reductions costs registers the callers' tiles need
        __builtin_amdgcn_sched_barrier(0);
    }
}
template <bool F16>
__device__ __forceinline__ void rope8(u32x4_t &lo, u32x4_t &hi, int pos, const float *freqs, int j0) {
    rope8_with<F16>(lo, hi, pos, *reinterpret_cast<const f32x4_t *>(freqs + j0),
                    *reinterpret_cast<const f32x4_t *>(freqs + j0 + 4));
}

// The same when consecutive lanes hold one row, 16 bytes (dims 8c .. 8c+7) each,
// and the first R dims rotate (R = 64, 128 or 256): piece c < R/8 pairs with
// piece c ^ (R/16), which is lane c ^ (R/16) of the row's lanes.  Every lane of
// the wave must call it (it shuffles); `apply` says whether this lane's piece
// is rotated.
template <bool F16>
__device__ __forceinline__ void rope_row(u32x4_t &piece, int c, int R, int pos, const float *freqs, bool apply) {
    const int hl = R / 16;
    u32x4_t other;
#pragma unroll
    for (int w = 0; w < 4; ++w) other[w] = (uint32_t)__shfl_xor((int)piece[w], hl);
    if (!apply || c >= R / 8) return;
    if (c < hl) {
        rope8<F16>(piece, other, pos, freqs, 8 * c);
    } else {
        rope8<F16>(other, piece, pos, freqs, 8 * (c - hl));
    }
}

// Sum over the 16 lanes of a DPP row (each lane gets the total).
__device__ __forceinline__ float row16_sum(float x) {
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

// x combined with lane l ^ 16 (xor16) or l ^ 32 (xor32) through gfx950's VALU
// lane swaps instead of LDS permutes.  v_permlane16_swap exchanges the odd
// 16-lane rows of its first register with the even rows of its second, and
// v_permlane32_swap the upper half of the first with the lower half of the
// second; with x in both, every lane ends up with its pair's two values, the
// lower lane's first, so both lanes compute the same bits.  The instructions
// are written out: this compiler folds the builtins' two results into one
// (as if the swap were lane-local), which loses the partner's value.  The
// s_nop before each gives the swap the wait states the compiler puts after a
// VALU write of its operands.
template <class Op>
__device__ __forceinline__ float xor16(float x, Op op) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
template <class Op>
__device__ __forceinline__ float xor32(float x, Op op) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
struct FMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct FAdd {
    __device__ float operator()(float a, float b) const { return a + b; }
};

// Over all 64 lanes (every lane gets the result): the 16-lane rows by DPP, then
// the rows by lane swaps.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)));
    return xor32(xor16(x, FMax{}), FMax{});
}
__device__ __forceinline__ float wave_sum(float x) { return xor32(xor16(row16_sum(x), FAdd{}), FAdd{}); }

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS round
// trips): shifts by 1, 2, 4 and 8 lanes within each 16-lane row (lanes shifted
// in from outside the row add 0), then lane 15's row total broadcast into rows
// 1 and 3 and lane 31's into rows 2 and 3.  These run at the start of every
// workgroup, before its first cache load.
__device__ __forceinline__ int wave_incl_scan(int x, int /*lane*/) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
    return __builtin_amdgcn_readlane(wave_incl_scan(x, 0), 63);
}

// Lane j's position for the chunk plan, sequence min(j, batch - 1): the first
// memory access of the attention and combine kernels, issued from the preloaded arguments
// with nothing to wait for.  locate_wave takes it raw and masks the lanes past
// the batch where it first uses it.
__device__ __forceinline__ int first_seq_pos(const int32_t *__restrict__ seq_pos, int batch, int lane) {
    return seq_pos[min(lane, batch - 1)];
}

// The chunk plan's per-launch values, computed by a whole wave: lane j of each
// pass holds sequence (pass + j), so the positions arrive in one vector load
// per 64 sequences instead of a chain of dependent scalar loads (every wave of
// the launch reads them while the cache streams, and a serial chain there costs
// microseconds).  Same results as balanced_chunk / locate.  `sp_first` is
// first_seq_pos()'s value for this lane (the first 64 sequences).
__device__ inline int balanced_chunk_wave(const AttnParams &p, const int32_t *__restrict__ seq_pos, int batch,
                                          int sp_first, int lane) {
    const int sp0 = lane < batch ? sp_first : -1;  // the first 64 sequences
    int64_t total = wave_sum_i(seq_pos_ok(p, sp0) ? sp0 + p.q_len : 0);
#pragma unroll 1
    for (int b0 = 64; __builtin_expect(b0 < batch, 0); b0 += 64) {
        const int b = b0 + lane;
        const int sp = b < batch ? seq_pos[b] : -1;
        total += wave_sum_i(seq_pos_ok(p, sp) ? sp + p.q_len : 0);
    }
    const int T = balanced_len(p, total, p.target_wg);
    // no chunk exceeds max_chunk: when that is even, the plan stands unchecked
    // (8192-key contexts on 8 KV heads of 32 sequences: no pass over the sequences)
    if (p.alt_target_wg <= 0 || !long_plan_uneven(p, total, p.max_chunk)) return T;
    // the longest chunk of that plan (lengths are at most 2^14: exact as floats)
    float longest = wave_max((float)seq_chunks_at(p, sp0, T).len);
#pragma unroll 1
    for (int b0 = 64; __builtin_expect(b0 < batch, 0); b0 += 64) {
        const int b = b0 + lane;
        longest = fmaxf(longest, wave_max((float)seq_chunks_at(p, b < batch ? seq_pos[b] : -1, T).len));
    }
    return long_plan_uneven(p, total, (int)longest) ? balanced_len(p, total, p.alt_target_wg) : T;
}

// locate() by a whole wave; also returns the sequence's seq_pos.  Every lane
// gets the same (uniform) results.  `seq_pos` and `batch` are p's, passed as
// the kernel's leading arguments: scalar arguments there are preloaded into
// registers when the wave starts, so the positions' load is issued before the
// parameter block's scalar loads return.  The loops run once per 64 sequences and
// are not unrolled: one copy of the chunk arithmetic.
__device__ inline bool locate_wave(const AttnParams &p, const int32_t *__restrict__ seq_pos, int batch,
                                   int sp_first, int &w, int &b, int &h, int &c, SeqChunks &sc, int &sp, int lane) {
    const int sp0 = lane < batch ? sp_first : -1;  // the first 64 sequences
    const int T = p.fixed_chunk > 0 ? p.fixed_chunk : balanced_chunk_wave(p, seq_pos, batch, sp_first, lane);
    // lane j holds sequence b0 + j, which has `here` items; the item is in the
    // sequence where the inclusive count first passes w
#pragma unroll 1
    for (int b0 = 0; b0 < batch; b0 += 64) {
        const int bb = b0 + lane;
        const int s1 = b0 == 0 ? sp0 : (bb < batch ? seq_pos[bb] : -1);
        const SeqChunks s = seq_chunks_at(p, s1, T);
        const int here = s.n * p.n_kv_heads;
        const int incl = wave_incl_scan(here, lane);
        const int tot = __builtin_amdgcn_readlane(incl, 63);
        if (w < tot) {
            const int L = __ffsll((unsigned long long)__ballot(incl > w)) - 1;
            w -= __builtin_amdgcn_readlane(incl - here, L);
            b = b0 + L;
            sc.n = __builtin_amdgcn_readlane(s.n, L);
            sc.len = __builtin_amdgcn_readlane(s.len, L);
            sc.ctx = __builtin_amdgcn_readlane(s.ctx, L);
            sp = __builtin_amdgcn_readlane(s1, L);
            h = w <= (1 << 22) ? div_small(w, sc.n) : w / sc.n;
            c = w - h * sc.n;
            return true;
        }
        w -= tot;
    }
    return false;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- partials shared across workgroups (the one-launch step's merge) ---------
//
// The merge of the one-launch step reads partials that workgroups on other
// XCDs wrote in the same launch, and each XCD has its own L2.  A release fence
// would write back the whole L2 after every partial (measured: it more than
// doubled the kernel's time), so instead:
//  - every partial is stored with a device-scope store, which writes through
//    the L2 to device-coherent memory;
//  - the storing wave waits until those stores are complete (vmcnt 0) before
//    it counts its arrival with a device-scope atomic add;
//  - the last arriver, which only gets there after every other arrival and so
//    after every other partial store completed, reads the partials with
//    device-scope loads, which fetch from device-coherent memory rather than
//    a possibly stale L2 line.

__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev4(float *p, float a, float b, float c, float d) {
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    __hip_atomic_store(q, (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)__float_as_uint(c) | ((uint64_t)__float_as_uint(d) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory access this wave issued is complete; also a compiler
// barrier, so no access moves across it.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Log-sum-exp merge state of one query row over some chunks: running maximum m
// (log2 units), sum l = sum_c 2^(m_c - m) l_c and this lane's D/64 dims of
// sum_c 2^(m_c - m) acc_c.
template <int D>
struct MergeState {
    static constexpr int NV = D / 64;
    float m, l, a[NV];
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int NV>
__device__ __forceinline__ void buffer_load_dims(float (&out)[NV], __amdgpu_buffer_rsrc_t r, int voff, uint32_t soff) {
    constexpr int kDevScope = 16;  // cache policy of the buffer loads: device scope
    if constexpr (NV == 2) {
        const f32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kDevScope);
        out[0] = x.x;
        out[1] = x.y;
    } else {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kDevScope);
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = __uint_as_float(x[k]);
    }
}

// Merge of chunks [c_lo, c_hi) of partial row `part` (= (b * Hkv + h) *
// n_chunks * rows + r) by one wave; lane j takes dims NV*j .. NV*j + NV-1.
//  - Per group of up to 64 chunks, lane k loads chunk k's (m, l): one
//    wave-wide max and sum give the group's weights w_k = 2^(m_k - M) and
//    sum of w_k l_k at once.
//  - The value rows are read sixteen chunks at a time with buffer loads that
//    share one lane offset and take the chunk offset from a scalar register
//    (no address registers per load), the first sixteen already in flight
//    while (m, l) are reduced.  Each is weighted by w_k, read from lane k.
// A chunk the row saw no key of (m_k = -inf) has weight 0.  Every load is
// device-scope (the partials may come from other XCDs in the same launch).
template <int D>
__device__ inline MergeState<D> merge_range(const AttnParams &p, size_t part, int c_lo, int c_hi, int lane) {
    constexpr int NV = D / 64;
    const float *ml = p.ws_ml + part * 2;
    const uint32_t cs_ml = (uint32_t)p.rows * 2;      // floats between chunks
    const uint32_t cs_acc = (uint32_t)p.rows * D * 4;  // bytes between chunks
    const __amdgpu_buffer_rsrc_t acc =
        __builtin_amdgcn_make_buffer_rsrc(p.ws_acc + part * D, 0, (int)(cs_acc * (uint32_t)p.n_chunks), 0x00020000);
    const int voff = lane * NV * 4;
    MergeState<D> s;
    s.m = -INFINITY;
    s.l = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) s.a[k] = 0.f;
    for (int g = c_lo; g < c_hi; g += 64) {
        const int cnt = min(64, c_hi - g);
        float m = -INFINITY, l = 0.f;
        if (lane < cnt) {
            m = ld_dev(ml + (size_t)(g + lane) * cs_ml);
            l = ld_dev(ml + (size_t)(g + lane) * cs_ml + 1);
        }
        float v[16][NV];
        auto load_batch = [&](int j) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (j + u < cnt) {
                    buffer_load_dims<NV>(v[u], acc, voff, (g + j + u) * cs_acc);
                } else {
#pragma unroll
                    for (int k = 0; k < NV; ++k) v[u][k] = 0.f;
                }
            }
        };
        load_batch(0);
        const float M = fmaxf(s.m, wave_max(m));
        if (M == -INFINITY) continue;
        const float f = s.m == -INFINITY ? 0.f : exp2_fast(s.m - M);
        const float w = m == -INFINITY ? 0.f : exp2_fast(m - M);
        s.l = fmaf(s.l, f, wave_sum(w * l));
#pragma unroll
        for (int k = 0; k < NV; ++k) s.a[k] *= f;
        s.m = M;
        for (int j = 0;;) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (j + u < cnt) {
                    const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j + u));
#pragma unroll
                    for (int k = 0; k < NV; ++k) s.a[k] = fmaf(wu, v[u][k], s.a[k]);
                }
            }
            j += 16;
            if (j >= cnt) break;
            load_batch(j);
        }
    }
    return s;
}

// Element offset of output row r of (b, h) (query token i, query head h*G + g).
__device__ __forceinline__ size_t out_row_off(const AttnParams &p, int b, int h, int r) {
    const int i = r / p.group, g = r - i * p.group;
    return (((size_t)b * p.q_len + i) * p.n_q_heads + (size_t)h * p.group + g) * p.head_dim;
}

// sigmoid(g) of a 16-bit gate element, fp32: 1 / (1 + 2^(-g log2 e)).
template <bool F16>
__device__ __forceinline__ float sigmoid16(uint16_t g) {
    float x, unused;
    unpack2<F16>((uint32_t)g, x, unused);
    return 1.f / (1.f + exp2_fast(-x * 1.4426950408889634f));
}

// Stores NV consecutive output values at element offset `off`, times the
// sigmoid output gate when the problem has one ("Architecture Diagram -
// Qwen3.5-35B-A3B", full-SDPA layers), rounded to nearest even.
template <bool F16, int NV>
__device__ __forceinline__ void store_out(const AttnParams &p, uint16_t *out, size_t off, const float (&x)[NV]) {
    float y[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) y[k] = x[k];
    if (p.out_gate) {
#pragma unroll
        for (int k = 0; k < NV; ++k) y[k] *= sigmoid16<F16>(p.out_gate[off + k]);
    }
    uint32_t *o = reinterpret_cast<uint32_t *>(out + off);
#pragma unroll
    for (int k = 0; k < NV; k += 2) o[k / 2] = (uint32_t)round16<F16>(y[k]) | ((uint32_t)round16<F16>(y[k + 1]) << 16);
}

// Merge of query row r of (b, h) over its n chunks by one wave, written to out:
//     out = (sum_c 2^(m_c - M) acc_c) / (sum_c 2^(m_c - M) l_c),  M = max_c m_c,
// (times the output gate), rounded to nearest even.
template <bool F16, int D>
__device__ inline void merge_row_wave(const AttnParams &p, uint16_t *out, int bh, int b, int h, int r, int n,
                                      int lane) {
    constexpr int NV = D / 64;
    const MergeState<D> s = merge_range<D>(p, (size_t)bh * p.n_chunks * p.rows + r, 0, n, lane);
    float x[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) x[k] = s.a[k] / s.l;
    store_out<F16, NV>(p, out, out_row_off(p, b, h, r) + NV * lane, x);
}

// The raw 16-bit gate values of the NV (2 or 4) output elements at `off`, one
// 4- or 8-byte load (`off` is a multiple of NV and the gate is 16-byte aligned);
// zeros without a gate.  Kept raw so that the load joins the merge's other loads
// in flight: the sigmoid is taken after all of them are issued.
template <int NV>
__device__ __forceinline__ void gate_raw(const AttnParams &p, size_t off, uint32_t (&g)[NV / 2]) {
    static_assert(NV == 2 || NV == 4, "two or four output elements per lane");
#pragma unroll
    for (int k = 0; k < NV / 2; ++k) g[k] = 0u;
    if (p.out_gate) {
        if constexpr (NV == 2) {
            g[0] = *reinterpret_cast<const uint32_t *>(p.out_gate + off);
        } else {
            const u32x2_t x = *reinterpret_cast<const u32x2_t *>(p.out_gate + off);
            g[0] = x[0];
            g[1] = x[1];
        }
    }
}

// sigmoid(gate) of the NV output elements from their raw values (1 without a gate).
template <bool F16, int NV>
__device__ __forceinline__ void gate_factors(const AttnParams &p, const uint32_t (&graw)[NV / 2], float (&g)[NV]) {
#pragma unroll
    for (int k = 0; k < NV; ++k) g[k] = 1.f;
    if (p.out_gate) {
#pragma unroll
        for (int k = 0; k < NV; ++k) g[k] = sigmoid16<F16>((uint16_t)(graw[k / 2] >> (16 * (k & 1))));
    }
}

// Merge of query rows r0 and r0 + r_step (when below p.rows) of (b, h) over their
// n <= 16 chunks by one wave, with every load of both rows in flight at once:
// the (m, l) pairs, the partial sums and the gate.  Same arithmetic as
// merge_row_wave.  (With the gate's sigmoid taken as each row's loads were
// issued, the wait for the first row's gate also waited for its partial sums
// before the second row's loads went out: the head_dim-256 merge took two
// round trips.)
template <bool F16, int D>
__device__ inline void merge_two_rows_wave(const AttnParams &p, int bh, int b, int h, int r0, int r_step, int n,
                                           int lane) {
    constexpr int NV = D / 64;
    const int r1 = r0 + r_step < p.rows ? r0 + r_step : r0;  // a missing second row repeats the first
    const uint32_t cs_ml = (uint32_t)p.rows * 2;
    const uint32_t cs_acc = (uint32_t)p.rows * D * 4;
    const int voff = lane * NV * 4;
    float m[2], l[2], v[2][16][NV];
    uint32_t graw[2][NV / 2];
    size_t off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = j ? r1 : r0;
        const size_t part = (size_t)bh * p.n_chunks * p.rows + r;
        m[j] = -INFINITY;
        l[j] = 0.f;
        if (lane < n) {
            m[j] = ld_dev(p.ws_ml + part * 2 + (size_t)lane * cs_ml);
            l[j] = ld_dev(p.ws_ml + part * 2 + (size_t)lane * cs_ml + 1);
        }
        const __amdgpu_buffer_rsrc_t acc =
            __builtin_amdgcn_make_buffer_rsrc(p.ws_acc + part * D, 0, (int)(cs_acc * (uint32_t)p.n_chunks), 0x00020000);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (u < n) {
                buffer_load_dims<NV>(v[j][u], acc, voff, u * cs_acc);
            } else {
#pragma unroll
                for (int k = 0; k < NV; ++k) v[j][u][k] = 0.f;
            }
        }
        off[j] = out_row_off(p, b, h, r) + NV * lane;
        gate_raw<NV>(p, off[j], graw[j]);
    }
    float g[2][NV];
#pragma unroll
    for (int j = 0; j < 2; ++j) gate_factors<F16, NV>(p, graw[j], g[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j == 1 && r1 == r0) break;
        const float M = wave_max(m[j]);
        const float w = m[j] == -INFINITY ? 0.f : exp2_fast(m[j] - M);
        const float L = wave_sum(w * l[j]);
        float a[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) a[k] = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (u < n) {
                const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
                for (int k = 0; k < NV; ++k) a[k] = fmaf(wu, v[j][u][k], a[k]);
            }
        }
        uint32_t *o = reinterpret_cast<uint32_t *>(p.out + off[j]);
#pragma unroll
        for (int k = 0; k < NV; k += 2)
            o[k / 2] = (uint32_t)round16<F16>(a[k] / L * g[j][k]) | ((uint32_t)round16<F16>(a[k + 1] / L * g[j][k + 1]) << 16);
    }
}

// One-launch step: the output rows of sequence b, whose seq_pos breaks the
// contract (it has no chunks), are flagged with NaN, as the separate combine
// does.  Written by `n_lanes` lanes starting at `lane`.
template <bool F16>
__device__ inline void flag_sequence_nan(const AttnParams &p, int b, int lane, int n_lanes) {
    const uint32_t nan16 = F16 ? 0x7e00u : 0x7fc0u;
    uint32_t *o = reinterpret_cast<uint32_t *>(p.out + (size_t)b * p.q_len * p.n_q_heads * p.head_dim);
    const int words = p.q_len * p.n_q_heads * (p.head_dim / 2);
    for (int x = lane; x < words; x += n_lanes) o[x] = nan16 | (nan16 << 16);
}

}  // namespace da
