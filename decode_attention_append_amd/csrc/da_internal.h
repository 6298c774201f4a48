// Internal declarations shared by the HIP translation units of libdecode_attn.
// Device helpers for gfx950 (CDNA4, wave64) and the parameter blocks the host
// launcher hands to each kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr int kHeadDim = 128;     // the only head_dim implemented
constexpr int kRowBytes = kHeadDim * 2;
constexpr int kMaxRows = 32;      // (Hq/Hkv) * q_len limit
constexpr int kMaxQLen = 8;
constexpr int kTokenTile = 64;    // chunk sizes are multiples of this
constexpr int kMaxChunk = 2048;

// ---- parameter blocks ------------------------------------------------------

struct AppendParams {
    uint8_t *k_cache;
    uint8_t *v_cache;
    const uint8_t *k_new;
    const uint8_t *v_new;
    const int32_t *seq_pos;
    int32_t batch, q_len, n_kv_heads, max_seq;
};

struct AttnParams {
    const uint8_t *q;
    const uint8_t *k_cache;
    const uint8_t *v_cache;
    const int32_t *seq_pos;
    float *ws_acc;  // [B*Hkv][n_chunks][rows][D] unnormalised weighted V sums
    float *ws_ml;   // [B*Hkv][n_chunks][rows][2]  (running max in log2 units, sum)
    int32_t batch, q_len, n_q_heads, n_kv_heads, max_seq;
    int32_t group;  // Hq / Hkv
    int32_t rows;   // group * q_len
    int32_t n_chunks;      // chunk slots per (sequence, KV head) in the workspace
    int32_t fixed_chunk;   // > 0: every chunk has this many keys; 0: balanced chunks
    int32_t target_wg;     // balanced: chunks to aim for over the whole launch
    int32_t min_chunk;     // balanced: smallest chunk (multiple of 32)
    int32_t max_chunk;     // largest chunk the kernel accepts (multiple of 32)
    float scale_log2;      // softmax scale * log2(e): scores are kept in log2 units
};

// ---- split-context chunk plan, computed identically by every kernel ---------
//
// Balanced mode: the chunk length aims at an equal share of all visible keys
// per chunk, T = ceil32(Hkv * sum_b ctx_b / target_wg) clamped to
// [min_chunk, max_chunk]; sequence b gets n_b = max(round(ctx_b / T),
// ceil(ctx_b / max_chunk)) chunks of ceil32(ctx_b / n_b) keys, so chunks of
// one sequence are equal and all chunks are close to T.  Fixed mode: chunks of
// fixed_chunk keys.  A sequence whose seq_pos breaks the contract has no
// chunks.  Work items (chunks) are laid out sequence-major: for b, for h, for c.

struct SeqChunks {
    int n;      // chunks of this sequence (0 if its seq_pos is out of range)
    int len;    // keys per chunk (the last may be shorter)
    int ctx;    // visible keys
};

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int round_up32(int a) { return (a + 31) & ~31; }

__host__ __device__ inline bool seq_pos_ok(const AttnParams &p, int sp) {
    return sp >= 0 && sp <= p.max_seq - p.q_len;
}

__host__ __device__ inline int balanced_chunk(const AttnParams &p) {
    int64_t total = 0;
    for (int b = 0; b < p.batch; ++b) {
        const int sp = p.seq_pos[b];
        if (seq_pos_ok(p, sp)) total += sp + p.q_len;
    }
    const int64_t want = (total * p.n_kv_heads + p.target_wg - 1) / p.target_wg;
    int t = (int)(want < p.max_chunk ? want : p.max_chunk);
    t = round_up32(t);
    return t < p.min_chunk ? p.min_chunk : (t > p.max_chunk ? p.max_chunk : t);
}

__host__ __device__ inline SeqChunks seq_chunks(const AttnParams &p, int b, int T) {
    SeqChunks s{0, 0, 0};
    const int sp = p.seq_pos[b];
    if (!seq_pos_ok(p, sp)) return s;
    s.ctx = sp + p.q_len;
    if (p.fixed_chunk > 0) {
        s.len = p.fixed_chunk;
        s.n = ceil_div(s.ctx, s.len);
        return s;
    }
    int n = (2 * s.ctx + T) / (2 * T);  // round(ctx / T)
    const int n_cap = ceil_div(s.ctx, p.max_chunk);
    if (n < n_cap) n = n_cap;
    if (n < 1) n = 1;
    if (n > p.n_chunks) n = p.n_chunks;
    s.n = n;
    s.len = round_up32(ceil_div(s.ctx, n));
    s.n = ceil_div(s.ctx, s.len);  // rounding the length up may leave the last chunk empty
    return s;
}

// Which (b, h, c) work item `w` is; false if w is past the last chunk.
__host__ __device__ inline bool locate(const AttnParams &p, int w, int &b, int &h, int &c, SeqChunks &sc) {
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
inline size_t ws_acc_floats(int32_t bh, int32_t n_chunks, int32_t rows) {
    return (size_t)bh * n_chunks * rows * kHeadDim;
}
inline size_t ws_ml_floats(int32_t bh, int32_t n_chunks, int32_t rows) {
    return (size_t)bh * n_chunks * rows * 2;
}

// ---- host-side launch entry points (one per translation unit) ---------------

hipError_t launch_kv_append(const AppendParams &p, int threads_total, hipStream_t s);
hipError_t launch_attn_valu(const AttnParams &p, int items, bool fp16, hipStream_t s);
hipError_t launch_attn_mfma(const AttnParams &p, int items, bool fp16, hipStream_t s);
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
__device__ __forceinline__ u32x2_t ld8(const uint8_t *p) {
    return *reinterpret_cast<const u32x2_t *>(p);
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

// Sum over the 16 lanes of a DPP row (each lane gets the total).
__device__ __forceinline__ float row16_sum(float x) {
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace da
