/*
 * Reference oracle for one decode step of grouped-query attention with a
 * KV-cache append.  TEST INFRASTRUCTURE ONLY: the product path never links,
 * loads or calls this file.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may use it.
 *
 * It is a plain, slow, double-precision restatement of what the pages define,
 * written so a reader can check it against them by eye:
 *
 *  - "Qwen MoE BringUp" (iree-org/onnxruntime-ep-iree issue 34), section
 *    "Per-Layer IR Patterns", 2. Self-Attention, "KV Cache Update (EP rewrite:
 *    tensor.insert_slice)": the new K/V rows of a step are written into the
 *    pre-allocated cache as one contiguous slice whose start on the sequence
 *    axis is seq_position; nothing else in the cache changes.  Fix A5 of the
 *    same page explains that the scatter with sequential indices is exactly
 *    such a slice write.
 *  - same page and section, "Attention Computation": scores = Q K^T, times
 *    1/sqrt(128); a key at position j is visible to the query token at
 *    position t when j <= t and j < seq_end (the LessOrEqual / Less / And
 *    mask, invisible keys get -inf); softmax over the key axis; the output is
 *    the softmax weights times V.
 *  - grouped query heads: consecutive query heads share one KV head
 *    (kv_head = q_head / (Hq/Hkv)); the pages only say GQA is handled inside
 *    the kernel ("Architecture Diagram - Qwen3-30B-A3B (Extern Dispatch)",
 *    Paged Attention block) and that K/V heads are broadcast 4 -> 32 on the
 *    native path; repeat-interleave is the plainest reading of both.
 *  - all arithmetic in double precision (the pages ask for fp32
 *    accumulation at least: fix A7 of "Qwen MoE BringUp", and BP-3 of
 *    "Design: Execution Provider aware model building").
 *
 * Layouts (all row-major, contiguous):
 *   q, out          [B][q_len][Hq][D]
 *   k_new, v_new    [B][q_len][Hkv][D]
 *   k_cache,v_cache [B][Hkv][S][D]      (S = allocated sequence length)
 *   seq_pos         [B]                 slot of the first new token
 * Elements of q / caches / new rows are 16-bit patterns (bf16 or fp16).
 *
 * Two passes, no chunking, no online rescaling: scores of all visible keys
 * first, then the maximum, then normalised weights, then the weighted sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_FP16 1

/* ---- element decoding, from the two formats' definitions ---------------- */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 7) & 0xff;
    int frac = bits & 0x7f;
    double mag;
    if (expo == 0xff)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, -126 - 7);           /* subnormal */
    else
        mag = ldexp(1.0 + frac / 128.0, expo - 127);
    return sign ? -mag : mag;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_fp16(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0x1f)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, -14 - 10);           /* subnormal */
    else
        mag = ldexp(1.0 + frac / 1024.0, expo - 15);
    return sign ? -mag : mag;
}

static double decode(int dtype, uint16_t bits)
{
    return dtype == ORACLE_FP16 ? oracle_decode_fp16(bits) : oracle_decode_bf16(bits);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- KV append -------------------------------------------------------------
 * cache[b][h][seq_pos[b] + i][:] = new[b][i][h][:]  for i < q_len, bit for bit.
 * Returns -1 (and writes nothing) if some slice would fall outside [0, S).
 */
int oracle_kv_append(int32_t B, int32_t q_len, int32_t Hkv, int32_t D, int32_t S,
                     const int32_t *seq_pos,
                     const uint16_t *k_new, const uint16_t *v_new,
                     uint16_t *k_cache, uint16_t *v_cache)
{
    for (int32_t b = 0; b < B; ++b)
        if (seq_pos[b] < 0 || seq_pos[b] + q_len > S)
            return -1;
    for (int32_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < q_len; ++i)
            for (int32_t h = 0; h < Hkv; ++h) {
                size_t src = (((size_t)b * q_len + i) * Hkv + h) * D;
                size_t dst = (((size_t)b * Hkv + h) * S + (size_t)(seq_pos[b] + i)) * D;
                memcpy(k_cache + dst, k_new + src, (size_t)D * sizeof(uint16_t));
                memcpy(v_cache + dst, v_new + src, (size_t)D * sizeof(uint16_t));
            }
    return 0;
}

/* ---- attention for one query row ----------------------------------------
 * q_row:  D elements of one query head at one query token
 * k_head, v_head: the [S][D] cache slab of the KV head that query head uses
 * t:       position of the query token (seq_pos + i)
 * seq_end: seq_pos + q_len
 * out_row: D doubles; weights (optional): S doubles, 0 for invisible keys.
 * Returns the number of visible keys (0 means the row is undefined and out_row
 * is filled with NaN).
 */
int32_t oracle_attend_row(int32_t dtype, int32_t D, int32_t S, int32_t t, int32_t seq_end,
                          double scale, const uint16_t *q_row,
                          const uint16_t *k_head, const uint16_t *v_head,
                          double *out_row, double *weights)
{
    double *score = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double *qd = (double *)malloc(sizeof(double) * (size_t)D);
    char *visible = (char *)malloc((size_t)(S > 0 ? S : 1));
    int32_t n_visible = 0;

    for (int32_t d = 0; d < D; ++d)
        qd[d] = decode(dtype, q_row[d]);

    /* pass 1: scaled dot products of the visible keys, and their maximum */
    double m = -INFINITY;
    for (int32_t j = 0; j < S; ++j) {
        visible[j] = (j <= t) && (j < seq_end);
        if (!visible[j])
            continue;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
            dot += qd[d] * decode(dtype, k_head[(size_t)j * D + d]);
        score[j] = dot * scale;
        if (score[j] > m)
            m = score[j];
        ++n_visible;
    }

    /* pass 2: softmax weights over the visible keys */
    double denom = 0.0;
    for (int32_t j = 0; j < S; ++j)
        if (visible[j]) {
            score[j] = exp(score[j] - m);
            denom += score[j];
        }
    for (int32_t j = 0; j < S; ++j)
        score[j] = visible[j] ? score[j] / denom : 0.0;

    /* pass 3: weighted sum of the value rows */
    for (int32_t d = 0; d < D; ++d)
        out_row[d] = n_visible ? 0.0 : NAN;
    for (int32_t j = 0; j < S; ++j) {
        if (!visible[j])
            continue;
        for (int32_t d = 0; d < D; ++d)
            out_row[d] += score[j] * decode(dtype, v_head[(size_t)j * D + d]);
    }
    if (weights)
        memcpy(weights, score, sizeof(double) * (size_t)S);

    free(score);
    free(qd);
    free(visible);
    return n_visible;
}

/* ---- one query row of the whole problem ---------------------------------- */
static int32_t attend_bih(int32_t dtype, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t S, double scale, const int32_t *seq_pos,
                          const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                          int32_t b, int32_t i, int32_t hq, double *out_row, double *weights)
{
    int32_t group = Hq / Hkv;
    int32_t h = hq / group; /* consecutive query heads share a KV head */
    const uint16_t *q_row = q + (((size_t)b * q_len + i) * Hq + hq) * D;
    const uint16_t *k_head = k_cache + ((size_t)b * Hkv + h) * (size_t)S * D;
    const uint16_t *v_head = v_cache + ((size_t)b * Hkv + h) * (size_t)S * D;
    return oracle_attend_row(dtype, D, S, seq_pos[b] + i, seq_pos[b] + q_len, scale,
                             q_row, k_head, v_head, out_row, weights);
}

static int check_problem(int32_t dtype, int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t S, const int32_t *seq_pos)
{
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16)
        return -1;
    if (B <= 0 || q_len <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S <= 0 || Hq % Hkv != 0)
        return -1;
    for (int32_t b = 0; b < B; ++b)
        if (seq_pos[b] < 0 || seq_pos[b] + q_len > S)
            return -1;
    return 0;
}

/* ---- the whole attention problem -----------------------------------------
 * out: [B][q_len][Hq][D] doubles.  weights (optional): [B][q_len][Hq][S].
 * The caches must already hold the appended rows.  Returns 0, or -1 on a bad
 * problem description.
 */
int oracle_gqa_decode(int32_t dtype, int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv,
                      int32_t D, int32_t S, double scale, const int32_t *seq_pos,
                      const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                      double *out, double *weights)
{
    if (check_problem(dtype, B, q_len, Hq, Hkv, D, S, seq_pos))
        return -1;
    int64_t n_rows = (int64_t)B * q_len * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int32_t hq = (int32_t)(r % Hq);
        int32_t i = (int32_t)((r / Hq) % q_len);
        int32_t b = (int32_t)(r / ((int64_t)Hq * q_len));
        attend_bih(dtype, q_len, Hq, Hkv, D, S, scale, seq_pos, q, k_cache, v_cache, b, i, hq,
                   out + (size_t)r * D, weights ? weights + (size_t)r * S : NULL);
    }
    return 0;
}

/* ---- selected rows of the attention problem ------------------------------
 * For full-size checks: computes only the rows (row_b[n], row_i[n], row_hq[n])
 * into out_rows[n][D].  Returns 0, or -1 on a bad description or row index.
 */
int oracle_gqa_decode_rows(int32_t dtype, int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t S, double scale, const int32_t *seq_pos,
                           const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                           int32_t n_rows, const int32_t *row_b, const int32_t *row_i,
                           const int32_t *row_hq, double *out_rows)
{
    if (check_problem(dtype, B, q_len, Hq, Hkv, D, S, seq_pos))
        return -1;
    for (int32_t n = 0; n < n_rows; ++n)
        if (row_b[n] < 0 || row_b[n] >= B || row_i[n] < 0 || row_i[n] >= q_len ||
            row_hq[n] < 0 || row_hq[n] >= Hq)
            return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t n = 0; n < n_rows; ++n)
        attend_bih(dtype, q_len, Hq, Hkv, D, S, scale, seq_pos, q, k_cache, v_cache,
                   row_b[n], row_i[n], row_hq[n], out_rows + (size_t)n * D, NULL);
    return 0;
}

/* ---- element encoding (round to nearest, ties to even), from the formats ---
 * A 16-bit format with `ebits` exponent bits (bias 2^(ebits-1) - 1) and
 * `mbits` fraction bits.  The value is rounded once, directly from double.
 * NaN becomes the quiet NaN with only the top fraction bit set; magnitudes
 * that round past the largest finite value become infinity.
 */
static uint16_t encode16(double x, int ebits, int mbits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const int emax_field = (1 << ebits) - 1;            /* all-ones exponent field */
    const uint16_t sign = signbit(x) ? (uint16_t)0x8000 : 0;
    const double ax = fabs(x);
    if (isnan(x))
        return (uint16_t)((emax_field << mbits) | (1 << (mbits - 1)));
    if (isinf(x))
        return (uint16_t)(sign | (emax_field << mbits));
    if (ax == 0.0)
        return sign;
    int e2;
    frexp(ax, &e2);                 /* ax = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                 /* ax in [2^e, 2^(e+1)) */
    const int emin = 1 - bias;      /* exponent of the smallest normal */
    if (e < emin)
        e = emin;                   /* subnormals share the smallest normal's quantum */
    const double quantum = ldexp(1.0, e - mbits);
    double n = nearbyint(ax / quantum);                 /* exact scaling, then RNE */
    if (n >= ldexp(1.0, mbits + 1)) {                   /* rounded up into the next binade */
        n /= 2.0;
        e += 1;
    }
    if (n < ldexp(1.0, mbits))                          /* subnormal (only when e == emin) */
        return (uint16_t)(sign | (uint16_t)n);
    const int field = e + bias;
    if (field >= emax_field)
        return (uint16_t)(sign | (emax_field << mbits));
    return (uint16_t)(sign | (field << mbits) | ((uint16_t)n - (1 << mbits)));
}

uint16_t oracle_encode_bf16(double x) { return encode16(x, 8, 7); }
uint16_t oracle_encode_fp16(double x) { return encode16(x, 5, 10); }

static uint16_t encode(int dtype, double x)
{
    return dtype == ORACLE_FP16 ? oracle_encode_fp16(x) : oracle_encode_bf16(x);
}

/* ---- rotary position embedding of rows ------------------------------------
 * "Qwen MoE BringUp", Per-Layer IR Patterns, 2. Self-Attention, "Rotary
 * Position Embeddings (RoPE)": a row at absolute position `pos` is rotated by
 * angles a_j = pos * freqs[j] (j < D/2), the product formed in single precision
 * as the page does (position cast to f32, then a f32 MatMul with the f32
 * frequency table); the table is doubled so dims j and j + D/2 share a_j; and
 *     out = x * cos(a) + rotate_half(x) * sin(a),  rotate_half(x) = [-x2, x1]
 * where x1, x2 are the two halves.  Per pair:
 *     out[j]       = x[j] cos a_j - x[j+D/2] sin a_j
 *     out[j+D/2]   = x[j+D/2] cos a_j + x[j] sin a_j.
 * cos, sin and the rotation are evaluated in double here and the result is
 * rounded once to the row's 16-bit format.
 *
 * Partial rotation ("Architecture Diagram - Qwen3.5-35B-A3B", full-SDPA layers:
 * partial RoPE over 25% of the dims): only the first R dims rotate, as above
 * with R in place of D (pairs j and j + R/2); dims R .. D-1 pass unchanged.
 *
 * rows: n rows of D 16-bit elements; pos: n positions; freqs: R/2 floats.
 */
int oracle_rope_rows(int32_t dtype, int32_t n, int32_t D, int32_t R, const int32_t *pos, const float *freqs,
                     const uint16_t *in, uint16_t *out)
{
    if (D <= 0 || R <= 0 || R > D || R % 2)
        return -1;
    const int32_t half = R / 2;
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < n; ++r) {
        const uint16_t *x = in + (size_t)r * D;
        uint16_t *y = out + (size_t)r * D;
        for (int32_t j = R; j < D; ++j)
            y[j] = x[j];
        for (int32_t j = 0; j < half; ++j) {
            /* the exact product of two floats fits a double; one rounding to float */
            const float a = (float)((double)(float)pos[r] * (double)freqs[j]);
            const double c = cos((double)a), s = sin((double)a);
            const double x1 = decode(dtype, x[j]), x2 = decode(dtype, x[j + half]);
            y[j] = encode(dtype, x1 * c - x2 * s);
            y[j + half] = encode(dtype, x2 * c + x1 * s);
        }
    }
    return 0;
}

/* ---- paged KV cache ----------------------------------------------------------
 * "Architecture Diagram - Qwen3-30B-A3B (Extern Dispatch, 75 tok/s)", Paged
 * Attention: the KV write goes to a page pool laid out [pages][KV heads][16
 * tokens per page][head dim].  A per-sequence block table (int32
 * [B][pages_per_seq]) names the pool page that holds logical page i of
 * sequence b, i.e. tokens 16 i .. 16 i + 15.  The sequence's cache is the
 * concatenation of its pages in block-table order; nothing else changes.
 *
 * gather: pool -> contiguous [B][Hkv][pages_per_seq * page_size][D].
 * append: writes new[b][i][h][:] into the pool slot of token seq_pos[b] + i.
 * Both return -1 (and write nothing) for a block-table entry outside the pool
 * or a position outside the sequence's pages.
 */
static int check_pages(int32_t B, int32_t pages_per_seq, int32_t n_pages, const int32_t *block_table)
{
    for (int64_t k = 0; k < (int64_t)B * pages_per_seq; ++k)
        if (block_table[k] < 0 || block_table[k] >= n_pages)
            return -1;
    return 0;
}

int oracle_gather_paged(int32_t B, int32_t Hkv, int32_t D, int32_t page_size, int32_t pages_per_seq,
                        int32_t n_pages, const int32_t *block_table, const uint16_t *pool, uint16_t *out)
{
    if (check_pages(B, pages_per_seq, n_pages, block_table))
        return -1;
    const int64_t S = (int64_t)pages_per_seq * page_size;
    for (int32_t b = 0; b < B; ++b)
        for (int32_t h = 0; h < Hkv; ++h)
            for (int64_t t = 0; t < S; ++t) {
                const int32_t page = block_table[(int64_t)b * pages_per_seq + t / page_size];
                const uint16_t *src = pool + (((int64_t)page * Hkv + h) * page_size + t % page_size) * D;
                uint16_t *dst = out + (((int64_t)b * Hkv + h) * S + t) * D;
                memcpy(dst, src, (size_t)D * sizeof(uint16_t));
            }
    return 0;
}

int oracle_kv_append_paged(int32_t B, int32_t q_len, int32_t Hkv, int32_t D, int32_t page_size,
                           int32_t pages_per_seq, int32_t n_pages, const int32_t *block_table,
                           const int32_t *seq_pos, const uint16_t *k_new, const uint16_t *v_new,
                           uint16_t *k_pool, uint16_t *v_pool)
{
    if (check_pages(B, pages_per_seq, n_pages, block_table))
        return -1;
    const int64_t S = (int64_t)pages_per_seq * page_size;
    for (int32_t b = 0; b < B; ++b)
        if (seq_pos[b] < 0 || seq_pos[b] + q_len > S)
            return -1;
    for (int32_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < q_len; ++i)
            for (int32_t h = 0; h < Hkv; ++h) {
                const int64_t t = (int64_t)seq_pos[b] + i;
                const int32_t page = block_table[(int64_t)b * pages_per_seq + t / page_size];
                const size_t row = (((size_t)b * q_len + i) * Hkv + h) * D;
                const size_t dst = (((size_t)page * Hkv + h) * page_size + (size_t)(t % page_size)) * D;
                memcpy(k_pool + dst, k_new + row, (size_t)D * sizeof(uint16_t));
                memcpy(v_pool + dst, v_new + row, (size_t)D * sizeof(uint16_t));
            }
    return 0;
}

/* ---- sigmoid output gate ------------------------------------------------------
 * "Qwen MoE BringUp", "Architecture Diagram - Qwen3.5-35B-A3B", full-SDPA
 * layers: the query projection also yields a gate ("Q(->8192)+gate" for 16
 * heads of 256 dims), and the attention output is multiplied elementwise by
 * sigmoid(gate) ("sigmoid gate") before the output projection.
 * out: n doubles (the attention output), multiplied in place by
 * 1 / (1 + exp(-g)) with g the decoded 16-bit gate element.
 */
void oracle_output_gate(int32_t dtype, int64_t n, const uint16_t *gate, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] *= 1.0 / (1.0 + exp(-decode(dtype, gate[i])));
}
