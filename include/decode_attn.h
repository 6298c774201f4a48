/*
 * decode_attn.h - one decode step of grouped-query attention over a KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The step, as the "Qwen MoE BringUp" page (iree-org/onnxruntime-ep-iree
 * issue 34) describes it:
 *
 *   1. da_kv_append: the new K/V rows of the step are written into the
 *      pre-allocated cache as one contiguous slice starting at the sequence's
 *      seq_position (section "Per-Layer IR Patterns", 2. Self-Attention,
 *      "KV Cache Update (EP rewrite: tensor.insert_slice)"; fix A5 explains why
 *      the scatter with sequential indices is such a slice write; opportunity
 *      10 keeps the cache a fixed-size buffer updated in place).
 *   2. da_gqa_decode_attn: split-context attention.  Scores Q K^T times the
 *      softmax scale, a causal mask (key j is visible to query token i iff
 *      j <= seq_pos + i, which also keeps j below seq_pos + q_len), softmax, times V
 *      (same page, "Attention Computation").  The context is cut into chunks;
 *      each chunk's fp32 online-softmax partial (max, sum, weighted V sum) goes
 *      to a caller-provided workspace.  One workgroup serves every query head
 *      of one KV head, so each K/V byte is read from memory once ("Architecture
 *      Diagram - Qwen3-30B-A3B (Extern Dispatch, 75 tok/s)": Paged Attention
 *      3-phase decode, split-KV phase, GQA handled in the kernel).
 *   3. da_gqa_decode_attn_combine: log-sum-exp merge of the chunk partials and
 *      the final normalisation, rounded to nearest-even into bf16/fp16 (same
 *      diagram, the reduce phase).
 *
 * All accumulation is fp32 (fix A7 of the same page; BP-3 of "Design:
 * Execution Provider aware model building").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except `p` is a DEVICE pointer, 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it, in call order; nothing here
 *    synchronises, allocates, frees, or reads device memory on the host.
 *  - The caller owns every buffer.  The library keeps no state between calls,
 *    except the scratch of da_decode_step_static (see there).
 *  - Layouts (row-major, contiguous, element = 2-byte bf16 or fp16):
 *        q, out          [B][q_len][Hq][D]
 *        k_new, v_new    [B][q_len][Hkv][D]
 *        k_cache,v_cache [B][Hkv][max_seq][D]
 *        seq_pos         int32 [B]: cache slot of the sequence's first new token
 *    Query head hq reads KV head hq / (Hq / Hkv) (consecutive query heads
 *    share a KV head).  Multi-head attention is Hq == Hkv.
 *  - Host-checkable errors are reported BEFORE anything is enqueued; on any
 *    error return nothing has been launched.  Device-side preconditions
 *    (0 <= seq_pos[b] and seq_pos[b] + q_len <= max_seq) cannot be checked on
 *    the host without a synchronisation: they are the caller's contract.  A
 *    sequence that breaks it is skipped by da_kv_append (its slice is not
 *    written) and its attention output is unspecified, but no kernel reads or
 *    writes outside the buffers described here.
 *  - No exceptions cross this interface.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DA_OK = 0,
    DA_ERR_INVALID_ARG = -1, /* null or misaligned pointer, non-positive size, Hq % Hkv != 0 */
    DA_ERR_UNSUPPORTED = -2, /* valid but not implemented: head_dim other than 128 / 256, q_len > 8, ... */
    DA_ERR_WORKSPACE = -3,   /* workspace smaller than da_workspace_bytes() */
    DA_ERR_HIP = -4,         /* the HIP runtime refused a launch */
    DA_ERR_SCRATCH_LIMIT = -5 /* da_decode_step_static: the problem needs more than its scratch */
} da_status;

typedef enum { DA_BF16 = 0, DA_FP16 = 1 } da_dtype;

/* Shape of one decode step.  Plain data, read only during the call. */
typedef struct {
    int32_t batch;        /* B >= 1, B * Hkv < 2^25                               */
    int32_t q_len;        /* new tokens per sequence this step, 1..8 (verify batches) */
    int32_t n_q_heads;    /* Hq >= 1                                              */
    int32_t n_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0, (Hq / Hkv) * q_len <= 32    */
    int32_t head_dim;     /* D: 128, or 256 (on the MFMA kernel)                  */
    int32_t max_seq;      /* allocated cache length (slots per KV head)           */
    int32_t dtype;        /* da_dtype of q, caches, new rows and out              */
    float scale;          /* softmax scale; <= 0 selects 1 / sqrt(head_dim)       */
    int32_t chunk_tokens; /* keys per split-context chunk: 0 = automatic, else a
                             multiple of 64 (a tuning and testing override)       */
    int32_t variant;      /* attention kernel: 0 = automatic, else DA_VARIANT_* + 1
                             (a tuning and testing override; the vector-ALU kernel
                             takes at most 16 rows per KV head)                   */
    int32_t work_items;   /* balanced chunking: chunks to aim for over the whole
                             launch, 0 = automatic (a tuning override)            */
    const float *rope_freqs; /* DEVICE pointer to head_dim/2 float32 rotary
                             frequencies (16-byte aligned), or NULL.  With a table,
                             the rotary embedding of the "Qwen MoE BringUp" page
                             (Per-Layer IR Patterns, 2. Self-Attention, "Rotary
                             Position Embeddings (RoPE)") is fused into the step: a
                             row at position pos has each pair of dims (j, j + D/2)
                             rotated by the angle pos * freqs[j], formed as a float32
                             product; k_new rows are rotated at seq_pos[b] + i as
                             they are appended, and q rows at seq_pos[b] + i before
                             the scores (the cache holds rotated keys).  Evaluated
                             in fp32 and rounded once to the 16-bit type.          */
    int32_t page_size;    /* 0: contiguous caches [B][Hkv][max_seq][D].  16: paged
                             caches, the page pool of the "Qwen MoE BringUp" page
                             ("Architecture Diagram - Qwen3-30B-A3B (Extern
                             Dispatch, 75 tok/s)", Paged Attention: KV write to a
                             page pool [pages][KV heads][16 tokens][head dim]):
                             k_cache / v_cache are pools [n_pages][Hkv][16][D] and
                             token t of sequence b lives in pool page
                             block_table[b][t / 16], slot t % 16.  Other sizes:
                             DA_ERR_UNSUPPORTED.                                   */
    int32_t pages_per_seq;/* paged: block-table row length; max_seq must equal
                             pages_per_seq * page_size                             */
    int32_t n_pages;      /* paged: pages in each pool                             */
    const int32_t *block_table; /* paged: DEVICE int32 [B][pages_per_seq], 4-byte
                             aligned.  Entries outside [0, n_pages) break the
                             contract: reads through them use page 0 and writes
                             through them are dropped, so no kernel touches memory
                             outside the pools; that sequence's results are
                             unspecified.                                          */
    int32_t rope_dim;     /* with rope_freqs: rotate only the first rope_dim dims of
                             each q / k row (pairs j and j + rope_dim/2; the table
                             holds rope_dim/2 values); 0 = head_dim.  64, 128 or 256
                             ("Qwen MoE BringUp", Model Architectures table and
                             "Architecture Diagram - Qwen3.5-35B-A3B": the rotary
                             embedding covers a quarter of the 256 dims)          */
    const void *out_gate; /* DEVICE [B][q_len][Hq][head_dim] in p->dtype, 16-byte
                             aligned, or NULL: the output is multiplied elementwise
                             by sigmoid(gate) in fp32 before rounding (the same
                             diagram's full-SDPA layers, whose Q projection also
                             yields a gate applied through a sigmoid)             */
    int32_t merge;        /* how da_decode_step combines the chunks' partials:
                             0 = automatic, 1 = inside the attention launch
                             whenever the plan allows it, 2 = always the separate
                             combine launch (a tuning and testing override).
                             Automatic merges inside the launch on the vector-ALU
                             kernel, and on the MFMA kernels only with at least
                             128 (sequence, KV head) pairs or at most 4 rows per
                             KV head; in every case only when no (sequence, KV
                             head) can have more than 256 chunk-rows (chunks x
                             rows; 512 on the vector-ALU kernel).  Other values:
                             DA_ERR_INVALID_ARG.                                  */
} da_problem;

/*
 * What the library will launch for a problem (a pure function of *p).
 *
 * Chunking.  With chunk_tokens == 0 the chunks are balanced on the device:
 * from the actual seq_pos values, every sequence's context is cut into equal
 * chunks whose length is close to an equal share of all visible keys (about
 * `target_items` chunks in all), never longer than `chunk_tokens` (the plan's
 * maximum) and never shorter than 64 keys.  With an explicit chunk_tokens every
 * chunk has that length.  Either way the attention and the combine derive the
 * same chunks from the same seq_pos.  A chunk is the work of one workgroup of
 * 4 waves.  On the vector-ALU kernel, with at most 2 rows per KV head and at
 * least 128 (sequence, KV head) pairs, chunks go up to 8192 keys (about 256 of
 * them), unless the contexts are so uneven that the longest of those chunks
 * would exceed 5/4 of an equal share: then about 1024 shorter chunks (automatic
 * targets only; the plan's workspace and grid hold either).
 */
typedef struct {
    int32_t chunk_tokens;    /* longest chunk (fixed mode: every chunk)          */
    int32_t n_chunks;        /* chunk slots per (sequence, KV head) in the workspace */
    int32_t rows;            /* query rows per KV head = (Hq / Hkv) * q_len      */
    int32_t variant;         /* DA_VARIANT_*                                     */
    int32_t balanced;        /* 1: balanced chunks, 0: fixed chunks              */
    int32_t target_items;    /* balanced: chunks aimed at                        */
    int32_t items;           /* chunks launched for (an upper bound; extras exit) */
    int32_t fused_combine;   /* da_decode_step merges inside its attention launch */
    size_t workspace_bytes;  /* bytes of fp32 partials (and the arrival counters
                                of da_decode_step) the attention needs           */
} da_plan;

enum { DA_VARIANT_VALU = 0, DA_VARIANT_MFMA = 1 };

/*
 * Plans the attention of *p: chunking, kernel variant, workspace size.  The
 * automatic variant is the MFMA kernel when rows >= 8 (Q K^T and P V are then
 * small matrix products, and on the vector ALU they would cost more issue
 * slots than streaming the keys from HBM), always for head_dim 256, and for
 * fewer than 128 (sequence, KV head) pairs with max_seq >= 1024 (its single
 * pass over a chunk has fewer dependent round trips than the vector-ALU
 * kernel's two); the vector-ALU kernel otherwise.
 * Returns DA_OK, DA_ERR_INVALID_ARG or DA_ERR_UNSUPPORTED.  Host only.
 */
da_status da_plan_attention(const da_problem *p, da_plan *plan);

/* Workspace bytes da_gqa_decode_attn needs for *p (0 if *p is invalid). */
size_t da_workspace_bytes(const da_problem *p);

/*
 * KV append ("KV Cache Update (EP rewrite: tensor.insert_slice)"):
 *   k_cache[b][h][seq_pos[b] + i][:] = k_new[b][i][h][:]   for i < q_len,
 * and the same for v_cache / v_new.  A bit copy: every other cache byte is
 * unchanged.  In place on the caller's cache.  k_new/v_new must not overlap
 * the caches.
 */
da_status da_kv_append(const da_problem *p, void *k_cache, void *v_cache, const void *k_new,
                       const void *v_new, const int32_t *seq_pos, void *stream);

/*
 * Split-context attention partials ("Attention Computation"; the split-KV
 * phase of the 3-phase decode).  Reads q and the caches (which must already
 * hold this step's rows: call da_kv_append first on the same stream), reads
 * only the visible cache slots [0, seq_pos[b] + q_len), and writes fp32
 * partials into `workspace` (at least da_workspace_bytes(p) bytes, not
 * aliasing any other argument).  Chunks beyond a sequence's context are not
 * written and not read later.
 */
da_status da_gqa_decode_attn(const da_problem *p, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *seq_pos, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Combine (the log-sum-exp reduce phase): merges the partials of every live
 * chunk and writes out[b][i][hq][:] rounded to nearest-even in p->dtype.
 * `workspace` must hold the partials of a da_gqa_decode_attn call with the
 * same *p and seq_pos, enqueued earlier on the same stream.
 */
da_status da_gqa_decode_attn_combine(const da_problem *p, const void *workspace,
                                     size_t workspace_bytes, const int32_t *seq_pos, void *out,
                                     void *stream);

/*
 * Prepares a workspace for da_decode_step: zeroes its arrival counters (one
 * int32 per sequence and KV head, 128 bytes apart, after the partials), on
 * `stream`, with a kernel (no memset).  Call once after allocating the
 * workspace, before its first da_decode_step; every da_decode_step leaves the
 * counters at zero again.
 * The three separate entry points neither need nor touch them.
 */
da_status da_workspace_init(const da_problem *p, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The whole decode step in one launch where it pays: KV append + attention +
 * combine with the results of da_kv_append, da_gqa_decode_attn and
 * da_gqa_decode_attn_combine called in that order (the same three steps of the
 * "Qwen MoE BringUp" page, Per-Layer IR Patterns, 2. Self-Attention, run as
 * the 3-phase decode of "Architecture Diagram - Qwen3-30B-A3B (Extern
 * Dispatch, 75 tok/s)"; the same page's update "11.6ms / 86 tok/s decode on
 * RX 7900 XTX", Key findings, measures per-dispatch overhead as over a quarter
 * of decode time and names fewer dispatches the main remaining opportunity).
 *
 *  - Append: the chunk holding a sequence's new positions reads those rows
 *    from k_new / v_new instead of the cache and stores them into the cache
 *    (a bit copy, same bytes as da_kv_append).  No chunk reads them from the
 *    cache, so there is no ordering hazard inside the launch.
 *  - Combine: with plan.fused_combine, every chunk counts its arrival on its
 *    (sequence, KV head) counter in the workspace, and the last one to arrive
 *    merges that head's rows into `out` and resets the counter; balanced
 *    chunking then gives a sequence at most 16 chunks (unless its length needs
 *    more chunks of the plan's longest length), so da_chunk_layout describes
 *    only the separate calls.  Otherwise the separate combine kernel follows on
 *    the same stream (two launches), and when the vector-ALU kernel is forced
 *    above 8 rows the step is the three separate launches.
 *
 * The workspace must have been prepared by da_workspace_init (once), and no
 * two calls may use one workspace concurrently (they would race on the
 * partials and the counters).  Contract-breaking seq_pos values: as for the
 * separate calls, the sequence's cache is not written and its output rows are
 * NaN.  k_new / v_new / q / out must not overlap the caches or the workspace.
 */
da_status da_decode_step(const da_problem *p, const void *q, void *k_cache, void *v_cache, const void *k_new,
                         const void *v_new, const int32_t *seq_pos, void *workspace, size_t workspace_bytes,
                         void *out, void *stream);

/*
 * da_decode_step without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and launches as da_decode_step
 * minus `workspace`: the partials and the arrival counters live in a scratch
 * array inside the library, 64 MiB on each GPU the library runs on, held until
 * the process ends (its device address is looked up once per device, and its
 * counters zeroed then, on `stream`).  Nothing here allocates.
 *  - A problem whose partials and counters do not fit returns
 *    DA_ERR_SCRATCH_LIMIT before anything is enqueued: with the merge inside
 *    the attention launch (plan.fused_combine) that takes
 *    B * Hkv * min(16, max_seq / 64) * rows * (head_dim + 2) * 4 bytes, plus
 *    1 MiB for the counters (128 bytes each, so at most 8192 sequence x KV
 *    head pairs); without it, the full da_workspace_bytes.  A problem too
 *    large for the latter may still fit with p->merge = 1 (the merge in the
 *    launch, where the plan allows it).
 *  - Every call on one GPU shares that GPU's scratch, which keeps the last
 *    call's partials: calls that overlap on one GPU (other streams, other
 *    threads) race and give wrong results.  Order them on one stream.
 */
da_status da_decode_step_static(const da_problem *p, const void *q, void *k_cache, void *v_cache,
                                const void *k_new, const void *v_new, const int32_t *seq_pos, void *out,
                                void *stream);

/*
 * The chunking da_gqa_decode_attn and the combine will use for these seq_pos
 * values, computed on the host (seq_pos_host is a HOST array of p->batch
 * values; the kernels derive the same layout from the device copy).  Writes
 * per sequence the number of chunks and their length in keys (0, 0 for a
 * sequence whose seq_pos breaks the contract).  Host only, no GPU needed.
 */
da_status da_chunk_layout(const da_problem *p, const int32_t *seq_pos_host, int32_t *n_chunks,
                          int32_t *chunk_len);

/* Static description of a status code. */
const char *da_status_str(da_status s);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
