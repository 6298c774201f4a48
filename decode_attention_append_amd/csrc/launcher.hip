// C-ABI entry points of libdecode_attn: argument checks, chunk planning and
// launches on the caller's stream.  Nothing here allocates, synchronises or
// reads device memory on the host.
#include "decode_attn.h"
#include "da_internal.h"

#include <math.h>

#include <mutex>

namespace {

using namespace da;

constexpr int kMaxSeq = 1 << 21;       // 2M slots: at most 2048 chunks of the shortest max chunk (1024)
constexpr int kMaxChunks = 2048;       // the combine keeps one weight per chunk in LDS
constexpr int kMaxValuRows = 16;       // the vector-ALU kernel's widest row set

bool aligned16(const void *x) { return ((uintptr_t)x & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

da_status check_problem(const da_problem *p) {
    if (!p) return DA_ERR_INVALID_ARG;
    if (p->batch <= 0 || p->q_len <= 0 || p->n_q_heads <= 0 || p->n_kv_heads <= 0 ||
        p->head_dim <= 0 || p->max_seq <= 0)
        return DA_ERR_INVALID_ARG;
    if (p->n_q_heads % p->n_kv_heads != 0) return DA_ERR_INVALID_ARG;
    if (p->q_len > p->max_seq) return DA_ERR_INVALID_ARG;
    if (isnan(p->scale) || isinf(p->scale)) return DA_ERR_INVALID_ARG;
    if (p->chunk_tokens != 0 &&
        (p->chunk_tokens < kTokenTile || p->chunk_tokens > kMaxChunk || p->chunk_tokens % kTokenTile))
        return DA_ERR_INVALID_ARG;
    if (p->variant < 0 || p->variant > DA_VARIANT_MFMA + 1) return DA_ERR_INVALID_ARG;
    if (p->work_items < 0 || p->work_items > (1 << 20)) return DA_ERR_INVALID_ARG;
    if (p->rope_freqs && !aligned16(p->rope_freqs)) return DA_ERR_INVALID_ARG;
    if (p->page_size != 0) {
        if (p->pages_per_seq <= 0 || p->n_pages <= 0 || !p->block_table || ((uintptr_t)p->block_table & 3u))
            return DA_ERR_INVALID_ARG;
        if ((int64_t)p->pages_per_seq * p->page_size != p->max_seq) return DA_ERR_INVALID_ARG;
        if (p->page_size != kPageTokens) return DA_ERR_UNSUPPORTED;
    }
    if (p->dtype != DA_BF16 && p->dtype != DA_FP16) return DA_ERR_UNSUPPORTED;
    if (p->head_dim != kHeadDim && p->head_dim != kMaxHeadDim) return DA_ERR_UNSUPPORTED;
    // head_dim 256 runs on the MFMA kernel only
    if (p->head_dim != kHeadDim && p->variant == DA_VARIANT_VALU + 1) return DA_ERR_UNSUPPORTED;
    if (p->rope_dim != 0 && (p->rope_dim > p->head_dim ||
                             (p->rope_dim != 64 && p->rope_dim != 128 && p->rope_dim != 256)))
        return DA_ERR_UNSUPPORTED;
    if (p->out_gate && !aligned16(p->out_gate)) return DA_ERR_INVALID_ARG;
    if (p->merge < 0 || p->merge > 2) return DA_ERR_INVALID_ARG;
    if (p->q_len > kMaxQLen) return DA_ERR_UNSUPPORTED;
    if ((int64_t)(p->n_q_heads / p->n_kv_heads) * p->q_len > kMaxRows) return DA_ERR_UNSUPPORTED;
    if (p->max_seq > kMaxSeq) return DA_ERR_UNSUPPORTED;
    if (p->variant == DA_VARIANT_VALU + 1 && (p->n_q_heads / p->n_kv_heads) * p->q_len > kMaxValuRows)
        return DA_ERR_UNSUPPORTED;
    // the vector-ALU kernel rotates q only up to 8 rows (it is chosen automatically
    // only below 8)
    if (p->rope_freqs && p->variant == DA_VARIANT_VALU + 1 && (p->n_q_heads / p->n_kv_heads) * p->q_len > 8)
        return DA_ERR_UNSUPPORTED;
    if (p->chunk_tokens != 0 && (p->max_seq + p->chunk_tokens - 1) / p->chunk_tokens > kMaxChunks)
        return DA_ERR_UNSUPPORTED;
    // grid sizes stay within int
    if ((int64_t)p->batch * p->n_kv_heads * ((p->max_seq + kTokenTile - 1) / kTokenTile) > INT32_MAX / 2)
        return DA_ERR_UNSUPPORTED;
    if ((int64_t)p->batch * p->q_len * p->n_q_heads * 16 > INT32_MAX / 2) return DA_ERR_UNSUPPORTED;
    // and so do the arrival counters' int32 offsets (B * Hkv <= 2^25)
    if ((int64_t)p->batch * p->n_kv_heads * kCounterStride > INT32_MAX / 2) return DA_ERR_UNSUPPORTED;
    return DA_OK;
}

// Chunks to aim for in balanced mode, per kernel: a few per compute unit (256
// on MI355X) at the kernel's occupancy.  A vector-ALU chunk is a 4-wave
// workgroup (about 7 fit per compute unit).  An MFMA chunk is a 4-wave
// workgroup too, whose waves share the chunk's tiles: one per compute unit
// keeps every wave streaming long runs of tiles.  Measured (attention launch,
// separate path): GQA-8 at 12k-16k context 50.0 / 49.7 / 52.1 us and the
// 4-token verify 27.6 / 28.7 / 34.6 us at 256 / 512 / 1024 chunks; head_dim 256
// on 16 x 2 KV heads at 8k context 52.8 / 55.3 / 56.2 us.
// With long chunks (below) the vector-ALU kernel also aims at one chunk per
// compute unit.
int default_target(int variant, bool long_chunks) {
    return variant == DA_VARIANT_MFMA || long_chunks ? 256 : 1024;
}

// Long chunks on the vector-ALU kernel.  Up to 2 rows, when there are at least
// 128 (sequence, KV head) units, a workgroup takes chunks of up to
// kValuLongChunk (8192) keys: a (sequence, KV head) of up to 8192 keys is one
// chunk, whose workgroup writes the output itself in the one-launch step: no
// partials, no arrival and no merge.  Its four waves, each with two 16-key
// slabs in flight, keep 32 KiB of non-temporal loads in flight per compute
// unit, where a loads-only probe streams best.  Measured against 8-wave
// workgroups on the same chunks (64 KiB in flight), steps by eager launches:
// batch 32, 8 KV heads, 8192 keys, 2 rows, 28 layers 4.28 against
// 4.40 ms; batch 64 at 4k 1258 / 1268 us for 8 layers, batch 32 MHA at 2k 641
// / 653 us, batch 16 at 16k 622 / 635 us for 4 layers, batch 4 MHA 32 heads at
// 4k and batch 32 at ragged 1k-8k contexts equal (two runs each); 16 waves
// were slower still (161.5 against 158.2 us a layer of that step).
bool valu_long_chunks(int variant, int rows, int units) {
    return variant == DA_VARIANT_VALU && rows <= 2 && units >= 128;
}

// The alternate target of the long chunks: the chunk plan switches to it
// when the contexts are too uneven for one chunk per compute unit (see
// long_plan_uneven).  None with an explicit work_items.
int alt_target_of(const da_problem *p, int variant, int rows, int units) {
    return p->work_items == 0 && valu_long_chunks(variant, rows, units) ? default_target(variant, false) : 0;
}

// Longest chunk a kernel accepts: the vector-ALU kernel keeps the chunk's
// scores in LDS (rows x chunk floats, at most 64 KiB).
int max_chunk_of(int variant, int rows, bool long_chunks) {
    if (variant == DA_VARIANT_MFMA) return 4096;
    if (long_chunks) return kValuLongChunk;
    const int rp = rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : 16;
    return rp <= 8 ? 2048 : 1024;
}

constexpr int kMinChunk = 64;

// Balanced chunk lengths on the head_dim-128 MFMA kernel are rounded up to whole
// multiples of 512 KiB of K (and V) rows, 2048 keys, when a chunk would be at
// least three quarters that long, so chunks start on 512 KiB boundaries of a
// (sequence, KV head) stream.  (From half that long, chunks of 1024-1535 keys
// grew by up to twice and halved the workgroups: batch-1 MHA at 16k, 1024-key
// chunks, took 38.7 us a layer rounded against 27.7 us not.)  Measured with the
// attention launch alone on the GQA-8 long-context workload (contexts 12k-16k):
// 47.8-48.2 us against 50.1-50.6 us with 32-key rounding (256 KiB: 47.5-48.2
// us, but it lengthens the 4-token verify's chunks and costs it 24%).  On the head_dim-256 kernel the same
// rounding slows the one-launch step by 1.6%, so there chunks keep 32-key
// rounding; the vector-ALU kernel's chunks are already whole 2048-key runs on
// full-length batches.
constexpr int kMfma128ChunkAlignBytes = 512 * 1024;

int chunk_align_of(int variant, int head_dim) {
    if (variant != DA_VARIANT_MFMA || head_dim != kHeadDim) return 32;
    return kMfma128ChunkAlignBytes / (head_dim * 2);
}

// Rows per KV head from which the matrix-core kernel is used (and for fewer
// rows, see auto_variant).  Below 8 rows the
// vector-ALU kernel is memory-bound (its dot products cost about 4 wave
// instructions per key and row); at 8 rows it needs some 34 wave instructions
// per key and becomes ALU-bound near 40% of HBM bandwidth, while the MFMA
// kernel streams at over 60%.
constexpr int kMfmaRows = 8;

// The automatic kernel.  The matrix-core kernel from kMfmaRows rows and for
// head_dim 256.  Below that, with fewer than 128 (sequence, KV head) pairs and a
// cache of at least 1024 slots, the matrix-core kernel as well: its 32-key
// tiles carry K and V together and two of them stay in flight per wave (32 KiB
// per wave against the vector-ALU kernel's 8 KiB, whose K and V passes each
// wait for their own round trips), which is what a step with few heads is
// short of.  Steps by graph replay, per layer, vector ALU / matrix cores:
// batch-1 MHA 16 heads at 4k 14.9 / 13.9 us, at 1k 12.0 / 11.6 us, at 16k
// 28.9 / 28.6 us; batch 1, 16:8, 32k 44.5 / 39.3 us; batch 8, 16:8, 2k 22.8 /
// 20.2 us; batch 2, 32:8, 8k 24.6 / 20.8 us.  At 512 slots (batch 1, 16:8) the
// vector-ALU kernel stays ahead (20.3 / 20.9 us), and from 128 pairs its long
// chunks, one per head, are (batch 4, MHA 32 heads, 4k: 46.2 /
// 48.3 us).
int auto_variant(const da_problem *p, int rows, int units) {
    if (rows >= kMfmaRows || p->head_dim != kHeadDim) return DA_VARIANT_MFMA;
    return units < 128 && p->max_seq >= 1024 ? DA_VARIANT_MFMA : DA_VARIANT_VALU;
}

// Most chunk-rows (chunks x query rows) one (sequence, KV head) may have for
// the one-launch step to merge them inside the attention launch, where the
// last workgroup of the (sequence, KV head) merges: on the MFMA kernels its
// four waves take two rows at a time with every load in flight, on the
// vector-ALU kernel the workgroup splits rows or chunks.  Beyond that the
// separate combine launch, with a workgroup per row, finishes sooner.
constexpr int kFusedMergeRowsMfma = 256;
constexpr int kFusedMergeRowsValu = 512;

int fused_merge_rows(int variant) {
    return variant == DA_VARIANT_MFMA ? kFusedMergeRowsMfma : kFusedMergeRowsValu;
}

// Chunks per sequence (balanced mode) when the one-launch step merges in the
// launch: every chunk counts its arrival on one atomic per (sequence, KV
// head), and those serialise; measured on a batch-1, 16-head, 4k-context MHA
// step, 16 chunks of 256 keys beat 64 chunks of 64 keys by a fifth.
constexpr int kOneLaunchSeqChunks = 16;

// The vector-ALU kernel carries the one-launch step's append and merge up to 8
// rows; beyond (only when it is forced) da_decode_step makes three launches.
bool one_launch_capable(int variant, int rows) { return variant == DA_VARIANT_MFMA || rows <= 8; }

// Automatic choice of the in-launch merge.  After the last chunk of a (sequence,
// KV head) ends, the merge inside the launch costs a chain of dependent memory
// round trips (the partial's stores acknowledged, the arrival atomic, the other
// partials' loads, the output store): about 5 us on the MFMA kernels, whose
// partials are 8-32 rows wide; a separate combine launch costs less there.
// Step times by graph replay, cold, in launch / separate combine: GQA 64:8 at
// 12k-16k context (32 heads) 57.1 / 55.7 us; head_dim-256 gated 16:2 at 6k-8k
// (32 heads) 50.7 / 48.0 us a layer; batch 1, 32:4, 32k context 40.1 / 21.9 us
// a layer and head_dim 256 at 8k 27.2 / 17.2 us (the merge's cap of 16 chunks
// a sequence also leaves most compute units idle there); batch 4, 32:4, 4k
// context 17.4 / 16.1 us.  With at least 128 heads (at most two chunks each)
// the merge is small and stays in the launch: batch 16, 64:8, 1k context 21.7 /
// 22.4 us.  The vector-ALU kernel's partials are 1-8 rows wide and its merge
// stays in the launch (batch-1 MHA at 4k: 14.9 / 15.1 us a layer; the
// 512-context layer 20.2 / 21.5 us).
constexpr int kMfmaMergeMinUnits = 128;
// ... or when the partials are at most 4 rows wide (the matrix-core kernel on
// few-head steps, above): batch-1 MHA at 4k 13.9 against 15.0 us a layer,
// batch 1, 16:8 at 32k 39.5 / 40.5 us, batch 8, 16:8 at 2k 20.25 / 20.9 us.
constexpr int kMfmaMergeMaxRows = 4;

bool merge_in_launch(const da_problem *p, int variant, int units) {
    if (p->merge == 2) return false;
    const int rows = (p->n_q_heads / p->n_kv_heads) * p->q_len;
    return p->merge == 1 || variant == DA_VARIANT_VALU || units >= kMfmaMergeMinUnits || rows <= kMfmaMergeMaxRows;
}

void plan_of(const da_problem *p, da_plan *pl) {
    const int rows = (p->n_q_heads / p->n_kv_heads) * p->q_len;
    const int units = p->batch * p->n_kv_heads;
    const int variant = p->variant ? p->variant - 1 : auto_variant(p, rows, units);
    pl->rows = rows;
    pl->variant = variant;
    if (p->chunk_tokens) {  // fixed chunks
        pl->balanced = 0;
        pl->chunk_tokens = p->chunk_tokens;
        pl->n_chunks = (p->max_seq + p->chunk_tokens - 1) / p->chunk_tokens;
        pl->target_items = units * pl->n_chunks;
        pl->items = units * pl->n_chunks;
    } else {
        const bool long_chunks = valu_long_chunks(variant, rows, units);
        const int max_chunk = max_chunk_of(variant, rows, long_chunks);
        pl->balanced = 1;
        pl->chunk_tokens = max_chunk;
        pl->target_items = p->work_items > 0 ? p->work_items : default_target(variant, long_chunks);
        // the larger of the two targets the device may plan for
        const int32_t alt = alt_target_of(p, variant, rows, units);
        const int32_t target = pl->target_items > alt ? pl->target_items : alt;
        // slots for the most chunks a sequence can get, whatever the seq_pos
        // values: round(ctx / T) with T >= Hkv * (all visible keys) / target
        // (a sequence holds at most all of them) is at most ceil(target / Hkv),
        // unless T is clamped to max_chunk, where a sequence gets
        // ceil(ctx / max_chunk); never more than one per 64 keys.  max_seq <=
        // 2048 * max_chunk keeps ceil(ctx / max_chunk) within them, so no chunk
        // exceeds max_chunk.
        const int64_t per_seq_target = ((int64_t)target + p->n_kv_heads - 1) / p->n_kv_heads;
        const int64_t per_seq_long = (p->max_seq + max_chunk - 1) / max_chunk;
        int64_t slots = per_seq_target > per_seq_long ? per_seq_target : per_seq_long;
        const int64_t by_min = (p->max_seq + kMinChunk - 1) / kMinChunk;
        if (slots > by_min) slots = by_min;
        pl->n_chunks = (int32_t)(slots < kMaxChunks ? slots : kMaxChunks);
        // at most target + one rounding chunk per (sequence, head), or every
        // sequence in chunks of max_chunk keys when the target is too few
        const int64_t a = (int64_t)target + units;
        const int64_t b = (int64_t)units * ((p->max_seq + max_chunk - 1) / max_chunk);
        pl->items = (int32_t)(a > b ? a : b);
    }
    // the one-launch step merges inside the attention launch when the last chunk
    // of a (sequence, KV head) can merge its rows quickly: at most
    // kFusedMergeRows chunk-rows per (sequence, KV head), bounded over all
    // seq_pos values.  There a balanced sequence gets at most
    // kOneLaunchSeqChunks chunks, or ceil(max_seq / max_chunk) if more.
    int64_t nb_max = pl->n_chunks;
    if (pl->balanced) {
        const int64_t need = (p->max_seq + pl->chunk_tokens - 1) / pl->chunk_tokens;
        const int64_t bound = need > kOneLaunchSeqChunks ? need : kOneLaunchSeqChunks;
        if (bound < nb_max) nb_max = bound;
    }
    pl->fused_combine = merge_in_launch(p, variant, units) && one_launch_capable(variant, rows) &&
                        nb_max * rows <= fused_merge_rows(variant);
    const int32_t bh = units;
    pl->workspace_bytes = align256(ws_acc_floats(bh, pl->n_chunks, rows, p->head_dim) * sizeof(float)) +
                          align256(ws_ml_floats(bh, pl->n_chunks, rows) * sizeof(float)) +
                          (size_t)bh * kCounterStride * sizeof(int32_t);
}

// Arrival counters of the one-launch step: int32 [B * Hkv] at kCounterStride,
// after the partials.
int32_t *counters_of(const da_problem *p, const da_plan &pl, void *workspace) {
    const int32_t bh = p->batch * p->n_kv_heads;
    return (int32_t *)((uint8_t *)workspace +
                       align256(ws_acc_floats(bh, pl.n_chunks, pl.rows, p->head_dim) * sizeof(float)) +
                       align256(ws_ml_floats(bh, pl.n_chunks, pl.rows) * sizeof(float)));
}

// Chunk slots per (sequence, KV head) the one-launch step with the fused merge
// can use: balanced chunking caps a sequence there at kOneLaunchSeqChunks
// chunks unless its length needs more of the longest chunk (the same bound
// plan_of checks), so the chunking itself is the same as with n_chunks slots.
int32_t fused_slots(const da_problem *p, const da_plan &pl) {
    int64_t nb_max = pl.n_chunks;
    if (pl.balanced) {
        const int64_t need = (p->max_seq + pl.chunk_tokens - 1) / pl.chunk_tokens;
        const int64_t bound = need > kOneLaunchSeqChunks ? need : kOneLaunchSeqChunks;
        if (bound < nb_max) nb_max = bound;
    }
    return (int32_t)nb_max;
}

KvLayout layout_of(const da_problem *p) {
    KvLayout L;
    L.row_bytes = p->head_dim * 2;
    L.block_table = p->page_size ? p->block_table : nullptr;
    L.pages_per_seq = p->page_size ? p->pages_per_seq : 0;
    L.n_pages = p->page_size ? p->n_pages : 0;
    return L;
}

AttnParams attn_params(const da_problem *p, const da_plan &pl, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *seq_pos, const void *workspace) {
    AttnParams a;
    a.q = (const uint8_t *)q;
    a.k_cache = (const uint8_t *)k_cache;
    a.v_cache = (const uint8_t *)v_cache;
    a.seq_pos = seq_pos;
    const int32_t bh = p->batch * p->n_kv_heads;
    a.ws_acc = (float *)workspace;
    a.ws_ml = (float *)((uint8_t *)workspace +
                        align256(ws_acc_floats(bh, pl.n_chunks, pl.rows, p->head_dim) * sizeof(float)));
    a.batch = p->batch;
    a.q_len = p->q_len;
    a.n_q_heads = p->n_q_heads;
    a.n_kv_heads = p->n_kv_heads;
    a.max_seq = p->max_seq;
    a.group = p->n_q_heads / p->n_kv_heads;
    a.rows = pl.rows;
    a.n_chunks = pl.n_chunks;
    a.fixed_chunk = pl.balanced ? 0 : pl.chunk_tokens;
    a.target_wg = pl.target_items;
    a.alt_target_wg = pl.balanced ? alt_target_of(p, pl.variant, pl.rows, p->batch * p->n_kv_heads) : 0;
    a.min_chunk = kMinChunk;
    a.max_chunk = pl.chunk_tokens;
    const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / sqrt((double)p->head_dim);
    a.scale_log2 = (float)(scale * 1.4426950408889634);  // log2(e)
    a.seq_chunk_cap = 0;
    a.chunk_align = chunk_align_of(pl.variant, p->head_dim);
    a.rope_freqs = p->rope_freqs;
    a.rope_dim = p->rope_dim ? p->rope_dim : p->head_dim;
    a.layout = layout_of(p);
    a.head_dim = p->head_dim;
    a.out_gate = (const uint16_t *)p->out_gate;
    a.k_cache_w = a.v_cache_w = nullptr;
    a.k_new = a.v_new = nullptr;
    a.counters = nullptr;
    a.out = nullptr;
    return a;
}

bool step_pointers_ok(const void *q, const void *k_cache, const void *v_cache, const void *k_new, const void *v_new,
                      const int32_t *seq_pos, const void *out) {
    if (!q || !k_cache || !v_cache || !k_new || !v_new || !seq_pos || !out) return false;
    return aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(k_new) && aligned16(v_new) &&
           aligned16(out) && ((uintptr_t)seq_pos & 3u) == 0;
}

// The one-launch step (or, where the plan does not fuse, its two or three
// launches) with the partials at acc / ml (`slots` chunk slots per (sequence,
// KV head)) and the arrival counters at `counters` (zero between calls).
da_status decode_step_on(const da_problem *p, const da_plan &pl, const void *q, void *k_cache, void *v_cache,
                         const void *k_new, const void *v_new, const int32_t *seq_pos, float *acc, float *ml,
                         int32_t slots, int32_t *counters, void *out, hipStream_t s) {
    const bool fp16 = p->dtype == DA_FP16;
    AttnParams a = attn_params(p, pl, q, k_cache, v_cache, seq_pos, nullptr);
    a.ws_acc = acc;
    a.ws_ml = ml;
    a.n_chunks = slots;
    if (!one_launch_capable(pl.variant, pl.rows)) {  // append, attention, combine
        AppendParams ap;
        ap.k_cache = (uint8_t *)k_cache;
        ap.v_cache = (uint8_t *)v_cache;
        ap.k_new = (const uint8_t *)k_new;
        ap.v_new = (const uint8_t *)v_new;
        ap.seq_pos = seq_pos;
        ap.rope_freqs = p->rope_freqs;
        ap.layout = layout_of(p);
        ap.head_dim = p->head_dim;
        ap.rope_dim = p->rope_dim ? p->rope_dim : p->head_dim;
        ap.batch = p->batch;
        ap.q_len = p->q_len;
        ap.n_kv_heads = p->n_kv_heads;
        ap.max_seq = p->max_seq;
        (void)hipGetLastError();
        hipError_t e = launch_kv_append(ap, p->batch * p->q_len * p->n_kv_heads * (p->head_dim / 8), fp16, s);
        if (e == hipSuccess) e = launch_attn_valu(a, pl.items, fp16, s);
        if (e == hipSuccess) e = launch_attn_combine(a, fp16, out, s);
        return e == hipSuccess ? DA_OK : DA_ERR_HIP;
    }
    a.k_cache_w = (uint8_t *)k_cache;
    a.v_cache_w = (uint8_t *)v_cache;
    a.k_new = (const uint8_t *)k_new;
    a.v_new = (const uint8_t *)v_new;
    int items = pl.items;
    if (pl.fused_combine) {
        a.seq_chunk_cap = pl.balanced ? kOneLaunchSeqChunks : 0;
        a.counters = counters;
        a.out = (uint16_t *)out;
        items += p->batch;  // the items past the chunks flag contract-breaking sequences
    }
    (void)hipGetLastError();
    hipError_t e = pl.variant == DA_VARIANT_MFMA ? launch_attn_mfma(a, items, fp16, s)
                                                 : launch_attn_valu(a, items, fp16, s);
    if (e == hipSuccess && !pl.fused_combine) e = launch_attn_combine(a, fp16, out, s);
    return e == hipSuccess ? DA_OK : DA_ERR_HIP;
}

// ---- the allocation-free step's scratch ------------------------------------------
// da_decode_step_static keeps its arrival counters (the first kScratchCounterBytes)
// and its partials in this array, one copy per GPU the library runs on, held
// until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, once per device, with that device current, and the
// counters are zeroed then, on the caller's stream, ahead of the step's kernels.
// 64 MiB holds every workload of the suite as planned (the largest, a 4-token
// verify with its separate combine, needs 32.5 MiB).
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr size_t kScratchCounterBytes = (size_t)1 << 20;  // counters of up to 8192 (sequence, KV head) pairs
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchOnDevice {
    std::once_flag once;
    uint8_t *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchOnDevice g_scratch[kMaxDevices];

hipError_t scratch_on_current_device(uint8_t **ptr, hipStream_t s) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchOnDevice &d = g_scratch[dev];
    std::call_once(d.once, [&] {
        void *addr = nullptr;
        d.err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess) {
            d.ptr = (uint8_t *)addr;
            (void)hipGetLastError();
            d.err = launch_fill_zero((int32_t *)d.ptr, (int)(kScratchCounterBytes / sizeof(int32_t)), s);
        }
    });
    *ptr = d.ptr;
    return d.err;
}

}  // namespace

extern "C" {

da_status da_plan_attention(const da_problem *p, da_plan *plan) {
    if (!plan) return DA_ERR_INVALID_ARG;
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    plan_of(p, plan);
    return DA_OK;
}

size_t da_workspace_bytes(const da_problem *p) {
    da_plan pl;
    if (da_plan_attention(p, &pl) != DA_OK) return 0;
    return pl.workspace_bytes;
}

da_status da_kv_append(const da_problem *p, void *k_cache, void *v_cache, const void *k_new,
                       const void *v_new, const int32_t *seq_pos, void *stream) {
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    if (!k_cache || !v_cache || !k_new || !v_new || !seq_pos) return DA_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
        ((uintptr_t)seq_pos & 3u))
        return DA_ERR_INVALID_ARG;
    AppendParams a;
    a.k_cache = (uint8_t *)k_cache;
    a.v_cache = (uint8_t *)v_cache;
    a.k_new = (const uint8_t *)k_new;
    a.v_new = (const uint8_t *)v_new;
    a.seq_pos = seq_pos;
    a.rope_freqs = p->rope_freqs;
    a.layout = layout_of(p);
    a.head_dim = p->head_dim;
    a.rope_dim = p->rope_dim ? p->rope_dim : p->head_dim;
    a.batch = p->batch;
    a.q_len = p->q_len;
    a.n_kv_heads = p->n_kv_heads;
    a.max_seq = p->max_seq;
    const int threads = p->batch * p->q_len * p->n_kv_heads * (p->head_dim / 8);
    (void)hipGetLastError();  // launch errors below are ours alone
    return launch_kv_append(a, threads, p->dtype == DA_FP16, (hipStream_t)stream) == hipSuccess ? DA_OK
                                                                                                  : DA_ERR_HIP;
}

da_status da_gqa_decode_attn(const da_problem *p, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *seq_pos, void *workspace,
                             size_t workspace_bytes, void *stream) {
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    if (!q || !k_cache || !v_cache || !seq_pos || !workspace) return DA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace) ||
        ((uintptr_t)seq_pos & 3u))
        return DA_ERR_INVALID_ARG;
    da_plan pl;
    plan_of(p, &pl);
    if (workspace_bytes < pl.workspace_bytes) return DA_ERR_WORKSPACE;
    const AttnParams a = attn_params(p, pl, q, k_cache, v_cache, seq_pos, workspace);
    (void)hipGetLastError();
    const hipError_t e = pl.variant == DA_VARIANT_MFMA
                             ? launch_attn_mfma(a, pl.items, p->dtype == DA_FP16, (hipStream_t)stream)
                             : launch_attn_valu(a, pl.items, p->dtype == DA_FP16, (hipStream_t)stream);
    return e == hipSuccess ? DA_OK : DA_ERR_HIP;
}

da_status da_gqa_decode_attn_combine(const da_problem *p, const void *workspace,
                                     size_t workspace_bytes, const int32_t *seq_pos, void *out,
                                     void *stream) {
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    if (!workspace || !seq_pos || !out) return DA_ERR_INVALID_ARG;
    if (!aligned16(workspace) || !aligned16(out) || ((uintptr_t)seq_pos & 3u)) return DA_ERR_INVALID_ARG;
    da_plan pl;
    plan_of(p, &pl);
    if (workspace_bytes < pl.workspace_bytes) return DA_ERR_WORKSPACE;
    const AttnParams a = attn_params(p, pl, nullptr, nullptr, nullptr, seq_pos, workspace);
    (void)hipGetLastError();
    return launch_attn_combine(a, p->dtype == DA_FP16, out, (hipStream_t)stream) == hipSuccess ? DA_OK
                                                                                                 : DA_ERR_HIP;
}

da_status da_workspace_init(const da_problem *p, void *workspace, size_t workspace_bytes, void *stream) {
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    if (!workspace || !aligned16(workspace)) return DA_ERR_INVALID_ARG;
    da_plan pl;
    plan_of(p, &pl);
    if (workspace_bytes < pl.workspace_bytes) return DA_ERR_WORKSPACE;
    (void)hipGetLastError();
    const int n_words = p->batch * p->n_kv_heads * kCounterStride;
    return launch_fill_zero(counters_of(p, pl, workspace), n_words, (hipStream_t)stream) ==
                   hipSuccess
               ? DA_OK
               : DA_ERR_HIP;
}

da_status da_decode_step(const da_problem *p, const void *q, void *k_cache, void *v_cache, const void *k_new,
                         const void *v_new, const int32_t *seq_pos, void *workspace, size_t workspace_bytes,
                         void *out, void *stream) {
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    if (!workspace || !aligned16(workspace)) return DA_ERR_INVALID_ARG;
    if (!step_pointers_ok(q, k_cache, v_cache, k_new, v_new, seq_pos, out)) return DA_ERR_INVALID_ARG;
    da_plan pl;
    plan_of(p, &pl);
    if (workspace_bytes < pl.workspace_bytes) return DA_ERR_WORKSPACE;
    const int32_t bh = p->batch * p->n_kv_heads;
    float *acc = (float *)workspace;
    float *ml = (float *)((uint8_t *)workspace + align256(ws_acc_floats(bh, pl.n_chunks, pl.rows, p->head_dim) * sizeof(float)));
    return decode_step_on(p, pl, q, k_cache, v_cache, k_new, v_new, seq_pos, acc, ml, pl.n_chunks,
                          counters_of(p, pl, workspace), out, (hipStream_t)stream);
}

da_status da_decode_step_static(const da_problem *p, const void *q, void *k_cache, void *v_cache,
                                const void *k_new, const void *v_new, const int32_t *seq_pos, void *out,
                                void *stream) {
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    if (!step_pointers_ok(q, k_cache, v_cache, k_new, v_new, seq_pos, out)) return DA_ERR_INVALID_ARG;
    da_plan pl;
    plan_of(p, &pl);
    // partials: with the fused merge only the slots that step can fill
    const int32_t bh = p->batch * p->n_kv_heads;
    const int32_t slots = pl.fused_combine ? fused_slots(p, pl) : pl.n_chunks;
    const size_t acc_bytes = align256(ws_acc_floats(bh, slots, pl.rows, p->head_dim) * sizeof(float));
    const size_t ml_bytes = align256(ws_ml_floats(bh, slots, pl.rows) * sizeof(float));
    if ((size_t)bh * kCounterStride * sizeof(int32_t) > kScratchCounterBytes ||
        kScratchCounterBytes + acc_bytes + ml_bytes > kScratchBytes)
        return DA_ERR_SCRATCH_LIMIT;
    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = nullptr;
    if (scratch_on_current_device(&base, s) != hipSuccess) return DA_ERR_HIP;
    return decode_step_on(p, pl, q, k_cache, v_cache, k_new, v_new, seq_pos, (float *)(base + kScratchCounterBytes),
                          (float *)(base + kScratchCounterBytes + acc_bytes), slots, (int32_t *)base, out, s);
}

da_status da_chunk_layout(const da_problem *p, const int32_t *seq_pos_host, int32_t *n_chunks,
                          int32_t *chunk_len) {
    const da_status st = check_problem(p);
    if (st != DA_OK) return st;
    if (!seq_pos_host || !n_chunks || !chunk_len) return DA_ERR_INVALID_ARG;
    da_plan pl;
    plan_of(p, &pl);
    const AttnParams a = attn_params(p, pl, nullptr, nullptr, nullptr, seq_pos_host, nullptr);
    const int T = a.fixed_chunk > 0 ? a.fixed_chunk : balanced_chunk(a);
    for (int b = 0; b < p->batch; ++b) {
        const SeqChunks sc = seq_chunks(a, b, T);
        n_chunks[b] = sc.n;
        chunk_len[b] = sc.n ? sc.len : 0;
    }
    return DA_OK;
}

const char *da_status_str(da_status s) {
    switch (s) {
        case DA_OK: return "ok";
        case DA_ERR_INVALID_ARG: return "invalid argument";
        case DA_ERR_UNSUPPORTED: return "unsupported problem";
        case DA_ERR_WORKSPACE: return "workspace too small";
        case DA_ERR_HIP: return "HIP launch failed";
        case DA_ERR_SCRATCH_LIMIT: return "problem needs more scratch than the allocation-free step holds";
    }
    return "unknown status";
}

}  // extern "C"
