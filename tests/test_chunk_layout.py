"""Host logic of the split-context chunking (the same code the kernels run on the device).

For any seq_pos values: the chunks of a sequence tile its visible context with no
empty chunk, stay within the kernel's longest chunk and the workspace's chunk
slots, and the launch grid covers every chunk.
"""
import numpy as np
import pytest

import decode_attention_append_amd as da


def check_layout(p, seq_pos):
    plan = da.plan_attention(p)
    lay = da.chunk_layout(p, seq_pos)
    total = 0
    for sp, (n, ln) in zip(seq_pos, lay):
        if sp < 0 or sp + p.q_len > p.max_seq:
            assert (n, ln) == (0, 0)
            continue
        ctx = sp + p.q_len
        assert n >= 1 and ln >= 1
        assert ln % 32 == 0
        assert ln <= plan["chunk_tokens"], "chunk longer than the kernel accepts"
        assert n <= plan["n_chunks"], "more chunks than workspace slots"
        assert (n - 1) * ln < ctx <= n * ln, "chunks must tile the context, last one non-empty"
        if not plan["balanced"]:
            assert ln == plan["chunk_tokens"]
        total += n
    total *= p.n_kv_heads
    assert total <= plan["items"], "launch grid misses chunks"
    return plan, lay, total


@pytest.mark.parametrize("seed", range(300))
def test_random_layouts(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    q_len = int(rng.integers(1, 9))
    while G * q_len > 32:
        q_len -= 1
    S = int(rng.choice([64, 100, 512, 777, 4096, 8192, 16384, 65536]))
    S = max(S, q_len)
    chunk = int(rng.choice([0, 0, 0, 64, 128, 256, 1024, 2048]))
    if chunk and -(-S // chunk) > 2048:
        chunk = 0
    variant = [None, "valu", "mfma"][int(rng.integers(0, 3))]
    if variant == "valu" and G * q_len > 16:
        variant = None
    wg = int(rng.choice([0, 0, 1, 37, 256, 5000]))
    p = da.problem(B, q_len, G * Hkv, Hkv, 128, S, "bf16", chunk_tokens=chunk, variant=variant,
                   work_items=wg)
    kind = rng.integers(0, 3)
    if kind == 0:
        sp = rng.integers(0, S - q_len + 1, B)
    elif kind == 1:  # one long, many short
        sp = np.zeros(B, dtype=np.int64)
        sp[0] = S - q_len
    else:  # all full
        sp = np.full(B, S - q_len)
    check_layout(p, sp.astype(np.int32))


@pytest.mark.parametrize("B,Hkv,S,work_items", [
    (1, 1, 65536, 0), (1, 1, 65536, 5000), (1, 8, 16384, 0), (3, 2, 8192, 37), (1, 4, 100000, 0),
    (2, 1, 1 << 21, 0),
])
def test_slots_bound_is_reached_not_exceeded(B, Hkv, S, work_items):
    """The workspace's chunk slots per (sequence, KV head) are the most chunks one
    sequence can get (ceil(target / Hkv), or ceil(S / longest chunk)): a single
    sequence among empty ones, at the context where chunks are the shortest, comes
    within a chunk of them, and no layout exceeds them."""
    p = da.problem(B, 1, 2 * Hkv, Hkv, 128, S, "bf16", work_items=work_items)
    plan = da.plan_attention(p)
    best = 0
    for ctx in (S, S - 1, S - 17, S // 2 + 31, 64 * plan["target_items"] // Hkv,
                64 * plan["target_items"] // Hkv - 40):
        if not 1 <= ctx <= S:
            continue
        sp = np.zeros(B, np.int32)
        sp[0] = ctx - 1
        _, lay, _ = check_layout(p, sp)
        best = max(best, lay[0][0])
    assert plan["n_chunks"] - 1 <= best <= plan["n_chunks"]


def test_contract_breaking_positions_get_no_chunks():
    p = da.problem(4, 2, 16, 8, 128, 1000, "bf16")
    _, lay, _ = check_layout(p, np.array([-1, 999, 998, 500], np.int32))
    assert lay[0] == (0, 0) and lay[1] == (0, 0) and lay[2][0] >= 1


def test_balanced_chunks_are_equal_share():
    """Ragged long contexts (GQA 64:8, batch 4, 12k..16k): every chunk close to one
    workgroup's share of all keys."""
    p = da.problem(4, 1, 64, 8, 128, 16384, "bf16", work_items=512)
    sp = np.array([15488, 13371, 15557, 14115], np.int32)
    plan, lay, total = check_layout(p, sp)
    share = 8 * int((sp + 1).sum()) / 512
    for n, ln in lay:
        assert 0.9 * share <= ln <= 1.15 * share
    assert 0.9 * 512 <= total <= 512 + 32  # lengths round up to 32 keys


def test_fixed_chunks_match_override():
    p = da.problem(2, 1, 16, 8, 128, 2500, "bf16", chunk_tokens=256)
    _, lay, _ = check_layout(p, np.array([2499, 1300], np.int32))
    assert lay == [(10, 256), (6, 256)]


def test_mfma128_chunks_start_on_512k_boundaries():
    """On the head_dim-128 MFMA kernel a balanced chunk that would be at least 1536 keys
    long is rounded up to a multiple of 2048 keys (512 KiB of K or V rows), so every
    chunk of such a sequence starts on a 512 KiB boundary of its stream; shorter chunks
    keep 32-key rounding, and head_dim 256 is not rounded."""
    rng = np.random.default_rng(5)
    p = da.problem(4, 1, 64, 8, 128, 16384, "bf16")
    assert da.plan_attention(p)["variant"] == "mfma"
    sp = rng.integers(12287, 16384, 4).astype(np.int32)
    _, lay, total = check_layout(p, sp)
    assert all(ln % 2048 == 0 for _, ln in lay)
    assert total <= 256
    # short contexts: chunks under 1024 keys stay 32-key multiples
    sp = np.array([3000, 2000, 5000, 4000], np.int32)
    _, lay, _ = check_layout(p, sp)
    assert any(ln % 2048 for _, ln in lay)
    # head_dim 256 keeps 32-key rounding
    p = da.problem(16, 1, 16, 2, 256, 8192, "fp16")
    sp = rng.integers(6143, 8192, 16).astype(np.int32)
    _, lay, _ = check_layout(p, sp)
    assert any(ln % 1024 for _, ln in lay)
    # chunks of 1024-1535 keys are not rounded (it would halve the workgroups)
    p = da.problem(1, 1, 16, 16, 128, 16384, "fp16")
    assert da.plan_attention(p)["variant"] == "mfma"
    _, lay, _ = check_layout(p, np.array([16383], np.int32))
    assert lay == [(16, 1024)]
    # the vector-ALU kernel is unaffected
    p = da.problem(4, 1, 16, 8, 128, 16384, "bf16", variant="valu")
    sp = rng.integers(12287, 16384, 4).astype(np.int32)
    _, lay, _ = check_layout(p, sp)
    assert any(ln % 2048 for _, ln in lay)


def test_long_chunks_fall_back_on_uneven_contexts():
    """The vector-ALU kernel's long chunks (up to 2 rows, at least 128 (sequence, KV
    head) pairs) aim at one chunk per compute unit, unless the contexts are so uneven
    that the longest chunk of that plan exceeds 5/4 of an equal share: then the plan
    aims at 1024 shorter chunks."""
    p = da.problem(32, 1, 16, 8, 128, 8192, "bf16")
    rng = np.random.default_rng(5)

    def lengths(sp):
        _, lay, total = check_layout(p, sp)
        return [ln for _, ln in lay], total

    full = np.full(32, 8191, np.int32)
    lens, total = lengths(full)
    assert set(lens) == {8192} and total == 32 * 8
    near = rng.integers(6143, 8192, 32).astype(np.int32)  # longest chunk under 5/4 of the share
    near[0] = 8191
    lens, total = lengths(near)
    assert total == 32 * 8 and max(lens) == 8192
    wide = rng.integers(1023, 8192, 32).astype(np.int32)
    wide[0] = 8191
    lens, total = lengths(wide)
    share = -(-8 * int((wide + 1).sum()) // 1024)  # keys per chunk for 1024 chunks
    # round(ctx / T) chunks of ceil32(ctx / n) keys: at most 1.5 T, rounded up
    assert total > 512 and max(lens) <= 1.5 * (share + 31) + 32
    # an explicit target keeps its own plan
    q = da.problem(32, 1, 16, 8, 128, 8192, "bf16", work_items=256)
    assert max(ln for _, ln in da.chunk_layout(q, wide)) > 2 * share
