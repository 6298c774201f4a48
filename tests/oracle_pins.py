"""Pins of the reference oracle against facts that do not come from the oracle.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError if
the oracle disagrees with a closed form, an invariant of the definition, a
value the pages print, or a library routine that computes the same special
case.  ``test_oracle.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on deliberately broken builds of it and expects each break caught.
"""
import json
import math
import os

import numpy as np
import torch

from oracle import BF16, FP16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bits(t: torch.Tensor) -> np.ndarray:
    """16-bit patterns of a bf16/fp16 tensor as a uint16 numpy array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _tdt(dtype):
    return torch.bfloat16 if dtype == BF16 else torch.float16


def rand_case(B, q_len, Hq, Hkv, D, S, seq_pos, dtype=BF16, seed=0, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    tdt = _tdt(dtype)
    q = (torch.randn(B, q_len, Hq, D, generator=g) * scale).to(tdt)
    kc = (torch.randn(B, Hkv, S, D, generator=g) * scale).to(tdt)
    vc = (torch.randn(B, Hkv, S, D, generator=g) * scale).to(tdt)
    kn = (torch.randn(B, q_len, Hkv, D, generator=g) * scale).to(tdt)
    vn = (torch.randn(B, q_len, Hkv, D, generator=g) * scale).to(tdt)
    sp = np.asarray(seq_pos, dtype=np.int32)
    return q, kc, vc, kn, vn, sp


# ---------------------------------------------------------------- decoding

def pin_decode_bf16_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = orc.decode(pats, BF16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_decode_fp16_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = orc.decode(pats, FP16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- append

def pin_append_insert_slice_box(orc):
    """The page's insert_slice box: [0, 0, offset, 0] + [1, 16, seq_len, 128]."""
    gold = _golden("insert_slice_box.json")
    B, H, S, D = gold["cache_shape"]
    g = torch.Generator().manual_seed(7)
    for case in gold["cases"]:
        off, n = case["offset"], case["seq_len"]
        kc = bits(torch.randn(B, H, S, D, generator=g).to(torch.bfloat16))
        vc = bits(torch.randn(B, H, S, D, generator=g).to(torch.bfloat16))
        # the page's block is [1, 16, seq_len, 128]; the oracle takes [B, q_len, Hkv, D]
        blk_k = bits(torch.randn(1, H, n, D, generator=g).to(torch.bfloat16))
        blk_v = bits(torch.randn(1, H, n, D, generator=g).to(torch.bfloat16))
        kn = np.ascontiguousarray(blk_k.transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(blk_v.transpose(0, 2, 1, 3))
        k2, v2 = orc.kv_append(kc, vc, kn, vn, [off])
        box = np.zeros((B, H, S, D), dtype=bool)
        box[0:1, 0:H, off:off + n, 0:D] = True
        for before, after, blk in ((kc, k2, blk_k), (vc, v2, blk_v)):
            assert np.array_equal(after[~box], before[~box]), "element outside the box changed"
            assert np.array_equal(after[box].reshape(1, H, n, D), blk), "box not written"


def pin_append_ragged_batch(orc):
    """Per-sequence offsets: sequence b gets its rows at seq_pos[b], nowhere else."""
    B, q_len, Hkv, D, S = 3, 3, 2, 16, 20
    q, kc, vc, kn, vn, sp = rand_case(B, q_len, 2, Hkv, D, S, [0, 9, 17])
    kc, vc, kn, vn = bits(kc), bits(vc), bits(kn), bits(vn)
    k2, v2 = orc.kv_append(kc, vc, kn, vn, sp)
    for b in range(B):
        for h in range(Hkv):
            for s in range(S):
                i = s - sp[b]
                if 0 <= i < q_len:
                    assert np.array_equal(k2[b, h, s], kn[b, i, h])
                    assert np.array_equal(v2[b, h, s], vn[b, i, h])
                else:
                    assert np.array_equal(k2[b, h, s], kc[b, h, s])
                    assert np.array_equal(v2[b, h, s], vc[b, h, s])


# ---------------------------------------------------------------- attention

def pin_one_key_context(orc):
    """Only one visible key (seq_pos 0, one new token): every output row is that value row."""
    for dtype in (BF16, FP16):
        q, kc, vc, kn, vn, sp = rand_case(2, 1, 8, 2, 128, 16, [0, 0], dtype, seed=1)
        k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
        out = orc.gqa_decode(bits(q), k2, v2, sp, dtype)
        vref = orc.decode(bits(vn), dtype)  # [B, 1, Hkv, D]
        for hq in range(8):
            assert np.array_equal(out[:, 0, hq, :], vref[:, 0, hq // 4, :])


def pin_identical_keys_mean(orc):
    """All visible keys equal: uniform weights, the output is the mean of the value rows."""
    B, Hq, Hkv, D, S = 1, 4, 2, 128, 64
    q, kc, vc, kn, vn, _ = rand_case(B, 1, Hq, Hkv, D, S, [0], seed=2)
    kc[:] = kc[:, :, :1, :]
    kn[:] = kc[:, :, :1, :].permute(0, 2, 1, 3)
    ctx = 50
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), [ctx - 1])
    out = orc.gqa_decode(bits(q), k2, v2, [ctx - 1], BF16)
    vdec = orc.decode(v2, BF16)
    for hq in range(Hq):
        mean = vdec[0, hq // 2, :ctx, :].sum(axis=0) / ctx
        np.testing.assert_allclose(out[0, 0, hq], mean, rtol=1e-13, atol=1e-15)


def pin_weights_sum_to_one(orc):
    q, kc, vc, kn, vn, sp = rand_case(2, 3, 6, 3, 32, 40, [10, 36], seed=3)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
    out, w = orc.gqa_decode(bits(q), k2, v2, sp, BF16, with_weights=True)
    assert np.all(np.abs(w.sum(axis=-1) - 1.0) <= 1e-13)
    assert np.all(w >= 0.0)
    for b in range(2):
        for i in range(3):
            assert np.all(w[b, i, :, sp[b] + i + 1:] == 0.0)
            assert np.all(w[b, i, :, :sp[b] + i + 1] > 0.0)


def pin_causal_mask_table(orc):
    """Visibility pattern equals the page's LessOrEqual/Less mask, worked out by hand."""
    gold = _golden("causal_mask_table.json")
    p, n, S = gold["seq_pos"], gold["q_len"], gold["cache_len"]
    q, kc, vc, kn, vn, _ = rand_case(1, n, 2, 1, 8, S, [p], seed=4, scale=0.25)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), [p])
    _, w = orc.gqa_decode(bits(q), k2, v2, [p], BF16, with_weights=True)
    vis = np.asarray(gold["visible"], dtype=bool)
    for hq in range(2):
        assert np.array_equal(w[0, :, hq, :] > 0.0, vis)


def pin_closed_form_three_keys(orc):
    gold = _golden("closed_form_three_keys.json")
    D = gold["head_dim"]
    e = math.e
    vals = np.asarray(gold["values"], dtype=np.float64)
    expect = (vals[0] + e * vals[1] + e * e * vals[2]) / (1.0 + e + e * e)
    for dtype in (BF16, FP16):
        tdt = _tdt(dtype)
        q = torch.tensor(gold["q"]).reshape(1, 1, 1, D).to(tdt)
        kc = torch.zeros(1, 1, 4, D)
        vc = torch.zeros(1, 1, 4, D)
        kc[0, 0, :2] = torch.tensor(gold["keys"][:2])
        vc[0, 0, :2] = torch.tensor(gold["values"][:2])
        kn = torch.tensor(gold["keys"][2]).reshape(1, 1, 1, D)
        vn = torch.tensor(gold["values"][2]).reshape(1, 1, 1, D)
        kc[0, 0, 3] = float("nan")  # beyond the context: must not matter
        vc[0, 0, 3] = float("nan")
        k2, v2 = orc.kv_append(bits(kc.to(tdt)), bits(vc.to(tdt)), bits(kn.to(tdt)),
                               bits(vn.to(tdt)), [2])
        out = orc.gqa_decode(bits(q), k2, v2, [2], dtype)
        np.testing.assert_allclose(out[0, 0, 0], expect, rtol=2e-15, atol=1e-15)


def pin_gqa_equals_mha_repeated(orc):
    """Query head hq uses KV head hq // (Hq/Hkv): same as MHA over repeat-interleaved KV heads."""
    B, q_len, Hq, Hkv, D, S = 2, 2, 8, 2, 32, 24
    q, kc, vc, kn, vn, sp = rand_case(B, q_len, Hq, Hkv, D, S, [5, 21], seed=5)
    G = Hq // Hkv
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
    out = orc.gqa_decode(bits(q), k2, v2, sp, BF16)
    k_rep = np.ascontiguousarray(np.repeat(k2, G, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(v2, G, axis=1))
    out_mha = orc.gqa_decode(bits(q), k_rep, v_rep, sp, BF16)
    assert np.array_equal(out, out_mha)


def pin_torch_sdpa_float64(orc):
    """Special case computed by a library: torch's CPU SDPA in float64 with enable_gqa."""
    B, q_len, Hq, Hkv, D, S = 2, 3, 8, 2, 64, 48
    q, kc, vc, kn, vn, sp = rand_case(B, q_len, Hq, Hkv, D, S, [7, 44], seed=6)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
    out = orc.gqa_decode(bits(q), k2, v2, sp, BF16)
    qd = q.double().permute(0, 2, 1, 3)                        # [B, Hq, q_len, D]
    kd = torch.from_numpy(k2.view(np.int16)).view(torch.bfloat16).double()  # [B, Hkv, S, D]
    vd = torch.from_numpy(v2.view(np.int16)).view(torch.bfloat16).double()
    j = torch.arange(S)
    for b in range(B):
        tpos = sp[b] + torch.arange(q_len)
        mask = (j[None, :] <= tpos[:, None]) & (j[None, :] < sp[b] + q_len)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qd[b:b + 1], kd[b:b + 1], vd[b:b + 1], attn_mask=mask[None, None], enable_gqa=True)
        ref = ref.permute(0, 2, 1, 3).numpy()[0]
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def pin_causal_prefix(orc):
    """Query token 0 of a 4-token verify sees exactly what a 1-token step at the same slot sees."""
    B, Hq, Hkv, D, S, p = 1, 4, 1, 64, 32, 20
    q, kc, vc, kn, vn, _ = rand_case(B, 4, Hq, Hkv, D, S, [p], seed=8)
    k4, v4 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), [p])
    out4 = orc.gqa_decode(bits(q), k4, v4, [p], BF16)
    k1, v1 = orc.kv_append(bits(kc), bits(vc), bits(kn[:, :1]), bits(vn[:, :1]), [p])
    out1 = orc.gqa_decode(bits(q[:, :1]), k1, v1, [p], BF16)
    assert np.array_equal(out4[:, 0], out1[:, 0])
    # and the later draft tokens see more keys, so their rows differ
    assert not np.array_equal(out4[:, 3], out1[:, 0])


def pin_value_homogeneity(orc):
    """Doubling every value row doubles the output exactly (powers of two are exact)."""
    q, kc, vc, kn, vn, sp = rand_case(1, 2, 4, 2, 32, 16, [9], seed=9)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
    out = orc.gqa_decode(bits(q), k2, v2, sp, BF16)
    _, v2x = orc.kv_append(bits(kc), bits(vc * 2), bits(kn), bits(vn * 2), sp)
    out2 = orc.gqa_decode(bits(q), k2, v2x, sp, BF16)
    assert np.array_equal(out2, 2.0 * out)


def pin_key_permutation_invariance(orc):
    """Reordering the (key, value) rows of the context leaves a one-token step unchanged."""
    S, ctx = 64, 57
    q, kc, vc, kn, vn, _ = rand_case(1, 1, 4, 2, 64, S, [ctx - 1], seed=10)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), [ctx - 1])
    out = orc.gqa_decode(bits(q), k2, v2, [ctx - 1], BF16)
    perm = np.random.default_rng(0).permutation(ctx)
    k3, v3 = k2.copy(), v2.copy()
    k3[:, :, :ctx] = k2[:, :, perm]
    v3[:, :, :ctx] = v2[:, :, perm]
    out3 = orc.gqa_decode(bits(q), k3, v3, [ctx - 1], BF16)
    np.testing.assert_allclose(out3, out, rtol=1e-13, atol=1e-14)


def pin_beyond_context_and_future_rows(orc):
    """Rows past the context never matter; a later draft token's row is hidden from earlier ones."""
    S, p = 32, 12
    q, kc, vc, kn, vn, _ = rand_case(1, 2, 2, 1, 16, S, [p], seed=11)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), [p])
    out = orc.gqa_decode(bits(q), k2, v2, [p], BF16)
    nan, inf = np.uint16(0x7fc0), np.uint16(0x7f80)
    k3, v3 = k2.copy(), v2.copy()
    k3[:, :, p + 2:] = nan
    v3[:, :, p + 2:] = inf
    assert np.array_equal(orc.gqa_decode(bits(q), k3, v3, [p], BF16), out)
    v4 = v2.copy()
    v4[:, :, p + 1] = nan  # the second draft token's value row
    out4 = orc.gqa_decode(bits(q), k2, v4, [p], BF16)
    assert np.array_equal(out4[:, 0], out[:, 0])
    assert np.all(np.isnan(out4[:, 1]))


def pin_rows_api_matches_full(orc):
    q, kc, vc, kn, vn, sp = rand_case(2, 2, 4, 2, 32, 20, [3, 17], seed=12)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
    out = orc.gqa_decode(bits(q), k2, v2, sp, BF16)
    rows = np.array([[0, 0, 0], [1, 1, 3], [1, 0, 2], [0, 1, 1]])
    got = orc.gqa_decode_rows(bits(q), k2, v2, sp, rows, BF16)
    for n, (b, i, hq) in enumerate(rows):
        assert np.array_equal(got[n], out[b, i, hq])


# ---------------------------------------------------------------- encoding

def _all_patterns():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def pin_encode_round_trip_all_patterns(orc):
    """Every finite pattern decodes and re-encodes to itself; NaNs stay NaN."""
    for dtype in (BF16, FP16):
        pats = _all_patterns()
        vals = orc.decode(pats, dtype)
        back = orc.encode(vals, dtype)
        nan = np.isnan(vals)
        assert np.array_equal(back[~nan], pats[~nan])
        assert np.isnan(orc.decode(back[nan], dtype)).all()


def _spread(rng, n):
    """Doubles over the whole 16-bit ranges: subnormals, normals, near overflow, both signs."""
    mag = np.exp2(rng.uniform(-30, 18, n)) * rng.uniform(1, 2, n)
    return np.where(rng.random(n) < 0.5, -mag, mag)


def pin_encode_fp16_matches_numpy(orc):
    """numpy's float64 -> float16 conversion rounds to nearest even in one step."""
    rng = np.random.default_rng(3)
    x = _spread(rng, 20000)
    with np.errstate(over="ignore"):  # magnitudes past 65504 round to infinity on both sides
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.encode(x, FP16), ref)


def pin_encode_bf16_matches_torch_on_floats(orc):
    """For values exactly representable in float32, torch's float32 -> bfloat16 rounding
    (nearest even) is the one rounding step."""
    rng = np.random.default_rng(4)
    x32 = _spread(rng, 20000).astype(np.float32)
    x32 = x32[np.abs(x32) < 3.0e38]
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.encode(x32.astype(np.float64), BF16), ref)


def pin_encode_bf16_direct_rounding(orc):
    """Cases the bfloat16 definition fixes, including two a float32 detour would get wrong
    (a tie broken by bits beyond float32)."""
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie between 1 and 1+2^-7: even
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # just above the tie: up
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie between 0x3F81 and 0x3F82: even
        (1.0 + 3 * 2.0 ** -8 - 2.0 ** -45, 0x3F81),
        (-2.0, 0xC000),
        ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
        ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # ties up to infinity
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # half of it: tie to even zero
        (1.5 * 2.0 ** -134, 0x0001),
    ]
    for x, want in cases:
        assert int(orc.encode([x], BF16)[0]) == want, (x, hex(want))


# ---------------------------------------------------------------- rotary embedding

def qwen_freqs(D, theta=1.0e6):
    """Inverse frequencies theta^(-2j/D), j < D/2, as a float32 table (an input)."""
    return (theta ** (-np.arange(0, D, 2, dtype=np.float64) / D)).astype(np.float32)


def _complex_rotation(x, positions, freqs):
    """Reference: dims j and j + D/2 as the real and imaginary parts of z_j, multiplied
    by exp(i a_j) with a_j the float32 product of position and frequency."""
    half = x.shape[-1] // 2
    a = (np.float32(1) * positions.astype(np.float32)[:, None] * freqs[None, :]).astype(np.float64)
    z = (x[:, :half] + 1j * x[:, half:]) * np.exp(1j * a)
    return np.concatenate([z.real, z.imag], axis=1)


def _ulp(ref, mbits, emin):
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** emin)))
    return np.exp2(e - mbits)


def pin_rope_position_zero_is_identity(orc):
    for dtype in (BF16, FP16):
        q, _, _, kn, _, _ = rand_case(2, 3, 4, 2, 128, 8, [0, 0], dtype, seed=21)
        x = bits(q).reshape(-1, 128)
        out = orc.rope_rows(x, np.zeros(x.shape[0], np.int32), qwen_freqs(128), dtype)
        assert np.array_equal(out, x)


def pin_rope_is_complex_rotation(orc):
    """Against complex multiplication in numpy: correctly rounded to the 16-bit format
    (bit-identical to numpy's rounding for fp16; within half an ulp for bf16)."""
    rng = np.random.default_rng(22)
    for dtype, freqs in ((FP16, qwen_freqs(128)), (BF16, qwen_freqs(128, 1.0e4))):
        q, _, _, _, _, _ = rand_case(1, 1, 64, 1, 128, 1, [0], dtype, seed=23)
        x = bits(q).reshape(-1, 128)
        pos = rng.integers(0, 1 << 20, x.shape[0]).astype(np.int32)
        pos[:4] = [1, 2, 4095, 16383]
        got = orc.rope_rows(x, pos, freqs, dtype)
        ref = _complex_rotation(orc.decode(x, dtype), pos, freqs)
        if dtype == FP16:
            assert np.array_equal(got, ref.astype(np.float16).view(np.uint16))
        else:
            err = np.abs(orc.decode(got, BF16) - ref)
            assert (err <= 0.5 * _ulp(ref, 7, -126) * (1 + 1e-9)).all()


def pin_rope_relative_position(orc):
    """With power-of-two frequencies every angle is exact, and the score between a query at
    position m and a key at position n depends only on m - n."""
    D = 128
    freqs = np.exp2(-np.arange(D // 2, dtype=np.float64) / 4.0).astype(np.float32)
    freqs = np.exp2(np.floor(np.log2(freqs))).astype(np.float32)
    q, _, _, kn, _, _ = rand_case(1, 1, 8, 8, D, 1, [0], BF16, seed=24)
    qx, kx = bits(q).reshape(-1, D), bits(kn).reshape(-1, D)
    for m, n in ((7, 3), (100, 36), (1000, 1)):
        a = orc.decode(orc.rope_rows(qx, np.full(8, m, np.int32), freqs, BF16), BF16)
        b = orc.decode(orc.rope_rows(kx, np.full(8, n, np.int32), freqs, BF16), BF16)
        c = orc.decode(orc.rope_rows(qx, np.full(8, m - n, np.int32), freqs, BF16), BF16)
        k0 = orc.decode(kx, BF16)
        lhs, rhs = (a * b).sum(1), (c * k0).sum(1)
        assert np.abs(lhs - rhs).max() < 0.25, (m, n, np.abs(lhs - rhs).max())


def pin_rope_append_and_query_positions(orc):
    """The rotated append writes k_new[b, i] rotated at seq_pos[b] + i (V unchanged), and
    the rotated query row (b, i) uses the same position; checked row by row against the
    complex rotation."""
    freqs = qwen_freqs(128)
    q, kc, vc, kn, vn, sp = rand_case(2, 3, 4, 2, 128, 40, [5, 30], FP16, seed=25)
    k2, v2 = orc.kv_append_rope(bits(kc), bits(vc), bits(kn), bits(vn), sp, freqs, FP16)
    k_plain, v_plain = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
    assert np.array_equal(v2, v_plain)
    qr = orc.rope_q(bits(q), sp, freqs, FP16)
    for b in range(2):
        for i in range(3):
            pos = np.array([sp[b] + i] * 2, np.int32)
            want_k = _complex_rotation(orc.decode(bits(kn)[b, i], FP16), pos, freqs)
            assert np.array_equal(k2[b, :, sp[b] + i], want_k.astype(np.float16).view(np.uint16))
            pos_q = np.array([sp[b] + i] * 4, np.int32)
            want_q = _complex_rotation(orc.decode(bits(q)[b, i], FP16), pos_q, freqs)
            assert np.array_equal(qr[b, i], want_q.astype(np.float16).view(np.uint16))
    untouched = np.ones(k2.shape[2], bool)
    for b in range(2):
        untouched[:] = True
        untouched[sp[b]:sp[b] + 3] = False
        assert np.array_equal(k2[b][:, untouched], k_plain[b][:, untouched])


# ---------------------------------------------------------------- paged KV cache

def pin_paged_pool_layout(orc):
    """Hand-worked positions of the page pool layout (tests/golden/paged_pool_layout.json)."""
    g = _golden("paged_pool_layout.json")
    shape = tuple(g["pool_shape"])
    pool = np.arange(np.prod(shape), dtype=np.uint16).reshape(shape)  # every element distinct
    out = orc.gather_paged(pool, np.array(g["block_table"], np.int32))
    for c in g["cases"]:
        assert out[c["b"], c["h"], c["t"], c["d"]] == pool[tuple(c["pool"])], c


def _paged_case(rng, B, Hkv, D, pps, n_pages):
    pool_k = rng.integers(0, 1 << 16, (n_pages, Hkv, 16, D), dtype=np.uint32).astype(np.uint16) & 0xBFFF
    pool_v = rng.integers(0, 1 << 16, (n_pages, Hkv, 16, D), dtype=np.uint32).astype(np.uint16) & 0xBFFF
    bt = rng.permutation(n_pages)[:B * pps].reshape(B, pps).astype(np.int32)
    return pool_k, pool_v, bt


def pin_paged_append_commutes_with_contiguous(orc):
    """Appending into the pool and then gathering equals gathering and then the (pinned)
    contiguous append; no other pool byte changes."""
    rng = np.random.default_rng(41)
    B, Hkv, D, pps, n_pages, q_len = 3, 2, 8, 4, 16, 3
    pk, pv, bt = _paged_case(rng, B, Hkv, D, pps, n_pages)
    kn = rng.integers(0, 1 << 16, (B, q_len, Hkv, D), dtype=np.uint32).astype(np.uint16)
    vn = rng.integers(0, 1 << 16, (B, q_len, Hkv, D), dtype=np.uint32).astype(np.uint16)
    sp = np.array([0, 14, 61], np.int32)  # one crossing a page boundary, one at the end
    pk2, pv2 = orc.kv_append_paged(pk, pv, kn, vn, sp, bt)
    kc, vc = orc.kv_append(orc.gather_paged(pk, bt), orc.gather_paged(pv, bt), kn, vn, sp)
    assert np.array_equal(orc.gather_paged(pk2, bt), kc)
    assert np.array_equal(orc.gather_paged(pv2, bt), vc)
    changed = np.argwhere((pk2 != pk).any(axis=(1, 3)))
    for page, h, tok in [(int(a), int(b_), int(c)) for a, b_, c in np.argwhere((pk2 != pk).any(axis=3))]:
        assert any(bt[b, (sp[b] + i) // 16] == page and (sp[b] + i) % 16 == tok
                   for b in range(B) for i in range(q_len)), (page, h, tok)
    assert len(changed) >= 1


def pin_paged_page_relabelling(orc):
    """Renumbering the pool's pages (and the block table with them) changes nothing."""
    rng = np.random.default_rng(42)
    pk, _, bt = _paged_case(rng, 2, 2, 8, 3, 10)
    perm = rng.permutation(10)
    pk_relabelled = np.empty_like(pk)
    pk_relabelled[perm] = pk  # page p moves to slot perm[p]
    assert np.array_equal(orc.gather_paged(pk_relabelled, perm[bt].astype(np.int32)), orc.gather_paged(pk, bt))


def pin_paged_rejects_bad_pages(orc):
    rng = np.random.default_rng(43)
    pk, pv, bt = _paged_case(rng, 2, 2, 8, 2, 6)
    bad = bt.copy()
    bad[1, 1] = 6
    try:
        orc.gather_paged(pk, bad)
    except ValueError:
        pass
    else:
        raise AssertionError("a block-table entry outside the pool was accepted")


# ---------------------------------------------------------------- head_dim 256, partial rotation, gate

def pin_partial_rope_256(orc):
    """Rotating the first 64 of 256 dims: those equal the complex rotation of pairs
    (j, j + 32), correctly rounded; dims 64..255 pass unchanged."""
    rng = np.random.default_rng(51)
    freqs = qwen_freqs(64, 1.0e7)
    q, _, _, _, _, _ = rand_case(1, 1, 32, 1, 256, 1, [0], FP16, seed=52)
    x = bits(q).reshape(-1, 256)
    pos = rng.integers(0, 1 << 18, x.shape[0]).astype(np.int32)
    got = orc.rope_rows(x, pos, freqs, FP16)
    assert np.array_equal(got[:, 64:], x[:, 64:])
    ref = _complex_rotation(orc.decode(x[:, :64], FP16), pos, freqs)
    assert np.array_equal(got[:, :64], ref.astype(np.float16).view(np.uint16))


def pin_output_gate_is_sigmoid(orc):
    """Against scipy's logistic function; gate 0 halves exactly; -inf closes the gate."""
    from scipy.special import expit
    rng = np.random.default_rng(53)
    for dtype in (BF16, FP16):
        g = bits((torch.randn(4, 256, generator=torch.Generator().manual_seed(54)) * 3).to(_tdt(dtype)))
        out = rng.standard_normal((4, 256))
        got = orc.output_gate(out, g, dtype)
        ref = out * expit(orc.decode(g, dtype))
        assert np.allclose(got, ref, rtol=1e-14, atol=0)
    half = orc.output_gate(np.array([3.0, -7.0]), np.zeros(2, np.uint16), BF16)
    assert np.array_equal(half, np.array([1.5, -3.5]))
    closed = orc.output_gate(np.array([2.0]), np.array([0xFF80], np.uint16), BF16)  # bf16 -inf
    assert closed[0] == 0.0


def pin_torch_sdpa_float64_d256(orc):
    """Head dim 256, GQA 16:2, a 4-token causal window: torch's float64 SDPA with
    enable_gqa and an explicit mask."""
    B, q_len, Hq, Hkv, D, S = 2, 4, 16, 2, 256, 90
    q, kc, vc, kn, vn, sp = rand_case(B, q_len, Hq, Hkv, D, S, [40, 86], BF16, seed=55)
    k2, v2 = orc.kv_append(bits(kc), bits(vc), bits(kn), bits(vn), sp)
    got = orc.gqa_decode(bits(q), k2, v2, sp, BF16)
    qd = torch.from_numpy(orc.decode(bits(q), BF16)).permute(0, 2, 1, 3)
    kd = torch.from_numpy(orc.decode(k2, BF16))
    vd = torch.from_numpy(orc.decode(v2, BF16))
    for b in range(B):
        t = sp[b] + torch.arange(q_len)[:, None]
        mask = torch.arange(S)[None, :] <= t
        ref = torch.nn.functional.scaled_dot_product_attention(qd[b:b + 1], kd[b:b + 1], vd[b:b + 1],
                                                               attn_mask=mask, enable_gqa=True)
        assert np.allclose(got[b], ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
