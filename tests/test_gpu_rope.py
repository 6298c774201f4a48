"""GPU parity of the fused rotary embedding (RoPE) against the oracle.

With a rotary table in the problem, the append rotates each new K row at its
position seq_pos + i and the attention rotates each query row at the same
position.  The oracle computes the rotation in double and rounds once; the GPU
evaluates it in fp32 and rounds once, so a rotated element may land one 16-bit
ulp away when the exact value sits next to a rounding boundary, and a little more
where x cos a - y sin a nearly cancels (the fp32 evaluation's own error, a few
2^-24 of |x| + |y|).  Hence: every cache byte outside the new K rows matches the
oracle bit for bit (V rows included), rotated K elements are within one ulp plus
that slack and almost all identical, and outputs meet the usual
|d| <= 1e-2 + 1e-2 |ref|.
"""
import numpy as np
import pytest
import torch

import decode_attention_append_amd as da
from decode_attention_append_amd.workloads import rope_freqs
from tests import gpu_util as gu
from tests.oracle_pins import bits

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def check_rope(p, inp, freqs, path, rows=None):
    dt = gu.odt(inp["q"].dtype)
    fr = freqs.cpu().numpy()
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    sp = inp["seq_pos"].cpu().numpy()
    k_ref, v_ref = gu.oracle.kv_append_rope(kc0, vc0, bits(inp["k_new"]), bits(inp["v_new"]), sp, fr, dt)
    q_rot = gu.oracle.rope_q(bits(inp["q"]), sp, fr, dt)
    out = gu.run_step(p, inp, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(bits(inp["v_cache"]), v_ref), "v_cache differs"
    kg = bits(inp["k_cache"])
    new_rows = gu.appended_rows(kg.shape, sp, p.q_len)
    frac = gu.check_rotated_k(kg, k_ref, new_rows, bits(inp["k_new"]), sp, p.q_len, 2 * freqs.numel(), dt,
                              what=path)
    if rows is None:
        ref = gu.oracle.gqa_decode(q_rot, k_ref, v_ref, sp, dt)
        return gu.compare_out(out, ref, f"{path}: all rows"), frac
    rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
    ref = gu.oracle.gqa_decode_rows(q_rot, k_ref, v_ref, sp, rows, dt)
    o = out.cpu()
    got = torch.stack([o[b, i, hq] for b, i, hq in rows])
    return gu.compare_out(got, ref, f"{path}: sampled rows"), frac


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,seq_pos,dtype,theta", [
    (2, 1, 16, 8, 700, [699, 345], torch.bfloat16, 1.0e6),        # vector ALU, 2 rows
    (2, 1, 16, 16, 1000, [999, 64], torch.float16, 1.0e4),        # MHA fp16
    (2, 1, 64, 8, 3000, [2999, 1537], torch.bfloat16, 1.0e6),     # MFMA, 8 rows
    (2, 4, 32, 4, 2100, [2096, 777], torch.bfloat16, 1.0e6),      # MFMA, 32 rows, causal
    (2, 4, 8, 8, 700, [600, 61], torch.bfloat16, 1.0e6),          # vector ALU, 4 draft tokens
    (2, 8, 4, 2, 500, [492, 3], torch.float16, 1.0e4),            # MFMA, q_len 8
])
def test_rope_shapes(B, q_len, Hq, Hkv, S, seq_pos, dtype, theta, path):
    _say("rope", B, q_len, Hq, Hkv, S, seq_pos, dtype, theta, path)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, dtype, seed=S + 7)
    freqs = rope_freqs(128, theta, "cuda")
    p = da.problem_for(inp["q"], inp["k_cache"], rope_freqs=freqs)
    stats, frac = check_rope(p, inp, freqs, path)
    _say(stats, "rotated elements off by one ulp:", frac)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("q_len,Hq,Hkv,variant", [(4, 8, 8, "valu"), (4, 32, 4, "mfma"), (2, 8, 4, "mfma")])
def test_rope_new_rows_across_chunks(q_len, Hq, Hkv, variant, path):
    """64-key chunks with the draft tokens straddling a chunk boundary: each chunk
    appends and rotates only its own new rows."""
    _say("rope straddle", q_len, Hq, Hkv, variant, path)
    inp = gu.make_case(2, q_len, Hq, Hkv, 300, [62, 126], seed=31)
    freqs = rope_freqs(128, 1.0e6, "cuda")
    p = da.problem_for(inp["q"], inp["k_cache"], chunk_tokens=64, variant=variant, rope_freqs=freqs)
    check_rope(p, inp, freqs, path)


@pytest.mark.parametrize("path", gu.PATHS)
def test_rope_long_positions(path):
    """Positions up to 131071: angles of 10^5 radians need an exact range reduction."""
    S = 131072
    _say("rope long", path)
    inp = gu.make_case(2, 1, 16, 8, S, [S - 1, 70000], seed=32)
    freqs = rope_freqs(128, 1.0e4, "cuda")
    p = da.problem_for(inp["q"], inp["k_cache"], rope_freqs=freqs)
    rows = np.array([[0, 0, h] for h in range(16)] + [[1, 0, h] for h in range(0, 16, 3)])
    check_rope(p, inp, freqs, path, rows=rows)


def test_rope_decode_loop():
    """Four one-launch steps through one workspace with the cache growing: every step's
    rotated rows and outputs against the oracle."""
    B, q_len, Hq, Hkv, S = 3, 2, 16, 8, 2000
    freqs = rope_freqs(128, 1.0e6, "cuda")
    fr = freqs.cpu().numpy()
    inp = gu.make_case(B, q_len, Hq, Hkv, S, [100, 1500, 1998], seed=33)
    p = da.problem_for(inp["q"], inp["k_cache"], rope_freqs=freqs)
    ws = da.new_workspace(p)
    k_ref, v_ref = bits(inp["k_cache"]), bits(inp["v_cache"])
    sp = np.array([100, 1500, 1996], np.int32)
    inp["seq_pos"] = torch.as_tensor(sp).cuda()
    gen = torch.Generator().manual_seed(34)
    for it in range(4):
        _say("rope loop", it, sp.tolist())
        if it:
            for k in ("q", "k_new", "v_new"):
                inp[k] = torch.randn(inp[k].shape, generator=gen).to(torch.bfloat16).cuda()
            inp["seq_pos"] = torch.as_tensor(sp).cuda()
        out = gu.run_step(p, inp, ws=ws)
        torch.cuda.synchronize()
        k_ref, v_ref = gu.oracle.kv_append_rope(k_ref, v_ref, bits(inp["k_new"]), bits(inp["v_new"]), sp, fr,
                                                gu.oracle.BF16)
        # the GPU's rotated rows may sit an ulp (plus the fp32 evaluation slack) away:
        # check them against the oracle's, then carry the GPU cache forward
        kg = bits(inp["k_cache"])
        assert np.array_equal(bits(inp["v_cache"]), v_ref)
        gu.check_rotated_k(kg, k_ref, gu.appended_rows(kg.shape, sp, q_len), bits(inp["k_new"]), sp, q_len, 128,
                           gu.oracle.BF16, what=f"step {it}")
        k_ref = kg
        q_rot = gu.oracle.rope_q(bits(inp["q"]), sp, fr, gu.oracle.BF16)
        ref = gu.oracle.gqa_decode(q_rot, k_ref, v_ref, sp, gu.oracle.BF16)
        gu.compare_out(out, ref, f"step {it}")
        sp = np.minimum(sp + q_len, S - q_len).astype(np.int32)


def test_rope_forced_16_row_valu_refused():
    inp = gu.make_case(1, 2, 32, 4, 256, [100], seed=35)
    freqs = rope_freqs(128, 1.0e6, "cuda")
    p = da.problem_for(inp["q"], inp["k_cache"], variant="valu", rope_freqs=freqs)
    with pytest.raises(da.DecodeAttnError):
        da.plan_attention(p)
