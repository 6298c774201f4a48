"""GPU parity of head_dim 256 (the full-attention layers of Qwen3.5-35B-A3B: 16 query
heads over 2 KV heads of 256 dims, rotary embedding on the first 64 dims, sigmoid
output gate) and of the partial rotary width and the gate on head_dim 128.

Every case runs through the three separate calls and the one-launch
da_decode_step.  Caches bit for bit (rotated K rows within one ulp plus the fp32
evaluation slack of gpu_util.check_rotated_k), outputs
|gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise.
"""
import numpy as np
import pytest
import torch

import decode_attention_append_amd as da
from decode_attention_append_amd.workloads import WORKLOADS, make_layer, rope_freqs
from tests import gpu_util as gu
from tests.oracle_pins import bits
from tests.test_gpu_paged import make_paged

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _problem(inp, freqs=None, rope_dim=0, **kw):
    return da.problem_for(inp["q"], inp["k_cache"], block_table=inp.get("block_table"),
                          rope_freqs=freqs, rope_dim=rope_dim, out_gate=inp.get("out_gate"), **kw)


@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,seq_pos,dtype", [
    (2, 1, 16, 2, 1000, [999, 300], torch.bfloat16),           # 8 rows
    (3, 1, 16, 2, 700, [0, 333, 699], torch.float16),          # ragged, first slot
    (2, 1, 4, 4, 900, [899, 64], torch.bfloat16),              # MHA, one row
    (2, 1, 8, 2, 600, [599, 17], torch.float16),               # 4 rows
    (2, 2, 24, 2, 600, [598, 255], torch.bfloat16),            # 24 rows: wave pairs
    (2, 4, 16, 2, 2100, [2096, 777], torch.float16),           # verify 4, 32 rows
    (2, 8, 4, 2, 500, [492, 3], torch.bfloat16),               # q_len 8, 16 rows
])
def test_d256_shapes(B, q_len, Hq, Hkv, S, seq_pos, dtype):
    _say("d256", B, q_len, Hq, Hkv, S, seq_pos, dtype)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, dtype, seed=S + Hq, head_dim=256)
    p = _problem(inp)
    assert da.plan_attention(p)["variant"] == "mfma"
    gu.check_full(p, inp)


@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,seq_pos,rope_dim,dtype", [
    (2, 1, 16, 2, 1200, [1199, 100], 64, torch.float16),       # the Qwen3.5 layer
    (2, 4, 16, 2, 900, [896, 31], 64, torch.float16),          # verify 4
    (2, 1, 16, 2, 800, [799, 5], 256, torch.bfloat16),         # full rotation
    (2, 1, 16, 2, 800, [700, 400], 128, torch.bfloat16),       # half rotation
])
def test_d256_gate_and_partial_rope(B, q_len, Hq, Hkv, S, seq_pos, rope_dim, dtype):
    _say("d256 gate rope", B, q_len, Hq, Hkv, S, seq_pos, rope_dim, dtype)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, dtype, seed=rope_dim + S, head_dim=256, gate=True)
    freqs = rope_freqs(rope_dim, 1.0e7, "cuda")
    p = _problem(inp, freqs, rope_dim)
    gu.check_full(p, inp, freqs=freqs)


@pytest.mark.parametrize("q_len,Hq,Hkv,pps,seq_pos", [
    (1, 16, 2, 60, [959, 17, 500]),
    (4, 16, 2, 40, [636, 62, 200]),
])
def test_d256_paged_gate_rope(q_len, Hq, Hkv, pps, seq_pos):
    _say("d256 paged", q_len, Hq, Hkv, pps, seq_pos)
    inp = make_paged(3, q_len, Hq, Hkv, pps, seq_pos, torch.float16, seed=pps, head_dim=256, gate=True)
    freqs = rope_freqs(64, 1.0e7, "cuda")
    p = _problem(inp, freqs, 64)
    gu.check_full(p, inp, freqs=freqs)


@pytest.mark.parametrize("chunk", [64, 128, 256, 0])
def test_d256_chunk_sweep(chunk):
    _say("d256 chunk", chunk)
    inp = gu.make_case(2, 2, 16, 2, 1500, [1498, 700], seed=chunk + 1, head_dim=256)
    p = _problem(inp, chunk_tokens=chunk)
    gu.check_full(p, inp)


@pytest.mark.parametrize("path", gu.PATHS)
def test_d256_one_key_returns_value_exactly(path):
    """seq_pos 0 without gate or rotation: the output is v_new exactly."""
    inp = gu.make_case(2, 1, 16, 2, 256, [0, 0], seed=5, head_dim=256)
    p = _problem(inp)
    out = gu.run_step(p, inp, path=path)
    assert torch.equal(out[:, 0], inp["v_new"][:, 0].repeat_interleave(8, dim=1))


@pytest.mark.parametrize("path", gu.PATHS)
def test_d256_beyond_context_poison(path):
    sp = [700, 1499, 63]
    inp = gu.make_case(3, 1, 16, 2, 1500, sp, seed=7, head_dim=256, gate=True)
    clean = {k: v.clone() for k, v in inp.items()}
    p_clean, p = _problem(clean), _problem(inp)
    out_clean = gu.run_step(p_clean, clean, path=path)
    for b, s in enumerate(sp):
        inp["k_cache"][b, :, s:] = float("nan")
        inp["v_cache"][b, :, s:] = float("inf")
    out = gu.run_step(p, inp, path=path)
    assert torch.equal(out, out_clean)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("S", [512, 1000])
def test_d256_contract_breaking_seq_pos(S, path):
    """seq_pos -1 and past max_seq - q_len: that sequence's cache is untouched and its
    output NaN; the others are unaffected."""
    sp = [-1, S // 2, S, S - 1]
    _say("d256 contract", S, path, sp)
    inp = gu.make_case(4, 1, 16, 2, S, sp, seed=16, head_dim=256, gate=True)
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    p = _problem(inp)
    out = gu.run_step(p, inp, path=path)
    torch.cuda.synchronize()
    kc, vc = bits(inp["k_cache"]), bits(inp["v_cache"])
    for b in (0, 2):
        assert np.array_equal(kc[b], kc0[b]) and np.array_equal(vc[b], vc0[b])
        assert torch.isnan(out[b].float()).all()
    good = [1, 3]
    sub = lambda x: np.ascontiguousarray(x[good])  # noqa: E731
    spg = np.asarray(sp, dtype=np.int32)[good]
    k_ref, v_ref = gu.oracle.kv_append(sub(kc0), sub(vc0), sub(bits(inp["k_new"])), sub(bits(inp["v_new"])), spg)
    assert np.array_equal(kc[good], k_ref) and np.array_equal(vc[good], v_ref)
    ref = gu.oracle.gqa_decode(sub(bits(inp["q"])), k_ref, v_ref, spg, gu.oracle.BF16)
    ref = gu.oracle.output_gate(ref, sub(bits(inp["out_gate"])), gu.oracle.BF16)
    gu.compare_out(out[good], ref)


@pytest.mark.parametrize("q_len,S,merge,fused", [(1, 512, "launch", True), (1, 4096, "launch", True),
                                                 (1, 4096, None, False), (4, 4096, "launch", False)])
def test_d256_decode_loop(q_len, S, merge, fused):
    """Consecutive steps through one workspace with fresh q, gate and new rows; the
    merge inside the attention launch (forced), or the separate one (automatic for
    4 heads, and the only one for 32 rows x 16 chunks)."""
    B, Hq, Hkv = 2, 16, 2
    sp = np.asarray([S - 4 * q_len - 2, S // 3], np.int32)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, sp, torch.float16, seed=S, head_dim=256, gate=True)
    freqs = rope_freqs(64, 1.0e7, "cuda")
    p = _problem(inp, freqs, 64, merge=merge)
    assert da.plan_attention(p)["fused_combine"] == fused
    ws = da.new_workspace(p)
    gen = torch.Generator(device="cpu").manual_seed(S)
    for it in range(4):
        _say("d256 loop", q_len, S, it, sp.tolist())
        if it:
            for k in ("q", "k_new", "v_new", "out_gate"):
                inp[k].copy_(torch.randn(inp[k].shape, generator=gen).to(torch.float16))
            inp["seq_pos"] = torch.as_tensor(sp).cuda()
        gu.check_full(p, inp, freqs=freqs, paths=("step",), ws=ws)
        sp = np.minimum(sp + q_len, S - q_len).astype(np.int32)


def test_d256_workload_layer():
    """The Qwen3.5 full-attention workload at full size: whole caches, every output row
    of layer 0, sampled rows of layer 9."""
    w = WORKLOADS["qwen35_gqa16x2_d256_gated_b16_ctx8192_10l"]
    freqs = rope_freqs(w.rope_dim, w.rope_theta, "cuda")
    _say(w.name, "layer 0")
    inp = make_layer(w, 0, "cuda")
    p = _problem(inp, freqs, w.rope_dim)
    stats = gu.check_full(p, inp, freqs=freqs)
    _say(w.name, da.plan_attention(p), stats)
    del inp, p
    inp = make_layer(w, 9, "cuda")
    p = _problem(inp, freqs, w.rope_dim)
    rng = np.random.default_rng(9)
    rows = np.stack([rng.integers(0, w.batch, 48), np.zeros(48, int), rng.integers(0, w.n_q_heads, 48)], 1)
    _say(w.name, "layer 9 sampled rows")
    gu.check_full(p, inp, freqs=freqs, rows=rows)


# ------------------------------------------------------------------ head_dim 128 with the new features

@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,seq_pos,variant", [
    (2, 1, 16, 8, 700, [699, 345], None),          # vector ALU, 2 rows
    (2, 1, 64, 8, 1500, [1499, 600], None),        # MFMA, 8 rows
    (2, 4, 32, 4, 900, [896, 77], None),           # MFMA, 32 rows
    (2, 4, 8, 8, 700, [600, 61], "valu"),          # vector ALU, 4 draft tokens
])
def test_d128_gate_and_partial_rope(B, q_len, Hq, Hkv, S, seq_pos, variant):
    _say("d128 gate rope64", B, q_len, Hq, Hkv, S, seq_pos, variant)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, seed=S + 3, gate=True)
    freqs = rope_freqs(64, 1.0e6, "cuda")
    p = _problem(inp, freqs, 64, variant=variant)
    gu.check_full(p, inp, freqs=freqs)


def test_d128_gate_paged():
    inp = make_paged(3, 1, 16, 8, 50, [799, 3, 400], seed=11, gate=True)
    p = _problem(inp)
    gu.check_full(p, inp)
