"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

KV caches must match the oracle's append bit for bit over the whole
allocation; outputs must satisfy |gpu - oracle| <= 1e-2 + 1e-2 |oracle|
elementwise.  Unless a test says otherwise, every case runs both through the
three separate calls and through the one-launch da_decode_step.
"""
import numpy as np
import pytest
import torch

import decode_attention_append_amd as da
import oracle
from decode_attention_append_amd.workloads import WORKLOADS, make_layer
from tests import gpu_util as gu
from tests.oracle_pins import bits

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("name", [
    "qwen3_0p6b_b1_ctx512",
    "gqa64x8_b4_ctx12k_16k",
    "verify4_gqa32x4_b8_pos2048_8188",
])
def test_workload_full(name):
    w = WORKLOADS[name]
    _say(name, "layer 0, every output row")
    inp = make_layer(w, 0, "cuda")
    p = da.problem_for(inp["q"], inp["k_cache"])
    stats = gu.check_layer(p, inp)
    _say(name, da.plan_attention(p), stats)


def test_workload_mha_fp16_layers():
    w = WORKLOADS["qwen15moe_mha16_b1_ctx4096_24l"]
    for layer in (0, 1, 23):
        _say(w.name, "layer", layer)
        inp = make_layer(w, layer, "cuda")
        p = da.problem_for(inp["q"], inp["k_cache"])
        stats = gu.check_layer(p, inp)
        _say(w.name, layer, stats)


def test_workload_batched_gqa_ctx8192():
    """Full size (1 GiB caches per layer): whole cache bit-exact; all rows of layer 0,
    sampled rows of layer 27."""
    w = WORKLOADS["gqa16x8_b32_ctx8192_28l"]
    _say(w.name, "layer 0 all rows")
    inp = make_layer(w, 0, "cuda")
    p = da.problem_for(inp["q"], inp["k_cache"])
    gu.check_layer(p, inp)
    del inp
    _say(w.name, "layer 27 sampled rows")
    inp = make_layer(w, 27, "cuda")
    rng = np.random.default_rng(27)
    rows = np.stack([rng.integers(0, w.batch, 64), np.zeros(64, int),
                     rng.integers(0, w.n_q_heads, 64)], axis=1)
    gu.check_layer(p, inp, rows=rows)


# ------------------------------------------------------------------ shapes and edges

@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,seq_pos,dtype", [
    (3, 1, 16, 8, 700, [0, 333, 699], torch.bfloat16),          # ragged, tail not a tile multiple
    (2, 1, 16, 16, 1000, [999, 64], torch.float16),              # MHA fp16
    (2, 1, 64, 8, 3000, [2999, 1537], torch.bfloat16),           # GQA 8 (rows 8)
    (2, 1, 32, 8, 1200, [1199, 100], torch.bfloat16),            # rows 4
    (2, 2, 24, 2, 600, [598, 255], torch.bfloat16),              # rows 24 -> MFMA
    (2, 3, 12, 3, 900, [10, 896], torch.float16),                # rows 12 -> VALU 16-wide
    (3, 4, 32, 4, 2100, [2096, 0, 1023], torch.bfloat16),        # verify 4 -> MFMA
    (2, 4, 32, 4, 2100, [2096, 777], torch.float16),             # MFMA fp16
    (2, 8, 4, 2, 500, [492, 3], torch.bfloat16),                 # q_len 8 rows 16 -> MFMA
    (2, 8, 2, 2, 500, [492, 61], torch.bfloat16),                # q_len 8 MHA rows 8 -> MFMA
    (2, 4, 8, 8, 700, [696, 300], torch.bfloat16),               # q_len 4 MHA rows 4 -> VALU
    (1, 1, 1, 1, 64, [63], torch.bfloat16),                      # smallest
])
def test_shapes(B, q_len, Hq, Hkv, S, seq_pos, dtype):
    _say("shape", B, q_len, Hq, Hkv, S, seq_pos, dtype)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, dtype, seed=B * 1000 + S)
    p = da.problem_for(inp["q"], inp["k_cache"])
    gu.check_layer(p, inp)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,seq_pos,dtype", [
    (2, 1, 64, 8, 3000, [2999, 1537], torch.bfloat16),           # rows 8
    (2, 1, 16, 8, 700, [0, 699], torch.bfloat16),                # rows 2
    (2, 1, 16, 16, 1000, [999, 64], torch.float16),              # rows 1, fp16
    (2, 2, 32, 4, 900, [898, 250], torch.bfloat16),              # rows 16, causal
    (2, 3, 12, 3, 900, [10, 896], torch.float16),                # rows 12, causal
])
def test_forced_variant(variant, B, q_len, Hq, Hkv, S, seq_pos, dtype):
    """Both attention kernels agree with the oracle on every shape they both accept."""
    _say("variant", variant, B, q_len, Hq, Hkv, S, seq_pos, dtype)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, dtype, seed=S + q_len)
    p = da.problem_for(inp["q"], inp["k_cache"], variant=variant)
    assert da.plan_attention(p)["variant"] == variant
    gu.check_layer(p, inp)


@pytest.mark.parametrize("chunk", [64, 128, 256, 512, 1024, 2048])
@pytest.mark.parametrize("q_len,Hq,Hkv", [(1, 16, 8), (1, 64, 8), (4, 32, 4)])
def test_chunk_sweep(chunk, q_len, Hq, Hkv):
    """Every chunk size agrees with the oracle: pins the split and the combine."""
    _say("chunk", chunk, q_len, Hq, Hkv)
    inp = gu.make_case(2, q_len, Hq, Hkv, 2500, [2500 - q_len, 1300], seed=chunk)
    p = da.problem_for(inp["q"], inp["k_cache"], chunk_tokens=chunk)
    gu.check_layer(p, inp)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("q_len,Hq,Hkv", [(1, 16, 8), (1, 64, 8), (4, 32, 4), (1, 16, 16)])
def test_one_key_returns_value_exactly(q_len, Hq, Hkv, path):
    """seq_pos 0: query token 0 sees only its own key, so its output is v_new exactly."""
    _say("one key", q_len, Hq, Hkv, path)
    inp = gu.make_case(2, q_len, Hq, Hkv, 128, [0, 0], seed=5)
    p = da.problem_for(inp["q"], inp["k_cache"])
    out = gu.run_step(p, inp, path=path)
    G = Hq // Hkv
    expect = inp["v_new"][:, 0].repeat_interleave(G, dim=1)  # [B, Hq, D]
    assert torch.equal(out[:, 0], expect)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("q_len,Hq,Hkv", [(1, 16, 8), (1, 64, 8), (4, 32, 4)])
def test_constant_values_return_value_exactly(q_len, Hq, Hkv, path):
    S = 3000
    _say("constant V", q_len, Hq, Hkv, path)
    inp = gu.make_case(2, q_len, Hq, Hkv, S, [S - q_len, 1777], seed=6)
    row = inp["v_cache"][0, 0, 0].clone()
    inp["v_cache"][:] = row
    inp["v_new"][:] = row
    p = da.problem_for(inp["q"], inp["k_cache"])
    out = gu.run_step(p, inp, path=path)
    assert torch.equal(out, row.expand_as(out))


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("q_len,Hq,Hkv", [(1, 16, 8), (1, 64, 8), (4, 32, 4), (1, 16, 16)])
def test_beyond_context_poison(q_len, Hq, Hkv, path):
    """Cache slots at or past seq_pos + q_len hold NaN/inf, and so do the slots the
    step appends to before it writes them: the output must not change."""
    S = 1500
    sp = [700, 1500 - q_len, 63]
    _say("poison", q_len, Hq, Hkv, path)
    inp = gu.make_case(3, q_len, Hq, Hkv, S, sp, seed=7)
    clean = {k: v.clone() for k, v in inp.items()}
    p = da.problem_for(inp["q"], inp["k_cache"])
    out_clean = gu.run_step(p, clean, path=path)
    for b, s in enumerate(sp):
        inp["k_cache"][b, :, s:] = float("nan")
        inp["v_cache"][b, :, s:] = float("inf")
    out = gu.run_step(p, inp, path=path)
    assert torch.equal(out, out_clean)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("path", gu.PATHS)
def test_later_draft_token_hidden_from_earlier_rows_valu(path):
    """A NaN value row of the second draft token leaves query token 0's rows finite
    (vector-ALU variant: the mask excludes the row exactly)."""
    q_len, Hq, Hkv = 2, 8, 2
    inp = gu.make_case(1, q_len, Hq, Hkv, 256, [100], seed=8)
    p = da.problem_for(inp["q"], inp["k_cache"], variant="valu")
    assert da.plan_attention(p)["variant"] == "valu"
    inp["v_new"][0, 1] = float("nan")
    out = gu.run_step(p, inp, path=path)
    assert torch.isfinite(out[:, 0].float()).all()
    assert torch.isnan(out[:, 1].float()).all()


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("bad", ["nan", "inf"])
@pytest.mark.parametrize("hidden_from", [1, "last"])
@pytest.mark.parametrize("B,q_len,Hq,Hkv,D,S,seq_pos", [
    (2, 4, 32, 4, 128, 512, [30, 300]),   # 32 rows: two row blocks; new rows straddle a 32-key tile
    (2, 4, 16, 4, 128, 512, [61, 200]),   # 16 rows: one row block
    (1, 2, 32, 8, 128, 256, [100]),       # 8 rows
    (2, 4, 16, 2, 256, 512, [14, 300]),   # head_dim 256, 32 rows (two row groups); straddles a 16-key tile
    (2, 2, 16, 2, 256, 512, [14, 300]),   # head_dim 256, 16 rows
])
def test_later_draft_token_hidden_from_earlier_rows_mfma(B, q_len, Hq, Hkv, D, S, seq_pos, hidden_from, bad, path):
    """A non-finite value row of a later draft token reaches only the rows that see
    it: every earlier token's rows stay finite and equal the oracle's (which
    excludes the hidden key), on the matrix-core kernels."""
    i_bad = 1 if hidden_from == 1 else q_len - 1
    _say("draft", B, q_len, Hq, Hkv, D, S, seq_pos, i_bad, bad, path)
    inp = gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, seed=31 + i_bad, head_dim=D)
    p = da.problem_for(inp["q"], inp["k_cache"])
    assert da.plan_attention(p)["variant"] == "mfma"
    inp["v_new"][:, i_bad] = float(bad)
    dt = gu.odt(inp["q"].dtype)
    sp = inp["seq_pos"].cpu().numpy()
    k_ref, v_ref = oracle.kv_append(bits(inp["k_cache"]), bits(inp["v_cache"]), bits(inp["k_new"]),
                                    bits(inp["v_new"]), sp)
    ref = oracle.gqa_decode(bits(inp["q"]), k_ref, v_ref, sp, dt)
    out = gu.run_step(p, inp, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(bits(inp["k_cache"]), k_ref) and np.array_equal(bits(inp["v_cache"]), v_ref)
    assert torch.isfinite(out[:, :i_bad].float()).all()
    gu.compare_out(out[:, :i_bad], ref[:, :i_bad], "tokens before the bad draft row")
    assert not torch.isfinite(out[:, i_bad:].float()).any()


def test_last_slot_and_exact_chunk_boundaries():
    """Contexts that end exactly on, one before and one after chunk boundaries."""
    S = 1024
    for chunk in (64, 256):
        sp = [chunk - 1, chunk, chunk - 2, S - 1]
        _say("boundaries", chunk, sp)
        inp = gu.make_case(4, 1, 16, 8, S, sp, seed=9)
        p = da.problem_for(inp["q"], inp["k_cache"], chunk_tokens=chunk)
        gu.check_layer(p, inp)


def test_long_context_max_cache():
    """A 128k-slot cache with one long sequence and one short one."""
    S = 131072
    _say("long", S)
    inp = gu.make_case(2, 1, 16, 8, S, [S - 1, 5000], seed=10)
    p = da.problem_for(inp["q"], inp["k_cache"])
    rows = np.array([[0, 0, h] for h in range(16)] + [[1, 0, h] for h in range(0, 16, 5)])
    gu.check_layer(p, inp, rows=rows)


def test_custom_scale():
    _say("scale")
    inp = gu.make_case(2, 1, 16, 8, 600, [599, 300], seed=11)
    p = da.problem_for(inp["q"], inp["k_cache"], scale=0.3)
    gu.check_layer(p, inp)


# ------------------------------------------------------------------ the ABI on the GPU

def test_variant_choice():
    assert da.plan_attention(da.problem(8, 4, 32, 4, 128, 8192, "bf16"))["variant"] == "mfma"
    assert da.plan_attention(da.problem(4, 1, 64, 8, 128, 16384, "bf16"))["variant"] == "mfma"
    assert da.plan_attention(da.problem(1, 2, 8, 1, 128, 64, "bf16"))["variant"] == "mfma"
    assert da.plan_attention(da.problem(1, 1, 15, 1, 128, 64, "bf16"))["variant"] == "mfma"
    assert da.plan_attention(da.problem(1, 1, 7, 1, 128, 64, "bf16"))["variant"] == "valu"
    # under 8 rows: matrix cores for fewer than 128 heads with at least 1024 slots
    assert da.plan_attention(da.problem(4, 1, 32, 8, 128, 16384, "bf16"))["variant"] == "mfma"
    assert da.plan_attention(da.problem(1, 1, 16, 16, 128, 4096, "fp16"))["variant"] == "mfma"
    assert da.plan_attention(da.problem(1, 1, 16, 8, 128, 512, "bf16"))["variant"] == "valu"
    assert da.plan_attention(da.problem(16, 1, 16, 8, 128, 4096, "bf16"))["variant"] == "valu"


def test_errors_launch_nothing():
    """Host-checkable errors return a status and enqueue nothing: the cache is untouched."""
    import ctypes
    inp = gu.make_case(2, 1, 16, 8, 256, [10, 20], seed=12)
    before_k, before_v = inp["k_cache"].clone(), inp["v_cache"].clone()
    good = da.problem_for(inp["q"], inp["k_cache"])
    bad_dim = da.problem_for(inp["q"], inp["k_cache"])
    bad_dim.head_dim = 64
    ptr = {k: v.data_ptr() for k, v in inp.items()}

    def append(prob, k_off=0):
        return da.lib.da_kv_append(ctypes.byref(prob), ptr["k_cache"] + k_off, ptr["v_cache"],
                                   ptr["k_new"], ptr["v_new"], ptr["seq_pos"], None)

    assert append(bad_dim) == da.DA_ERR_UNSUPPORTED
    assert append(good, k_off=2) == da.DA_ERR_INVALID_ARG  # misaligned cache pointer
    ws = da.new_workspace(good)
    st = da.lib.da_gqa_decode_attn(ctypes.byref(good), ptr["q"], ptr["k_cache"], ptr["v_cache"],
                                   ptr["seq_pos"], ws.data_ptr(), ws.numel() - 1, None)
    assert st == da.DA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(inp["k_cache"], before_k) and torch.equal(inp["v_cache"], before_v)


def test_non_default_stream_ordering():
    """Append, attention and combine enqueued on a side stream behind a long copy."""
    inp = gu.make_case(4, 1, 16, 8, 4096, [4095, 100, 2000, 3000], seed=13)
    p = da.problem_for(inp["q"], inp["k_cache"])
    s = torch.cuda.Stream()
    big = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        big.fill_(1)  # keeps the stream busy before the step starts
        stats = gu.check_layer(p, inp, stream=s)
    torch.cuda.synchronize()
    _say("side stream", stats)


def test_kernel_reads_caller_data():
    """Two steps on different caches through the same workspace give each its own answer."""
    a = gu.make_case(1, 1, 16, 8, 512, [511], seed=14)
    b = gu.make_case(1, 1, 16, 8, 512, [511], seed=15)
    p = da.problem_for(a["q"], a["k_cache"])
    ws = da.new_workspace(p)
    outs = []
    for inp in (a, b):
        out = torch.empty_like(inp["q"])
        da.decode_step(p, inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"],
                       inp["seq_pos"], ws, out)
        outs.append(out)
    torch.cuda.synchronize()
    assert not torch.equal(outs[0], outs[1])
    for inp, out in zip((a, b), outs):
        ref = gu.oracle.gqa_decode(bits(inp["q"]), bits(inp["k_cache"]), bits(inp["v_cache"]),
                                   inp["seq_pos"].cpu().numpy(), gu.oracle.BF16)
        gu.compare_out(out, ref)


# ------------------------------------------------------------------ the one-launch step

@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,sp0,merge,fused", [
    (3, 1, 16, 8, 3000, [2990, 100, 1500], None, True),       # MFMA (few heads), 2 rows: merge in the launch
    (3, 1, 16, 8, 1000, [990, 100, 500], None, True),         # vector ALU, merge in the launch
    (1, 1, 64, 8, 512, [500], "launch", True),                # MFMA, 8 rows, merge in the launch
    (4, 1, 64, 8, 16384, [15000, 12288, 16380, 13000], "launch", True),  # MFMA, 8 rows x 16 chunks
    (4, 1, 64, 8, 16384, [15000, 12288, 16380, 13000], None, False),     # the same, separate merge
    (16, 1, 64, 8, 1024, [1000, 10, 600, 1023] * 4, None, True),         # MFMA, 128 heads: in the launch
    (2, 4, 32, 4, 2100, [2000, 60], "launch", False),         # MFMA, 32 rows, separate merge
    (2, 4, 8, 8, 700, [600, 61], None, True),                 # vector ALU, 4 draft tokens
])
def test_decode_loop_reuses_workspace(B, q_len, Hq, Hkv, S, sp0, merge, fused):
    """Consecutive steps through one workspace (its arrival counters must return to
    zero after every step), the cache growing by q_len per step and fresh q / new
    rows each step, checked against the oracle step by step."""
    p = da.problem(B, q_len, Hq, Hkv, 128, S, "bf16", merge=merge)
    assert da.plan_attention(p)["fused_combine"] == fused
    inp = gu.make_case(B, q_len, Hq, Hkv, S, sp0, seed=S + B)
    ws = da.new_workspace(p)
    k_ref, v_ref = bits(inp["k_cache"]), bits(inp["v_cache"])
    sp = np.asarray(sp0, dtype=np.int32)
    gen = torch.Generator(device="cpu").manual_seed(S)
    for it in range(4):
        _say("decode loop", B, q_len, Hq, Hkv, S, "step", it, sp.tolist())
        if it:
            for k in ("q", "k_new", "v_new"):
                inp[k] = torch.randn(inp[k].shape, generator=gen).to(torch.bfloat16).cuda()
            inp["seq_pos"] = torch.as_tensor(sp).cuda()
        out = gu.run_step(p, inp, ws=ws)
        torch.cuda.synchronize()
        k_ref, v_ref = gu.oracle.kv_append(k_ref, v_ref, bits(inp["k_new"]), bits(inp["v_new"]), sp)
        assert np.array_equal(bits(inp["k_cache"]), k_ref), f"step {it}: k_cache"
        assert np.array_equal(bits(inp["v_cache"]), v_ref), f"step {it}: v_cache"
        ref = gu.oracle.gqa_decode(bits(inp["q"]), k_ref, v_ref, sp, gu.oracle.BF16)
        gu.compare_out(out, ref, f"step {it}")
        sp = np.minimum(sp + q_len, S - q_len).astype(np.int32)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("q_len,Hq,Hkv,S", [(1, 16, 8, 1000), (1, 64, 8, 1000), (1, 64, 8, 512),
                                            (4, 32, 4, 1000)])
def test_contract_breaking_seq_pos(q_len, Hq, Hkv, S, path):
    """seq_pos -1 and seq_pos past max_seq - q_len: that sequence's cache is untouched
    and its output rows are NaN; the other sequences are unaffected (merged in the
    attention launch or by the separate combine)."""
    sp = [-1, S // 2, S - q_len + 1, S - q_len]
    _say("contract", q_len, Hq, Hkv, path, sp)
    inp = gu.make_case(4, q_len, Hq, Hkv, S, sp, seed=16)
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    p = da.problem_for(inp["q"], inp["k_cache"])
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
    gu.compare_out(out[good], ref)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("Hq,Hkv,D,work_items", [
    (64, 8, 128, 0),      # MFMA, 8 rows
    (32, 8, 128, 0),      # vector ALU, 4 rows
    (16, 2, 256, 0),      # head_dim 256
    (64, 8, 128, 77),     # a chunk target that is not a power of two
    (32, 8, 128, 1000),   # many short chunks
])
def test_many_sequences(Hq, Hkv, D, work_items, path):
    """130 sequences: every workgroup walks three 64-sequence groups of positions to find
    its chunk, with ragged contexts and three contract-breaking positions (their caches
    untouched, their rows NaN)."""
    B, S = 130, 400
    rng = np.random.default_rng(D + Hq + work_items)
    sp = rng.integers(0, S, B).astype(np.int32)
    sp[[3, 64, 129]] = [-1, S, S + 7]
    sp[[0, 63, 65, 128]] = [S - 1, 0, S - 1, 1]
    _say("many sequences", Hq, Hkv, D, work_items, path)
    inp = gu.make_case(B, 1, Hq, Hkv, S, sp, seed=29, head_dim=D)
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    p = da.problem_for(inp["q"], inp["k_cache"], work_items=work_items)
    out = gu.run_step(p, inp, path=path)
    torch.cuda.synchronize()
    kc, vc = bits(inp["k_cache"]), bits(inp["v_cache"])
    bad = [3, 64, 129]
    for b in bad:
        assert np.array_equal(kc[b], kc0[b]) and np.array_equal(vc[b], vc0[b])
        assert torch.isnan(out[b].float()).all()
    good = [b for b in range(B) if b not in bad]
    sub = lambda x: np.ascontiguousarray(x[good])  # noqa: E731
    spg = sp[good]
    k_ref, v_ref = gu.oracle.kv_append(sub(kc0), sub(vc0), sub(bits(inp["k_new"])), sub(bits(inp["v_new"])), spg)
    assert np.array_equal(kc[good], k_ref) and np.array_equal(vc[good], v_ref)
    ref = gu.oracle.gqa_decode(sub(bits(inp["q"])), k_ref, v_ref, spg, gu.oracle.BF16)
    gu.compare_out(out[good], ref)


def test_decode_step_errors_launch_nothing():
    import ctypes
    inp = gu.make_case(2, 1, 16, 8, 256, [10, 20], seed=17)
    before_k = inp["k_cache"].clone()
    p = da.problem_for(inp["q"], inp["k_cache"])
    ws = da.new_workspace(p)
    out = torch.zeros_like(inp["q"])
    ptr = {k: v.data_ptr() for k, v in inp.items()}

    def step(nbytes, out_ptr):
        return da.lib.da_decode_step(ctypes.byref(p), ptr["q"], ptr["k_cache"], ptr["v_cache"], ptr["k_new"],
                                     ptr["v_new"], ptr["seq_pos"], ws.data_ptr(), nbytes, out_ptr, None)

    assert step(ws.numel() - 1, out.data_ptr()) == da.DA_ERR_WORKSPACE
    assert step(ws.numel(), out.data_ptr() + 2) == da.DA_ERR_INVALID_ARG
    assert step(ws.numel(), None) == da.DA_ERR_INVALID_ARG
    assert da.lib.da_workspace_init(ctypes.byref(p), ws.data_ptr(), ws.numel() - 1, None) == da.DA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(inp["k_cache"], before_k) and not out.any()


# ------------------------------------------------------------------ vector-ALU long chunks

@pytest.mark.parametrize("B,Hq,Hkv,S,dtype,seed", [
    (16, 16, 8, 3000, torch.bfloat16, 1),     # 2 rows, 128 units, ragged: one chunk or several
    (128, 1, 1, 9000, torch.float16, 2),      # 1 row, 128 units, chunks up to 8192 keys
    (32, 8, 4, 1500, torch.bfloat16, 3),      # 2 rows, 128 units, short contexts
])
def test_valu_long_chunks(B, Hq, Hkv, S, dtype, seed):
    """At least 128 (sequence, KV head) units with up to 2 rows take chunks of up to 8192
    keys (two pages' worth of block-table entries per thread when paged); in the one-launch step a sequence that is one chunk writes its
    output directly, the others merge in the launch."""
    rng = np.random.default_rng(seed)
    sp = rng.integers(0, S, B).astype(np.int32)
    sp[0], sp[-1] = S - 1, 0
    _say("valu long chunks", B, Hq, Hkv, S, dtype)
    inp = gu.make_case(B, 1, Hq, Hkv, S, sp, dtype, seed=seed)
    p = da.problem_for(inp["q"], inp["k_cache"])
    pl = da.plan_attention(p)
    assert pl["variant"] == "valu" and pl["chunk_tokens"] == 8192 and pl["target_items"] == 256
    lay = da.chunk_layout(p, sp)
    assert any(n == 1 for n, _ in lay) and any(n > 1 for n, _ in lay)
    gu.check_layer(p, inp)



def test_valu_long_chunks_uneven_many_sequences():
    """130 sequences (three groups of 64 positions for every workgroup's chunk plan) whose
    contexts are so uneven that the long plan's longest chunk exceeds 5/4 of an equal
    share: every kernel switches to the plan for 1024 chunks, on every path."""
    B, S = 130, 400
    rng = np.random.default_rng(31)
    sp = rng.integers(0, 60, B).astype(np.int32)
    sp[[5, 70, 129]] = S - 1
    _say("valu long chunks, uneven, many sequences", B, S)
    inp = gu.make_case(B, 1, 16, 8, S, sp, seed=31)
    p = da.problem_for(inp["q"], inp["k_cache"])
    pl = da.plan_attention(p)
    assert pl["variant"] == "valu" and pl["target_items"] == 256 and pl["chunk_tokens"] == 8192
    lay = da.chunk_layout(p, sp)
    assert max(n for n, _ in lay) > 1  # the long sequences are split: the shorter plan
    gu.check_layer(p, inp)


def test_valu_merge_split_over_waves():
    """More than 16 chunks and fewer than 4 rows: the merge splits each row's chunks over the
    4 waves (fixed 64-key chunks)."""
    sp = [2047, 1500, 900, 64] * 16
    inp = gu.make_case(64, 1, 4, 2, 2048, sp, seed=4)
    p = da.problem_for(inp["q"], inp["k_cache"], chunk_tokens=64)
    assert da.plan_attention(p)["fused_combine"]
    gu.check_layer(p, inp)


@pytest.mark.parametrize("path", gu.PATHS)
def test_valu_long_chunks_rope_and_paged(path):
    from tests.test_gpu_paged import make_paged, check_paged
    from decode_attention_append_amd.workloads import rope_freqs
    freqs = rope_freqs(128, 1.0e6, "cuda")
    inp = make_paged(16, 1, 16, 8, 120, list(range(100, 1900, 113))[:16], seed=9)
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=inp["block_table"], rope_freqs=freqs)
    assert da.plan_attention(p)["chunk_tokens"] == 8192
    check_paged(p, inp, path, freqs=freqs)


def test_valu_long_chunks_decode_loop():
    B, S = 32, 2000
    p = da.problem(B, 1, 8, 4, 128, S, "bf16")  # 2 rows, 128 units
    assert da.plan_attention(p)["chunk_tokens"] == 8192
    sp = np.random.default_rng(6).integers(100, S - 8, B).astype(np.int32)
    inp = gu.make_case(B, 1, 8, 4, S, sp, seed=6)
    ws = da.new_workspace(p)
    k_ref, v_ref = bits(inp["k_cache"]), bits(inp["v_cache"])
    gen = torch.Generator(device="cpu").manual_seed(6)
    for it in range(4):
        _say("valu long chunks loop", it)
        if it:
            for k in ("q", "k_new", "v_new"):
                inp[k] = torch.randn(inp[k].shape, generator=gen).to(torch.bfloat16).cuda()
            inp["seq_pos"] = torch.as_tensor(sp).cuda()
        out = gu.run_step(p, inp, ws=ws)
        torch.cuda.synchronize()
        k_ref, v_ref = gu.oracle.kv_append(k_ref, v_ref, bits(inp["k_new"]), bits(inp["v_new"]), sp)
        assert np.array_equal(bits(inp["k_cache"]), k_ref) and np.array_equal(bits(inp["v_cache"]), v_ref)
        gu.compare_out(out, gu.oracle.gqa_decode(bits(inp["q"]), k_ref, v_ref, sp, gu.oracle.BF16), f"step {it}")
        sp = sp + 1
