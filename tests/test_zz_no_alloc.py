"""The allocation-free step, da_decode_step_static, called through the C ABI
against da_decode_step on the same inputs: the caches bit for bit, the outputs
bit for bit (same kernels, same chunking), and the outputs within the oracle's
tolerance.  Calls in a row on one GPU, each with a smaller problem than the one
before, so each starts from the scratch the previous call left behind."""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_append_amd as da
import oracle
from tests import gpu_util as gu
from tests.oracle_pins import bits

pytestmark = pytest.mark.gpu

# (B, q_len, Hq, Hkv, max_seq, seq_pos, dtype, merge): the matrix-core kernel with
# the merge forced into the launch (several chunks per head), the same kernel with
# its automatic separate combine launch, then a smaller vector-ALU case.
CASES = [
    (4, 1, 64, 8, 6000, [5999, 4100, 3000, 5500], torch.bfloat16, "launch"),
    (2, 1, 64, 8, 3000, [2999, 1537], torch.bfloat16, None),
    (1, 2, 16, 8, 700, [640], torch.float16, None),
]


def _case(c, seed):
    B, q_len, Hq, Hkv, S, sp, dt, _ = c
    return gu.make_case(B, q_len, Hq, Hkv, S, sp, dtype=dt, seed=seed)


def _clone(inp):
    return {k: v.clone() for k, v in inp.items()}


def _same_bits(a, b):
    """Equal bit patterns (page pools hold NaN in their unused pages)."""
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_static_step_matches_workspace_step_twice():
    for n, c in enumerate(CASES):
        print(f"[no-alloc] call {n}: B, q_len, Hq, Hkv, max_seq, seq_pos = {c[:6]}", flush=True)
        inp = _case(c, seed=900 + n)
        ref_inp, st_inp = _clone(inp), _clone(inp)
        p = da.problem_for(inp["q"], inp["k_cache"], merge=c[7])
        out_ws = gu.run_step(p, ref_inp)
        out_st = torch.empty_like(out_ws)
        da.decode_step_static(p, st_inp["q"], st_inp["k_cache"], st_inp["v_cache"], st_inp["k_new"],
                              st_inp["v_new"], st_inp["seq_pos"], out_st)
        torch.cuda.synchronize()
        assert torch.equal(st_inp["k_cache"], ref_inp["k_cache"]) and torch.equal(st_inp["v_cache"], ref_inp["v_cache"])
        assert torch.equal(out_st.view(torch.int16), out_ws.view(torch.int16)), f"call {n}: outputs differ"
        # and the oracle: append bit for bit, attention within the tolerance
        dt = gu.odt(inp["q"].dtype)
        sp = inp["seq_pos"].cpu().numpy()
        k_ref, v_ref = oracle.kv_append(bits(inp["k_cache"]), bits(inp["v_cache"]), bits(inp["k_new"]),
                                        bits(inp["v_new"]), sp)
        assert np.array_equal(bits(st_inp["k_cache"]), k_ref) and np.array_equal(bits(st_inp["v_cache"]), v_ref)
        ref = oracle.gqa_decode(bits(inp["q"]), k_ref, v_ref, sp, dt)
        gu.compare_out(out_st, ref, f"static step, call {n}")


def test_static_step_repeats_bit_for_bit():
    """The scratch's counters return to zero: the same step again gives the same bits."""
    c = CASES[0]
    print(f"[no-alloc] repeat: {c[:6]}", flush=True)
    inp = _case(c, seed=77)
    p = da.problem_for(inp["q"], inp["k_cache"], merge=c[7])
    outs = []
    for _ in range(3):
        out = torch.empty_like(inp["q"])
        da.decode_step_static(p, inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"],
                              inp["seq_pos"], out)
        outs.append(out)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_static_step_random_problems_in_a_row():
    """The random problems of the parity sweep, one after another through
    da_decode_step_static (each call starting from the scratch the one before left
    behind), against da_decode_step on the same inputs bit for bit; a problem whose
    partials do not fit the scratch is refused before anything is enqueued, with the
    caches untouched."""
    from tests.test_gpu_random import N_CASES, case_inputs, spec
    ran = 0
    for i in range(N_CASES):
        s = spec(i)
        print(f"[no-alloc] random case {i}: {s}", flush=True)
        inp, _, p = case_inputs(s)
        ref_inp, st_inp = _clone(inp), _clone(inp)
        out_st = torch.empty_like(inp["q"])
        status = da.lib.da_decode_step_static(
            ctypes.byref(p), st_inp["q"].data_ptr(), st_inp["k_cache"].data_ptr(), st_inp["v_cache"].data_ptr(),
            st_inp["k_new"].data_ptr(), st_inp["v_new"].data_ptr(),
            ctypes.cast(st_inp["seq_pos"].data_ptr(), ctypes.POINTER(ctypes.c_int32)), out_st.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
        if status == da.DA_ERR_SCRATCH_LIMIT:
            torch.cuda.synchronize()
            assert _same_bits(st_inp["k_cache"], inp["k_cache"]) and _same_bits(st_inp["v_cache"], inp["v_cache"])
            continue
        assert status == da.DA_OK, da.status_str(status)
        out_ws = gu.run_step(p, ref_inp)
        torch.cuda.synchronize()
        assert _same_bits(st_inp["k_cache"], ref_inp["k_cache"]), f"case {i}: k caches differ"
        assert _same_bits(st_inp["v_cache"], ref_inp["v_cache"]), f"case {i}: v caches differ"
        assert _same_bits(out_st, out_ws), f"case {i}: outputs differ"
        ran += 1
    print(f"[no-alloc] {ran} of {N_CASES} random cases fit the scratch", flush=True)
    assert ran >= N_CASES // 2, f"only {ran} of {N_CASES} cases fit the scratch"


@pytest.mark.parametrize("name", ["verify4_gqa32x4_b8_pos2048_8188", "qwen35_gqa16x2_d256_gated_b16_ctx8192_10l"])
def test_static_step_full_size_workloads(name):
    """The two workloads whose partials take the most scratch (their separate-call
    workspaces, 32.5 and 32.3 MiB), one full-size layer each (the head_dim-256 one
    with its rotary table and gate), against da_decode_step bit for bit."""
    from decode_attention_append_amd.workloads import WORKLOADS, make_layer, rope_freqs
    w = WORKLOADS[name]
    print(f"[no-alloc] full size: {name}", flush=True)
    inp = make_layer(w, 0, "cuda")
    freqs = rope_freqs(w.rope_dim or w.head_dim, w.rope_theta, "cuda") if w.rope_theta > 0 else None
    p = da.problem(w.batch, w.q_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_seq, w.dtype,
                   rope_freqs=freqs, rope_dim=w.rope_dim, out_gate=inp.get("out_gate"))
    ref_inp, st_inp = _clone(inp), _clone(inp)
    out_ws = gu.run_step(p, ref_inp)
    out_st = torch.empty_like(out_ws)
    da.decode_step_static(p, st_inp["q"], st_inp["k_cache"], st_inp["v_cache"], st_inp["k_new"], st_inp["v_new"],
                          st_inp["seq_pos"], out_st)
    torch.cuda.synchronize()
    assert _same_bits(st_inp["k_cache"], ref_inp["k_cache"]) and _same_bits(st_inp["v_cache"], ref_inp["v_cache"])
    assert _same_bits(out_st, out_ws), f"{name}: outputs differ"
