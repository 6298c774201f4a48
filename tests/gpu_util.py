"""Helpers for the GPU parity tests: run the library through its C ABI, compare with the oracle."""
import numpy as np
import pytest
import torch

import decode_attention_append_amd as da
import oracle
from tests.oracle_pins import bits

ABS_TOL = 1e-2
REL_TOL = 1e-2


def odt(dtype) -> int:
    return oracle.FP16 if dtype == torch.float16 else oracle.BF16


# the three separate calls; da_decode_step as planned; da_decode_step with the merge
# forced into the attention launch (run only where that changes what is launched)
PATHS = ("separate", "step", "step_launch")


def with_merge(p, merge: str):
    """A copy of problem ``p`` with its merge override set ("launch" or "separate")."""
    q = type(p).from_buffer_copy(p)
    q.merge = {"launch": 1, "separate": 2}[merge]
    q._refs = getattr(p, "_refs", None)
    return q


def path_differs(p, path) -> bool:
    """False for "step_launch" when forcing the merge into the launch changes nothing
    (the plan already merges there, or cannot)."""
    if path != "step_launch":
        return True
    return da.plan_attention(with_merge(p, "launch"))["fused_combine"] != da.plan_attention(p)["fused_combine"]


def run_step(p, inp, stream=None, path="step", ws=None):
    """One decode step on the GPU through ``path``.  ``inp`` holds device tensors; the
    caches are updated in place.  Returns the output tensor (device)."""
    if path == "step_launch":
        p, path = with_merge(p, "launch"), "step"
    if ws is None:
        ws = da.new_workspace(p, stream=stream)
    out = torch.empty((p.batch, p.q_len, p.n_q_heads, p.head_dim), dtype=inp["q"].dtype,
                      device=inp["q"].device)
    fn = da.decode_step if path == "step" else da.decode_step_separate
    fn(p, inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["seq_pos"], ws, out,
       stream)
    return out


def compare_out(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    """Elementwise |got - ref| <= ABS_TOL + REL_TOL * |ref|; returns diagnostics."""
    g = got.detach().float().cpu().double().numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    diff = np.abs(g - ref)
    bound = ABS_TOL + REL_TOL * np.abs(ref)
    bad = ~(diff <= bound)  # NaN counts as bad
    stats = {
        "max_abs": float(np.nanmax(diff)) if diff.size else 0.0,
        "max_over_bound": float(np.nanmax(diff - REL_TOL * np.abs(ref))) if diff.size else 0.0,
        "rms": float(np.sqrt(np.nanmean(diff ** 2))) if diff.size else 0.0,
        "max_rel_to_max_ref": float(np.nanmax(diff) / max(np.nanmax(np.abs(ref)), 1e-30)) if diff.size else 0.0,
        "n_bad": int(bad.sum()),
    }
    assert stats["n_bad"] == 0, f"{what}: {stats['n_bad']} elements outside tolerance, {stats}"
    return stats


def check_layer(p, inp, rows=None, stream=None, paths=PATHS):
    """Runs a step through each of ``paths`` (each from the same starting caches; the
    last one updates ``inp`` in place), checks the whole cache bit for bit and the
    output against the oracle.

    rows: None for every output row, else an [n, 3] array of (b, i, hq) to check.
    Returns the output diagnostics of each path.
    """
    dt = odt(inp["q"].dtype)
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    kn, vn = bits(inp["k_new"]), bits(inp["v_new"])
    sp = inp["seq_pos"].cpu().numpy()
    k_ref, v_ref = oracle.kv_append(kc0, vc0, kn, vn, sp)
    del kc0, vc0
    qb = bits(inp["q"])
    scale = p.scale if p.scale > 0 else None
    if rows is None:
        ref = oracle.gqa_decode(qb, k_ref, v_ref, sp, dt, scale=scale)
    else:
        rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
        ref = oracle.gqa_decode_rows(qb, k_ref, v_ref, sp, rows, dt, scale=scale)
    stats = {}
    paths = [x for x in paths if path_differs(p, x)]
    if not paths:
        pytest.skip("forcing the merge into the attention launch changes nothing for this plan")
    for n, path in enumerate(paths):
        last = n == len(paths) - 1
        run = inp if last else dict(inp, k_cache=inp["k_cache"].clone(), v_cache=inp["v_cache"].clone())
        out = run_step(p, run, stream, path)
        torch.cuda.synchronize()
        assert np.array_equal(bits(run["k_cache"]), k_ref), f"{path}: k_cache differs from the oracle's append"
        assert np.array_equal(bits(run["v_cache"]), v_ref), f"{path}: v_cache differs from the oracle's append"
        if rows is None:
            stats[path] = compare_out(out, ref, f"{path}: all rows")
        else:
            o = out.cpu()
            got = torch.stack([o[b, i, hq] for b, i, hq in rows])
            stats[path] = compare_out(got, ref, f"{path}: sampled rows")
        del run, out
    return stats


def make_case(B, q_len, Hq, Hkv, S, seq_pos, dtype=torch.bfloat16, seed=0, scale=1.0,
              device="cuda", head_dim=128, gate=False):
    from decode_attention_append_amd.workloads import make_tensors
    t = make_tensors(B, q_len, Hq, Hkv, head_dim, S, dtype, seed, device, scale, gate=gate)
    sp = torch.as_tensor(np.asarray(seq_pos, dtype=np.int32)).to(device)
    out = {"q": t[0], "k_cache": t[1], "v_cache": t[2], "k_new": t[3], "v_new": t[4], "seq_pos": sp}
    if gate:
        out["out_gate"] = t[5]
    return out


def _ulp(ref, dt):
    mbits, emin = (10, -14) if dt == oracle.FP16 else (7, -126)
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** emin))) - mbits)


# Rotated K rows are an fp32 evaluation rounded once to 16 bits (the rotary
# embedding's precision reading): besides that rounding, the angle's reduction to
# a float fraction of a turn (up to 2 pi 2^-26 rad), the hardware sine and cosine
# and the fp32 products each err by a few 2^-24 of |x| + |y| for the pair (x, y)
# the element comes from.  Where x cos a - y sin a nearly cancels, that error is
# larger than one 16-bit ulp of the tiny result (measured worst: 1.1e-7 (|x| + |y|)
# over 600 random problems), so a rotated element may differ from the oracle by one
# ulp plus this slack.
ROPE_EVAL_SLACK = 2.0 ** -21


def rope_slack_rows(new, kn_raw, sp, q_len, R, dt, block_table=None):
    """[n, D] slack ROPE_EVAL_SLACK * (|x| + |y|) for the appended rows selected by the
    boolean row mask ``new`` (in its C order), from the pre-rotation new rows
    ``kn_raw`` [B, q_len, Hkv, D]; 0 on the dims past the rotary width R."""
    x = oracle.decode(kn_raw, dt)
    half = R // 2
    mag = np.zeros(x.shape)
    pm = np.abs(x[..., :half]) + np.abs(x[..., half:R])
    mag[..., :half] = pm
    mag[..., half:R] = pm
    src = {}
    for b, s in enumerate(sp):
        if s < 0 or (block_table is not None and (int(s) + q_len - 1) // 16 >= block_table.shape[1]):
            continue  # a sequence whose position breaks the contract appends nothing
        for i in range(q_len):
            t = int(s) + i
            src[(b, t) if block_table is None else (int(block_table[b, t // 16]), t % 16)] = (b, i)
    rows = []
    for a0, a1, a2 in zip(*np.nonzero(new)):
        b, i = src[(int(a0), int(a2))]
        rows.append(mag[b, i, a1])
    return ROPE_EVAL_SLACK * np.asarray(rows).reshape(-1, x.shape[-1])


def check_rotated_k(kg, k_ref, new, kn_raw, sp, q_len, R, dt, block_table=None, what=""):
    """The appended rows of a rotated K cache against the oracle's: within one ulp plus
    the fp32 evaluation slack on the rotated dims, bit for bit past them and outside
    the appended rows, and at most 1% of the appended elements not bit-identical.
    Returns that fraction."""
    d = kg != k_ref
    assert not d[~new].any(), f"{what}: k cache differs outside the appended rows"
    if not new.any():  # every sequence broke the contract: nothing was appended
        return 0.0
    a, r = oracle.decode(kg[new], dt), oracle.decode(k_ref[new], dt)
    slack = rope_slack_rows(new, kn_raw, sp, q_len, R, dt, block_table)
    assert (np.abs(a - r) <= _ulp(r, dt) + slack).all(), f"{what}: rotated K beyond one ulp and the fp32 slack"
    assert not d[new][:, R:].any(), f"{what}: K dims past the rotary width differ"
    frac = float(d[new].mean())
    assert frac <= 0.01, f"{what}: {frac:.4f} of rotated K off the oracle's bits"
    return frac


def appended_rows(kshape, sp, q_len, block_table=None):
    """Mask over the cache's (or pool's) rows [.., .., 16 or S] that the step appends."""
    m = np.zeros(kshape[:3], bool)
    for b, s in enumerate(sp):
        for i in range(q_len):
            if block_table is None:
                m[b, :, s + i] = True
            else:
                m[block_table[b, (s + i) // 16], :, (s + i) % 16] = True
    return m


def check_full(p, inp, freqs=None, rows=None, stream=None, paths=PATHS, ws=None):
    """check_layer for every feature of the step: optional rotary table (rope_dim from
    the table's length), paged caches (inp["block_table"]) and output gate
    (inp["out_gate"]; ``p`` must carry the same tensors).  V caches bit for bit; K
    caches bit for bit without a rotary table, else as check_rotated_k: the appended
    rows' rotated dims within one ulp plus the fp32 evaluation slack (at most 1% of
    their elements off the oracle's bits), bit for bit elsewhere."""
    dt = odt(inp["q"].dtype)
    sp = inp["seq_pos"].cpu().numpy()
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    kn, vn, qb = bits(inp["k_new"]), bits(inp["v_new"]), bits(inp["q"])
    kn_raw = kn
    bt = inp.get("block_table")
    bt = None if bt is None else bt.cpu().numpy()
    if freqs is not None:
        fr = freqs.cpu().numpy()
        pos = sp[:, None, None] + np.arange(p.q_len, dtype=np.int32)[None, :, None]
        kn = oracle.rope_rows(kn, np.broadcast_to(pos, kn.shape[:3]), fr, dt)
        qb = oracle.rope_q(qb, sp, fr, dt)
    if bt is None:
        k_ref, v_ref = oracle.kv_append(kc0, vc0, kn, vn, sp)
        kc, vc = k_ref, v_ref
    else:
        k_ref, v_ref = oracle.kv_append_paged(kc0, vc0, kn, vn, sp, bt)
        kc, vc = oracle.gather_paged(k_ref, bt), oracle.gather_paged(v_ref, bt)
    del kc0, vc0
    scale = p.scale if p.scale > 0 else None
    gate = inp.get("out_gate")
    gb = None if gate is None else bits(gate)
    if rows is None:
        ref = oracle.gqa_decode(qb, kc, vc, sp, dt, scale=scale)
    else:
        rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
        ref = oracle.gqa_decode_rows(qb, kc, vc, sp, rows, dt, scale=scale)
        if gb is not None:
            gb = np.ascontiguousarray(gb[rows[:, 0], rows[:, 1], rows[:, 2]])
    if gb is not None:
        ref = oracle.output_gate(ref, gb, dt)
    new = appended_rows(k_ref.shape, sp, p.q_len, bt)
    stats = {}
    paths = [x for x in paths if path_differs(p, x)]
    if not paths:
        pytest.skip("forcing the merge into the attention launch changes nothing for this plan")
    for n, path in enumerate(paths):
        last = n == len(paths) - 1
        run = inp if last else dict(inp, k_cache=inp["k_cache"].clone(), v_cache=inp["v_cache"].clone())
        out = run_step(p, run, stream, path, ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(run["v_cache"]), v_ref), f"{path}: v cache differs from the oracle's append"
        kg = bits(run["k_cache"])
        if freqs is None:
            assert np.array_equal(kg, k_ref), f"{path}: k cache differs from the oracle's append"
        else:
            check_rotated_k(kg, k_ref, new, kn_raw, sp, p.q_len, 2 * freqs.numel(), dt, bt, path)
        if rows is None:
            stats[path] = compare_out(out, ref, f"{path}: all rows")
        else:
            o = out.cpu()
            got = torch.stack([o[b, i, hq] for b, i, hq in rows])
            stats[path] = compare_out(got, ref, f"{path}: sampled rows")
        del run, out
    return stats
