"""Helpers for the GPU parity tests: run the library through its C ABI, compare with the oracle."""
import numpy as np
import torch

import decode_attention_append_amd as da
import oracle
from tests.oracle_pins import bits

ABS_TOL = 1e-2
REL_TOL = 1e-2


def odt(dtype) -> int:
    return oracle.FP16 if dtype == torch.float16 else oracle.BF16


def run_step(p, inp, stream=None):
    """One decode step on the GPU.  ``inp`` holds device tensors; the caches are
    updated in place.  Returns the output tensor (device)."""
    ws = da.new_workspace(p)
    out = torch.empty((p.batch, p.q_len, p.n_q_heads, p.head_dim), dtype=inp["q"].dtype,
                      device=inp["q"].device)
    da.decode_step(p, inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"],
                   inp["seq_pos"], ws, out, stream)
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


def check_layer(p, inp, rows=None, stream=None):
    """Runs a step; checks the whole cache bit for bit and the output against the oracle.

    rows: None for every output row, else an [n, 3] array of (b, i, hq) to check.
    Returns output diagnostics.
    """
    dt = odt(inp["q"].dtype)
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    kn, vn = bits(inp["k_new"]), bits(inp["v_new"])
    sp = inp["seq_pos"].cpu().numpy()
    out = run_step(p, inp, stream)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.kv_append(kc0, vc0, kn, vn, sp)
    del kc0, vc0
    assert np.array_equal(bits(inp["k_cache"]), k_ref), "k_cache differs from the oracle's append"
    assert np.array_equal(bits(inp["v_cache"]), v_ref), "v_cache differs from the oracle's append"
    qb = bits(inp["q"])
    if rows is None:
        ref = oracle.gqa_decode(qb, k_ref, v_ref, sp, dt, scale=p.scale if p.scale > 0 else None)
        return compare_out(out, ref, "all rows")
    rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
    ref = oracle.gqa_decode_rows(qb, k_ref, v_ref, sp, rows, dt,
                                 scale=p.scale if p.scale > 0 else None)
    o = out.cpu()
    got = torch.stack([o[b, i, hq] for b, i, hq in rows])
    return compare_out(got, ref, "sampled rows")


def make_case(B, q_len, Hq, Hkv, S, seq_pos, dtype=torch.bfloat16, seed=0, scale=1.0,
              device="cuda"):
    from decode_attention_append_amd.workloads import make_tensors
    q, kc, vc, kn, vn = make_tensors(B, q_len, Hq, Hkv, 128, S, dtype, seed, device, scale)
    sp = torch.as_tensor(np.asarray(seq_pos, dtype=np.int32)).to(device)
    return {"q": q, "k_cache": kc, "v_cache": vc, "k_new": kn, "v_new": vn, "seq_pos": sp}
